"""Pins for the oracle's neighbouring steps: causal conv1d + SiLU with a rolling
history, and gated RMSNorm.  Each takes an ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with something fixed independently of
its C loops: torch's own depthwise ``conv1d``, ``rms_norm`` and ``silu`` on the
CPU in float64 (library routines), exact closed forms built on
sigmoid(ln a) = a / (1 + a), and invariants that hold exactly in floating
point (power-of-two scaling, splitting a run, batch independence)."""
from __future__ import annotations

import math

import numpy as np

import ssm_inputs


def rel_err(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref) / (1.0 + np.abs(ref))))


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------ conv
def small_conv_case(seed, D=5, K=4, lengths=(5, 1, 0, 8, 3, 2), fresh=(1, 0, 1, 0, 0, 1)):
    n = len(lengths)
    slots = np.random.Generator(np.random.PCG64(seed + 7)).permutation(n + 2)[:n]
    return ssm_inputs.make_conv_case(D, K, list(lengths), list(fresh), seed,
                                     slots=slots.astype(np.int32), n_slots=n + 2,
                                     sentinel_unused=True, name=f"conv_small_K{K}")


def conv_by_torch(case):
    """Expected output and final history in float64 from torch's depthwise
    cross-correlation (F.conv1d with groups = D) over each sequence's history
    followed by its inputs, then F.silu.  The final history is the last K-1
    entries of that extended sequence."""
    torch = _torch()
    F = torch.nn.functional
    K, D = case.K, case.D
    out = np.zeros((case.n_tokens, D))
    st = case.state.astype(np.float64).copy()
    w = torch.from_numpy(case.w.astype(np.float64)).reshape(D, 1, K)
    for s in range(case.n_seqs):
        a, b = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        hist0 = (np.zeros((D, K - 1)) if case.fresh[s]
                 else case.state[case.slot[s]].astype(np.float64))
        ext = np.concatenate([hist0, case.x[a:b].astype(np.float64).T], axis=1)  # [D, K-1+len]
        if b > a:
            pre = F.conv1d(torch.from_numpy(ext)[None], w, groups=D)[0]          # [D, len]
            out[a:b] = F.silu(pre).numpy().T
        st[case.slot[s]] = ext[:, b - a:b - a + K - 1]
    return out, st


def pin_conv_torch_conv1d(orc):
    for K in (1, 2, 3, 4):
        case = small_conv_case(100 + K, K=K)
        out_ref, st_ref = conv_by_torch(case)
        used = np.unique(case.slot)
        out64, st64 = orc.conv_case(case, precision="f64", threads=2)
        assert rel_err(out64, out_ref) <= 1e-12, f"K={K}: f64 output"
        assert rel_err(st64[used], st_ref[used]) == 0.0, f"K={K}: f64 history"
        out32, st32 = orc.conv_case(case, precision="f32", threads=2)
        assert rel_err(out32, out_ref) <= 1e-5, f"K={K}: f32 output"
        assert rel_err(st32[used], st_ref[used]) == 0.0, f"K={K}: f32 history"


def pin_conv_workload_torch(orc):
    """The mixed-batch workload (resume, fresh, poisoned fresh slots, unused
    slots) against torch."""
    case = ssm_inputs.conv_workload("mixed")
    # torch needs finite history for fresh sequences only in the sense that it
    # never reads it: conv_by_torch uses zeros there, as the oracle must.
    out_ref, st_ref = conv_by_torch(case)
    out32, st32 = orc.conv_case(case, precision="f32")
    used = np.unique(case.slot)
    assert np.all(np.isfinite(out32))
    assert rel_err(out32, out_ref) <= 1e-5
    assert rel_err(st32[used], st_ref[used]) == 0.0


def pin_conv_impulse_closed_form(orc):
    """Fresh history, a unit impulse at token t0 of channel c: the
    pre-activation at t0 + j is w[c][K-1-j] for j < K and zero elsewhere.  With
    the taps set to ln a the output is ln a * a / (1 + a), since
    sigmoid(ln a) = a / (1 + a); silu(0) = 0 exactly."""
    K, D, T, t0 = 4, 3, 9, 2
    taps = {0: 2.0, 1: 3.0, 2: 1.0 / 3.0, 3: 5.0}      # tap i holds ln(taps[i])
    w = np.zeros((D, K), np.float32)
    for i, a in taps.items():
        w[:, i] = np.float32(math.log(a))
    for c in range(D):
        x = np.zeros((T, D), np.float32)
        x[t0, c] = 1.0
        cu = np.array([0, T], np.int32)
        st = np.full((1, D, K - 1), np.nan, np.float32)
        for precision, tol in (("f32", 5e-7), ("f64", 1e-15)):
            out, _ = orc.conv1d_silu(K, cu, [0], [1], x, w, st, precision=precision, threads=1)
            for t in range(T):
                for cc in range(D):
                    j = t - t0
                    if cc == c and 0 <= j < K:
                        a = float(np.float32(math.log(taps[K - 1 - j])))   # the fp32 tap
                        ea = math.exp(a)
                        expect = a * ea / (1.0 + ea)
                    else:
                        expect = 0.0
                    got = float(out[t, cc])
                    assert abs(got - expect) <= tol * (1.0 + abs(expect)), \
                        f"{precision} t={t} c={cc}: {got} vs {expect}"


def pin_conv_split_resume(orc):
    """A run of tokens in one call equals the same tokens in two calls with the
    history carried through the slot (bitwise: nothing crosses the split but
    the stored raw inputs)."""
    for K in (2, 4):
        case = ssm_inputs.make_conv_case(6, K, [11], [0], 300 + K)
        out_all, st_all = orc.conv_case(case, threads=1)
        for cut in (1, 2, 5, 10):
            cu1 = np.array([0, cut], np.int32)
            o1, s1 = orc.conv1d_silu(K, cu1, case.slot, case.fresh, case.x[:cut], case.w,
                                     case.state, threads=1)
            cu2 = np.array([0, 11 - cut], np.int32)
            o2, s2 = orc.conv1d_silu(K, cu2, case.slot, [0], case.x[cut:], case.w, s1,
                                     threads=1)
            assert np.array_equal(np.concatenate([o1, o2]), out_all), f"K={K} cut={cut}"
            assert np.array_equal(s2, st_all), f"K={K} cut={cut} history"


def pin_conv_batch_independence(orc):
    """Each sequence alone gives bitwise what it gives inside the batch."""
    case = small_conv_case(400)
    out, st = orc.conv_case(case, threads=3)
    for s in range(case.n_seqs):
        a, b = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        o1, s1 = orc.conv1d_silu(case.K, np.array([0, b - a], np.int32), case.slot[s:s + 1],
                                 case.fresh[s:s + 1], case.x[a:b], case.w, case.state,
                                 threads=1)
        assert np.array_equal(o1, out[a:b])
        assert np.array_equal(s1[case.slot[s]], st[case.slot[s]])


def pin_conv_slot_hygiene(orc):
    """Unused slots come back bitwise; a zero-length fresh sequence zeroes its
    slot, a zero-length resuming one leaves it bitwise; a fresh slot full of
    NaN is never read."""
    lengths, fresh = [3, 0, 0, 4], [1, 1, 0, 0]
    case = ssm_inputs.make_conv_case(4, 4, lengths, fresh, 500, slots=[5, 1, 3, 0],
                                     n_slots=6, poison_fresh=True, sentinel_unused=True)
    out, st = orc.conv_case(case, threads=2)
    assert np.all(np.isfinite(out))
    for k in (2, 4):                                    # unused
        assert np.array_equal(st[k], case.state[k])
    assert np.array_equal(st[1], np.zeros_like(st[1]))  # zero-length fresh
    assert np.array_equal(st[3], case.state[3])         # zero-length resume
    assert np.all(np.isfinite(st[5]))


def pin_conv_snapshots(orc):
    """Snapshot t equals the final history of a run that stops after token t;
    the last snapshot of a sequence equals its final history."""
    case = small_conv_case(600, D=4, K=4, lengths=(5, 2, 7), fresh=(1, 0, 0))
    out, st, snaps = orc.conv_case(case, snapshots=True, threads=2)
    for s in range(case.n_seqs):
        a, b = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        for t in range(a, b):
            cu = np.array([0, t + 1 - a], np.int32)
            _, s1 = orc.conv1d_silu(case.K, cu, case.slot[s:s + 1], case.fresh[s:s + 1],
                                    case.x[a:t + 1], case.w, case.state, threads=1)
            assert np.array_equal(snaps[t], s1[case.slot[s]]), f"seq {s} token {t}"
        assert np.array_equal(snaps[b - 1], st[case.slot[s]])


def pin_conv_thread_count(orc):
    case = ssm_inputs.conv_workload("mixed")
    o1, s1 = orc.conv_case(case, threads=1)
    o3, s3 = orc.conv_case(case, threads=3)
    assert np.array_equal(o1, o3) and np.array_equal(s1, s3, equal_nan=True)


# ------------------------------------------------------------------ norm
def norm_by_torch(y, z, w, eps):
    torch = _torch()
    F = torch.nn.functional
    y64 = torch.from_numpy(np.asarray(y, np.float64))
    z64 = torch.from_numpy(np.asarray(z, np.float64))
    w64 = torch.from_numpy(np.asarray(w, np.float64))
    return (F.rms_norm(y64, (w64.shape[0],), w64, eps) * F.silu(z64)).numpy()


def pin_norm_torch(orc):
    for name in ("tiny", "mixed"):
        case = ssm_inputs.norm_workload(name)
        ref = norm_by_torch(case.y, case.z, case.w, case.eps)
        assert rel_err(orc.norm_case(case, precision="f64"), ref) <= 1e-12, name
        assert rel_err(orc.norm_case(case, precision="f32"), ref) <= 1e-5, name
    for L in (1, 3, 100):
        case = ssm_inputs.make_norm_case(5, 3, L, 700 + L, eps=0.25)
        ref = norm_by_torch(case.y, case.z, case.w, case.eps)
        assert rel_err(orc.norm_case(case, precision="f32"), ref) <= 1e-5, f"L={L}"


def pin_norm_single_nonzero(orc):
    """eps = 0, a row with one nonzero value a at index j (L = 16): the root
    mean square is |a| / 4, so out[j] = sign(a) * 4 * w[j] * silu(z[j]) and
    every other entry is 0.  With z[j] = ln b, silu(z[j]) = ln b * b / (1 + b)."""
    L = 16
    w = (np.arange(L, dtype=np.float32) + 1.0) / 8.0          # exact in fp32
    for j, a, b in ((0, 3.0, 3.0), (5, -0.5, 2.0), (15, 7.0, 1.0 / 3.0), (9, 1e-3, 5.0)):
        y = np.zeros((1, L), np.float32)
        y[0, j] = a
        z = np.zeros((1, L), np.float32)
        z[0, j] = np.float32(math.log(b))
        zj = float(z[0, j])
        expect = math.copysign(1.0, a) * 4.0 * float(w[j]) * zj * math.exp(zj) / (1.0 + math.exp(zj))
        for precision, tol in (("f32", 1e-6), ("f64", 1e-14)):
            out = orc.gated_rmsnorm(y, z, w, 0.0, precision=precision, threads=1)
            others = np.delete(out[0], j)
            assert np.all(others == 0.0), precision
            assert abs(out[0, j] - expect) <= tol * abs(expect), (precision, j, out[0, j], expect)


def pin_norm_scale_invariance(orc):
    """eps = 0: scaling a row by a power of two leaves every output bitwise
    unchanged (each rounding step scales exactly)."""
    case = ssm_inputs.make_norm_case(7, 5, 24, 800, eps=0.0)
    base = orc.gated_rmsnorm(case.y, case.z, case.w, 0.0, threads=1)
    for k in (-6, -1, 1, 5):
        scaled = (case.y * np.float32(2.0 ** k)).astype(np.float32)
        assert np.array_equal(orc.gated_rmsnorm(scaled, case.z, case.w, 0.0, threads=1), base), k
    # a sign flip of y flips the output
    assert np.array_equal(orc.gated_rmsnorm(-case.y, case.z, case.w, 0.0, threads=1), -base)


def pin_norm_eps(orc):
    """A constant row y = c with eps = 3 c^2: the root mean square is 2 |c|,
    so out = sign(c) * w * silu(z) / 2.  A zero row with eps > 0 gives zeros."""
    L = 8
    w = np.linspace(0.5, 2.0, L).astype(np.float32)
    b = np.array([3.0, 2.0, 0.5, 4.0, 1.0, 1.0 / 3.0, 6.0, 0.25])
    z = np.log(b).astype(np.float32)[None]
    zf = z[0].astype(np.float64)
    silu = zf * np.exp(zf) / (1.0 + np.exp(zf))
    for c in (0.5, -2.0):
        y = np.full((1, L), c, np.float32)
        out = orc.gated_rmsnorm(y, z, w, 3.0 * c * c, threads=1)
        expect = math.copysign(0.5, c) * w.astype(np.float64) * silu
        assert rel_err(out[0], expect) <= 1e-6, c
    zero = orc.gated_rmsnorm(np.zeros((2, L), np.float32), np.ones((2, L), np.float32), w,
                             1e-5, threads=1)
    assert np.array_equal(zero, np.zeros_like(zero))


def pin_norm_thread_count(orc):
    case = ssm_inputs.norm_workload("mixed")
    assert np.array_equal(orc.norm_case(case, threads=1), orc.norm_case(case, threads=4))


CONV_PINS = [pin_conv_torch_conv1d, pin_conv_workload_torch, pin_conv_impulse_closed_form,
             pin_conv_split_resume, pin_conv_batch_independence, pin_conv_slot_hygiene,
             pin_conv_snapshots, pin_conv_thread_count]
NORM_PINS = [pin_norm_torch, pin_norm_single_nonzero, pin_norm_scale_invariance, pin_norm_eps,
             pin_norm_thread_count]
