"""Pins for the CPU oracle: each takes an ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with something fixed independently of
it (hand-worked values, the unrolled closed form, textbook special cases and
invariants that hold exactly).  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies with planted mistakes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import ssm_inputs
from closed_form import brute_force, brute_force_general, softplus_rule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def rel_err(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - ref) / (1.0 + np.abs(ref))))


def _run(orc, case, precision="f32", threads=2):
    return orc.scan_case(case, precision=precision, threads=threads)


def _from_json(c):
    f32 = lambda v: np.asarray(v, dtype=np.float32)
    lengths = np.asarray(c["lengths"], dtype=np.int32)
    return ssm_inputs.ScanCase(
        H=c["H"], P=c["P"], N=c["N"], G=c["G"], lengths=lengths,
        cu_seqlens=ssm_inputs.lengths_to_cu(lengths),
        slot=np.asarray(c["slot"], dtype=np.int32),
        fresh=np.asarray(c["fresh"], dtype=np.uint8),
        x=f32(c["x"]).reshape(-1, c["H"], c["P"]), dt=f32(c["dt"]).reshape(-1, c["H"]),
        A=f32(c["A"]), B=f32(c["B"]).reshape(-1, c["G"], c["N"]),
        C=f32(c["C"]).reshape(-1, c["G"], c["N"]),
        state=f32(c["state_in"]).reshape(c["n_slots"], c["H"], c["P"], c["N"]),
        name=c["name"])


def golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    out = []
    for c in data["cases"]:
        out.append((_from_json(c), np.asarray(c["y"], dtype=np.float64),
                    np.asarray(c["state_out"], dtype=np.float64)))
    return out


# ---------------------------------------------------------------- pins
def pin_hand_worked(orc):
    for case, y_ref, st_ref in golden_cases():
        for prec in ("f32", "f64"):
            y, st = _run(orc, case, prec)
            assert rel_err(y, y_ref.reshape(y.shape)) < 1e-6, (case.name, prec)
            assert rel_err(st, st_ref.reshape(st.shape)) < 1e-6, (case.name, prec)


def small_random_case(seed, H=4, P=3, N=5, G=2, lengths=(5, 1, 0, 8, 3),
                      fresh=(1, 0, 0, 1, 0), n_slots=7, a_log_hi=math.log(16.0)):
    rng = np.random.Generator(np.random.PCG64(10_000 + seed))
    slots = rng.permutation(n_slots)[: len(lengths)]
    return ssm_inputs.make_case(H, P, N, G, list(lengths), list(fresh), seed, slots=slots,
                                n_slots=n_slots, a_log_hi=a_log_hi)


def pin_brute_force(orc):
    """Unrolled closed form on several small packed batches (several groups,
    fresh and resuming sequences, an empty one, permuted slots)."""
    shapes = [dict(), dict(H=6, P=2, N=7, G=3), dict(H=2, P=4, N=3, G=1),
              dict(H=4, P=2, N=4, G=4, lengths=(8,), fresh=(0,), n_slots=2)]
    for i, kw in enumerate(shapes):
        case = small_random_case(i, **kw)
        y_bf, st_bf = brute_force(case.H, case.P, case.N, case.G, case.cu_seqlens,
                                  case.slot, case.fresh, case.x, case.dt, case.A,
                                  case.B, case.C, case.state)
        y64, st64 = _run(orc, case, "f64")
        assert rel_err(y64, y_bf) < 1e-12 and rel_err(st64, st_bf) < 1e-12, i
        y32, st32 = _run(orc, case, "f32")
        assert rel_err(y32, y_bf) < 1e-5 and rel_err(st32, st_bf) < 1e-5, i


def pin_brute_force_tiny_workload(orc):
    """The tiny workload truncated to 8 tokens, against the closed form."""
    full = ssm_inputs.workload("tiny")
    T = 8
    lengths = np.array([T], dtype=np.int32)
    case = ssm_inputs.ScanCase(H=full.H, P=full.P, N=full.N, G=full.G, lengths=lengths,
                               cu_seqlens=ssm_inputs.lengths_to_cu(lengths),
                               slot=full.slot, fresh=full.fresh, x=full.x[:T],
                               dt=full.dt[:T], A=full.A, B=full.B[:T], C=full.C[:T],
                               state=full.state)
    y_bf, st_bf = brute_force(case.H, case.P, case.N, case.G, case.cu_seqlens, case.slot,
                              case.fresh, case.x, case.dt, case.A, case.B, case.C,
                              case.state)
    y64, st64 = _run(orc, case, "f64")
    assert rel_err(y64, y_bf) < 1e-12 and rel_err(st64, st_bf) < 1e-12
    y32, st32 = _run(orc, case, "f32")
    assert rel_err(y32, y_bf) < 1e-5 and rel_err(st32, st_bf) < 1e-5


def pin_single_token_dot(orc):
    """T=1 from the zero state: h = dt*x (outer) B and y = dt*x*(B.C)."""
    case = ssm_inputs.make_case(8, 6, 33, 4, [1, 1, 1], [1, 1, 1], seed=7)
    y32, st32 = _run(orc, case, "f32")
    y64, st64 = _run(orc, case, "f64")
    hpg = case.H // case.G
    for s in range(3):
        for hd in range(case.H):
            g = hd // hpg
            b = case.B[s, g].astype(np.float64)
            c = case.C[s, g].astype(np.float64)
            u = float(case.dt[s, hd]) * case.x[s, hd].astype(np.float64)
            y_ref = u * math.fsum(b * c)
            h_ref = np.outer(u, b)
            for y, st, tol in ((y64, st64, 1e-12), (y32, st32, 2e-6)):
                assert rel_err(y[s, hd], y_ref) < tol, (s, hd)
                assert rel_err(st[case.slot[s], hd], h_ref) < tol, (s, hd)


def pin_prefix_sum(orc):
    """A=0 (no decay), dt=1, one-hot B=e_i and C=e_j, small-integer x: y is
    the running sum of x when i == j and zero otherwise, exactly in fp32."""
    H, P, N, G, T = 4, 5, 6, 2, 40
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.integers(-8, 9, size=(T, H, P)).astype(np.float32)
    B = np.zeros((T, G, N), np.float32)
    C = np.zeros((T, G, N), np.float32)
    # group 0: B = e_1, C = e_1 (matching); group 1: B = e_2, C = e_4 (not)
    B[:, 0, 1] = 1
    C[:, 0, 1] = 1
    B[:, 1, 2] = 1
    C[:, 1, 4] = 1
    case = ssm_inputs.ScanCase(H=H, P=P, N=N, G=G, lengths=np.array([T], np.int32),
                               cu_seqlens=np.array([0, T], np.int32),
                               slot=np.array([0], np.int32), fresh=np.array([1], np.uint8),
                               x=x, dt=np.ones((T, H), np.float32),
                               A=np.zeros(H, np.float32), B=B, C=C,
                               state=np.zeros((1, H, P, N), np.float32))
    y, st = _run(orc, case, "f32")
    run = np.cumsum(x.astype(np.int64), axis=0)
    assert np.array_equal(y[:, :2], run[:, :2].astype(np.float32))       # heads of group 0
    assert np.array_equal(y[:, 2:], np.zeros_like(y[:, 2:]))             # heads of group 1
    assert np.array_equal(st[0, :2, :, 1], run[-1, :2].astype(np.float32))
    assert np.array_equal(st[0, 2:, :, 2], run[-1, 2:].astype(np.float32))
    st_other = st.copy()
    st_other[0, :2, :, 1] = 0
    st_other[0, 2:, :, 2] = 0
    assert not np.any(st_other)


def pin_decay_only(orc):
    """x = 0: the state only decays.  With constant dt the final state is
    exp(T*dt*A) * h0; per token y_t = exp(t*dt*A) * (h0 . C_t)."""
    H, P, N, G, T = 3, 2, 4, 1, 30
    case = ssm_inputs.make_case(H, P, N, G, [T], [0], seed=11)
    case.x[:] = 0
    case.dt[:] = np.float32(0.05)
    y64, st64 = _run(orc, case, "f64")
    y32, st32 = _run(orc, case, "f32")
    for hd in range(H):
        lam = float(np.float32(0.05)) * float(case.A[hd])
        h0 = case.state[0, hd].astype(np.float64)
        ref_st = math.exp(T * lam) * h0
        ref_y = np.array([math.exp((t + 1) * lam) * (h0 @ case.C[t, 0].astype(np.float64))
                          for t in range(T)])
        assert rel_err(st64[0, hd], ref_st) < 1e-12
        assert rel_err(y64[:, hd], ref_y) < 1e-12
        assert rel_err(st32[0, hd], ref_st) < 1e-5
        assert rel_err(y32[:, hd], ref_y) < 1e-5


def pin_split_resume(orc):
    """T tokens in one call equal T1 tokens, then T-T1 resumed from the slot,
    bit for bit (fp32 and fp64)."""
    T = 37
    case = ssm_inputs.make_case(4, 3, 9, 2, [T], [1], seed=13, n_slots=1)
    for prec in ("f32", "f64"):
        y_all, st_all = _run(orc, case, prec)
        for T1 in (0, 1, 16, 36, 37):
            c1 = ssm_inputs.ScanCase(H=4, P=3, N=9, G=2, lengths=np.array([T1], np.int32),
                                     cu_seqlens=np.array([0, T1], np.int32), slot=case.slot,
                                     fresh=case.fresh, x=case.x[:T1], dt=case.dt[:T1],
                                     A=case.A, B=case.B[:T1], C=case.C[:T1], state=case.state)
            y1, st1 = _run(orc, c1, prec)
            c2 = ssm_inputs.ScanCase(H=4, P=3, N=9, G=2, lengths=np.array([T - T1], np.int32),
                                     cu_seqlens=np.array([0, T - T1], np.int32),
                                     slot=case.slot, fresh=np.array([0], np.uint8),
                                     x=case.x[T1:], dt=case.dt[T1:], A=case.A,
                                     B=case.B[T1:], C=case.C[T1:],
                                     state=st1)
            y2, st2 = _run(orc, c2, prec)
            assert np.array_equal(np.concatenate([y1, y2]), y_all), (prec, T1)
            assert np.array_equal(st2, st_all), (prec, T1)


def pin_batch_independence(orc):
    """A sequence alone equals the same sequence inside a packed batch, bit for
    bit; decode (every length 1) equals one-token prefills one at a time."""
    case = small_random_case(3, lengths=(4, 1, 6, 1), fresh=(0, 1, 0, 0), n_slots=5)
    y, st = _run(orc, case, "f32")
    for s in range(case.n_seqs):
        t0, t1 = case.cu_seqlens[s], case.cu_seqlens[s + 1]
        alone = ssm_inputs.ScanCase(H=case.H, P=case.P, N=case.N, G=case.G,
                                    lengths=np.array([t1 - t0], np.int32),
                                    cu_seqlens=np.array([0, t1 - t0], np.int32),
                                    slot=np.array([case.slot[s]], np.int32),
                                    fresh=np.array([case.fresh[s]], np.uint8),
                                    x=case.x[t0:t1], dt=case.dt[t0:t1], A=case.A,
                                    B=case.B[t0:t1], C=case.C[t0:t1], state=case.state)
        ya, sta = _run(orc, alone, "f32")
        assert np.array_equal(ya, y[t0:t1]), s
        assert np.array_equal(sta[case.slot[s]], st[case.slot[s]]), s


def pin_linearity(orc):
    """Scaling x and h0 by 2 scales y and the final state by 2 exactly;
    superposition in (x, h0) at fixed dt, A, B, C holds to rounding."""
    case = small_random_case(4, lengths=(9, 4), fresh=(0, 0), n_slots=2)
    y, st = _run(orc, case, "f32")
    c2 = small_random_case(4, lengths=(9, 4), fresh=(0, 0), n_slots=2)
    c2.x = case.x * np.float32(2)
    c2.state = case.state * np.float32(2)
    y2, st2 = _run(orc, c2, "f32")
    assert np.array_equal(y2, 2 * y) and np.array_equal(st2, 2 * st)
    cb = small_random_case(5, lengths=(9, 4), fresh=(0, 0), n_slots=2)
    cb.dt, cb.A, cb.B, cb.C = case.dt, case.A, case.B, case.C
    cb.slot = case.slot
    yb, stb = _run(orc, cb, "f64")
    ya, sta = _run(orc, case, "f64")
    csum = small_random_case(4, lengths=(9, 4), fresh=(0, 0), n_slots=2)
    csum.x = (case.x.astype(np.float64) + cb.x).astype(np.float32)
    csum.state = (case.state.astype(np.float64) + cb.state).astype(np.float32)
    ys, sts = _run(orc, csum, "f64")
    assert rel_err(ys, ya + yb) < 1e-6 and rel_err(sts, sta + stb) < 1e-6


def pin_group_equivalence(orc):
    """G = H with B and C repeated per head gives the same result as G = 1."""
    base = ssm_inputs.make_case(4, 3, 6, 1, [7, 3], [1, 0], seed=17)
    y1, st1 = _run(orc, base, "f32")
    rep = ssm_inputs.make_case(4, 3, 6, 4, [7, 3], [1, 0], seed=17)
    rep.A, rep.dt, rep.x, rep.state = base.A, base.dt, base.x, base.state
    rep.B = np.repeat(base.B, 4, axis=1)
    rep.C = np.repeat(base.C, 4, axis=1)
    y4, st4 = _run(orc, rep, "f32")
    assert np.array_equal(y1, y4) and np.array_equal(st1, st4)


def pin_slot_hygiene(orc):
    """Fresh slots poisoned with NaN give finite results; slots no sequence
    names come back bit for bit; a zero-length resume leaves its slot alone and
    a zero-length fresh sequence zeroes its slot."""
    case = ssm_inputs.make_case(2, 3, 4, 1, [3, 0, 2, 0], [1, 0, 0, 1], seed=19,
                                slots=[4, 0, 2, 1], n_slots=6, poison_fresh=True,
                                sentinel_unused=True)
    y, st = _run(orc, case, "f32")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(st[[4, 0, 2, 1]]))
    for k in (3, 5):                                           # unused slots
        assert np.array_equal(st[k], case.state[k])
    assert np.array_equal(st[0], case.state[0])                # empty resume
    assert not np.any(st[1])                                   # empty fresh


def pin_thread_count(orc):
    """The (sequence, head) split over host threads changes no bit."""
    case = ssm_inputs.workload("mixed")
    y1, st1 = orc.scan_case(case, threads=1)
    y8, st8 = orc.scan_case(case, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(st1, st8, equal_nan=True)


# ------------------------------------------------------------ option pins
def pin_softplus_single_token(orc):
    """T = 1 from zero with dt_eff = softplus(dt + bias): y = dt_eff*x*(B.C),
    h = dt_eff * x (outer) B; biases put dt + bias on both sides of the 20
    cut-off (and right next to it); bias without softplus just adds."""
    H, P, N, G = 6, 3, 5, 2
    case = ssm_inputs.make_case(H, P, N, G, [1, 1], [1, 1], seed=31)
    bias = np.array([-3.0, 0.5, 19.93, 20.05, 25.0, -0.2], np.float32)
    for softplus in (True, False):
        y64, st64 = orc.scan_case(case, precision="f64", dt_bias=bias, dt_softplus=softplus)
        y32, st32 = orc.scan_case(case, precision="f32", dt_bias=bias, dt_softplus=softplus)
        for s in range(2):
            for hd in range(H):
                v = float(case.dt[s, hd]) + float(bias[hd])
                d = softplus_rule(v) if softplus else v
                g = hd // (H // G)
                b = case.B[s, g].astype(np.float64)
                u = d * case.x[s, hd].astype(np.float64)
                y_ref = u * math.fsum(b * case.C[s, g].astype(np.float64))
                for y, st, tol in ((y64, st64, 1e-12), (y32, st32, 2e-6)):
                    assert rel_err(y[s, hd], y_ref) < tol, (softplus, s, hd)
                    assert rel_err(st[case.slot[s], hd], np.outer(u, b)) < tol, (softplus, s, hd)


def pin_per_state_A_closed_form(orc):
    """A per (head, state index): unrolled closed form with a decay per n, on
    a packed batch with softplus and bias on as well."""
    case = small_random_case(41, lengths=(5, 0, 7, 2), fresh=(1, 0, 0, 1), n_slots=5)
    rng = np.random.Generator(np.random.PCG64(42))
    A_hn = (-np.exp(rng.uniform(0.0, math.log(16.0), size=(case.H, case.N)))).astype(np.float32)
    bias = rng.uniform(-2.0, 2.0, size=case.H).astype(np.float32)
    dt_eff = np.array([[softplus_rule(float(case.dt[t, h]) + float(bias[h]))
                        for h in range(case.H)] for t in range(case.n_tokens)])
    y_bf, st_bf = brute_force_general(case.H, case.P, case.N, case.G, case.cu_seqlens, case.slot,
                                      case.fresh, case.x, dt_eff, A_hn.astype(np.float64),
                                      case.B, case.C, case.state)
    kw = dict(dt_bias=bias, dt_softplus=True, A_per_state=True)
    c2 = small_random_case(41, lengths=(5, 0, 7, 2), fresh=(1, 0, 0, 1), n_slots=5)
    c2.A = A_hn
    y64, st64 = orc.scan_case(c2, precision="f64", **kw)
    y32, st32 = orc.scan_case(c2, precision="f32", **kw)
    assert rel_err(y64, y_bf) < 1e-12 and rel_err(st64, st_bf) < 1e-12
    assert rel_err(y32, y_bf) < 1e-5 and rel_err(st32, st_bf) < 1e-5


def pin_per_state_A_constant_rows(orc):
    """A[h][n] equal for every n gives the scalar-A scan, bit for bit."""
    case = small_random_case(43)
    y1, st1 = orc.scan_case(case, precision="f32")
    c2 = small_random_case(43)
    c2.A = np.repeat(case.A[:, None], case.N, axis=1)
    y2, st2 = orc.scan_case(c2, precision="f32", A_per_state=True)
    assert np.array_equal(y1, y2) and np.array_equal(st1, st2)


def pin_snapshots(orc):
    """Snapshots: the state after every token.  The last one of each sequence
    is its final state, and the snapshot after token t equals the final state
    of the same sequence run only through t (bit for bit)."""
    case = small_random_case(47, lengths=(4, 1, 6), fresh=(0, 1, 0), n_slots=4)
    y, st, snaps = orc.scan_case(case, precision="f32", snapshots=True)
    y0, st0 = orc.scan_case(case, precision="f32")
    assert np.array_equal(y, y0) and np.array_equal(st, st0)
    for s in range(case.n_seqs):
        t0, t1 = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        assert np.array_equal(snaps[t1 - 1], st[case.slot[s]]), s
        for t in range(t0, t1):
            part = ssm_inputs.ScanCase(
                H=case.H, P=case.P, N=case.N, G=case.G, lengths=np.array([t + 1 - t0], np.int32),
                cu_seqlens=np.array([0, t + 1 - t0], np.int32), slot=case.slot[s:s + 1],
                fresh=case.fresh[s:s + 1], x=case.x[t0:t + 1], dt=case.dt[t0:t + 1], A=case.A,
                B=case.B[t0:t + 1], C=case.C[t0:t + 1], state=case.state)
            _, stp = orc.scan_case(part, precision="f32")
            assert np.array_equal(snaps[t], stp[case.slot[s]]), (s, t)


ALL_PINS = [pin_hand_worked, pin_brute_force, pin_brute_force_tiny_workload,
            pin_single_token_dot, pin_prefix_sum, pin_decay_only, pin_split_resume,
            pin_batch_independence, pin_linearity, pin_group_equivalence,
            pin_slot_hygiene, pin_thread_count, pin_softplus_single_token,
            pin_per_state_A_closed_form, pin_per_state_A_constant_rows, pin_snapshots]

# the neighbouring steps (conv1d + SiLU, gated RMSNorm)
from neighbour_pins import CONV_PINS, NORM_PINS  # noqa: E402

ALL_PINS = ALL_PINS + CONV_PINS + NORM_PINS

# the gated delta-rule recurrence
from gdn_pins import GDN_PINS  # noqa: E402

ALL_PINS = ALL_PINS + GDN_PINS
