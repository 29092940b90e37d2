"""GPU parity for the steps beside the scan: causal conv1d + SiLU with a
rolling history (prefill and slot-decode entry points) and gated RMSNorm,
through the C ABI against the CPU oracle.

Bar: max |gpu - ref| / (1 + |ref|) <= 1e-4 on every output against the fp32
oracle (and the fp64 oracle on the workloads).  The conv history holds raw
inputs, so it is compared bit for bit, as are unused slots, snapshots,
split runs, batch composition and repeated runs.
"""
import numpy as np
import pytest

import oracle
import ssm_inputs
from gpu_helpers import (TOL, assert_conv_parity, rel_err, run_conv_gpu, run_norm_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mamba2_selective_scan_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


WORKLOADS = ["tiny", "decode16", "mixed", "prefill4096", "decode256"]


# ------------------------------------------------------------------ conv
@pytest.mark.parametrize("name", WORKLOADS)
def test_conv_workload(ssm, orc, name):
    case = ssm_inputs.conv_workload(name)
    say(f"conv workload {case.name} via ssm_conv1d_silu_prefill")
    out, st = run_conv_gpu(case)
    o32, s32 = orc.conv_case(case, precision="f32")
    assert_conv_parity(case, out, st, o32, s32, label=f"{name} vs fp32 oracle")
    o64, _ = orc.conv_case(case, precision="f64")
    assert rel_err(out, o64) <= TOL


@pytest.mark.parametrize("name", ["decode16", "decode256"])
def test_conv_decode_entry(ssm, orc, name):
    case = ssm_inputs.conv_workload(name)
    say(f"conv workload {case.name} via ssm_conv1d_silu_decode")
    out, st = run_conv_gpu(case, "decode")
    o32, s32 = orc.conv_case(case)
    assert_conv_parity(case, out, st, o32, s32)
    op, sp = run_conv_gpu(case, "prefill")
    assert np.array_equal(out, op) and np.array_equal(st, sp), "decode and prefill entries differ"


CHUNK_EDGE_LENGTHS = [0, 1, 2, 3, 31, 32, 33, 64, 65, 100, 0, 7]


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("D", [1, 5, 96, 1024, 1028, 1030, 2336])
def test_conv_shapes(ssm, orc, K, D):
    n = len(CHUNK_EDGE_LENGTHS)
    fresh = [i % 2 for i in range(n)]
    slots = np.random.Generator(np.random.PCG64(K * 1000 + D)).permutation(n + 3)[:n]
    case = ssm_inputs.make_conv_case(D, K, CHUNK_EDGE_LENGTHS, fresh, K * 7 + D,
                                     slots=slots.astype(np.int32), n_slots=n + 3,
                                     poison_fresh=True, sentinel_unused=True,
                                     name=f"conv_K{K}_D{D}")
    say(f"conv shape K={K} D={D} lengths={CHUNK_EDGE_LENGTHS}")
    out, st = run_conv_gpu(case)
    o32, s32 = orc.conv_case(case)
    assert_conv_parity(case, out, st, o32, s32)


@pytest.mark.parametrize("K", [2, 4])
def test_conv_scalar_path(ssm, orc, K):
    """Arrays off 16-byte alignment take the one-channel-per-lane path."""
    case = ssm_inputs.make_conv_case(1024, K, [40, 1, 0, 70], [1, 0, 0, 1], 31 + K,
                                     name=f"conv_scalar_K{K}")
    say(f"conv scalar path K={K}")
    out, st = run_conv_gpu(case, offset_floats=1)
    o32, s32 = orc.conv_case(case)
    assert_conv_parity(case, out, st, o32, s32)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("offset", [0, 1])
def test_conv_snapshots(ssm, orc, K, offset):
    case = ssm_inputs.make_conv_case(260, K, [5, 0, 70, 1, 33], [1, 0, 0, 1, 0], 50 + K,
                                     name=f"conv_snaps_K{K}")
    say(f"conv snapshots K={K} offset={offset}")
    out, st, sn = run_conv_gpu(case, offset_floats=offset, snapshots=True)
    o32, s32, sn32 = orc.conv_case(case, snapshots=True)
    assert_conv_parity(case, out, st, o32, s32)
    assert np.array_equal(sn, sn32), "snapshots differ"


def test_conv_split_resume_bitwise(ssm, orc):
    """Tokens in one call equal the same tokens in two calls (bitwise)."""
    case = ssm_inputs.make_conv_case(6144, 4, [300], [0], 61, name="conv_split")
    say("conv split-resume")
    out, st = run_conv_gpu(case)
    for cut in (1, 2, 32, 45, 299):
        first = ssm_inputs.ConvCase(D=case.D, K=4, lengths=np.array([cut], np.int32),
                                    cu_seqlens=np.array([0, cut], np.int32), slot=case.slot,
                                    fresh=case.fresh, x=case.x[:cut], w=case.w, state=case.state)
        o1, s1 = run_conv_gpu(first)
        rest = ssm_inputs.ConvCase(D=case.D, K=4, lengths=np.array([300 - cut], np.int32),
                                   cu_seqlens=np.array([0, 300 - cut], np.int32), slot=case.slot,
                                   fresh=case.fresh, x=case.x[cut:], w=case.w, state=s1)
        o2, s2 = run_conv_gpu(rest)
        assert np.array_equal(np.concatenate([o1, o2]), out), cut
        assert np.array_equal(s2, st), cut


def test_conv_batch_independence_and_determinism(ssm, orc):
    case = ssm_inputs.conv_workload("mixed")
    say("conv batch independence")
    out, st = run_conv_gpu(case)
    out2, st2 = run_conv_gpu(case)
    assert np.array_equal(out, out2) and np.array_equal(st, st2, equal_nan=True)
    for s in range(case.n_seqs):
        a, b = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        one = ssm_inputs.ConvCase(D=case.D, K=case.K, lengths=case.lengths[s:s + 1],
                                  cu_seqlens=np.array([0, b - a], np.int32),
                                  slot=case.slot[s:s + 1], fresh=case.fresh[s:s + 1],
                                  x=case.x[a:b], w=case.w, state=case.state)
        o1, s1 = run_conv_gpu(one)
        assert np.array_equal(o1, out[a:b]), s
        assert np.array_equal(s1[case.slot[s]], st[case.slot[s]]), s


def test_conv_many_sequences(ssm, orc):
    """More than 256 sequences: the workgroup -> sequence search takes two
    rounds."""
    rng = np.random.Generator(np.random.PCG64(77))
    lengths = rng.choice([0, 1, 2, 5, 31, 32, 33, 70], size=700)
    fresh = rng.integers(0, 2, size=700)
    case = ssm_inputs.make_conv_case(64, 4, lengths, fresh, 78, name="conv_700seq")
    say(f"conv 700 sequences, {int(lengths.sum())} tokens")
    out, st = run_conv_gpu(case)
    o32, s32 = orc.conv_case(case)
    assert_conv_parity(case, out, st, o32, s32)


def test_conv_empty(ssm, orc):
    """No tokens at all: fresh slots zeroed, resuming slots unchanged."""
    case = ssm_inputs.make_conv_case(96, 4, [0, 0, 0], [1, 0, 1], 79, slots=[2, 0, 3], n_slots=4,
                                     poison_fresh=True, sentinel_unused=True, name="conv_empty")
    say("conv empty batch")
    out, st = run_conv_gpu(case)
    o32, s32 = orc.conv_case(case)
    assert out.shape == (0, 96)
    assert_conv_parity(case, out, st, o32, s32)


# ------------------------------------------------------------------ norm
@pytest.mark.parametrize("name", WORKLOADS)
def test_norm_workload(ssm, orc, name):
    case = ssm_inputs.norm_workload(name)
    say(f"norm workload {case.name}")
    out = run_norm_gpu(case)
    e32 = rel_err(out, orc.norm_case(case, precision="f32"))
    e64 = rel_err(out, orc.norm_case(case, precision="f64"))
    say(f"  max rel err vs fp32 {e32:.3e}, vs fp64 {e64:.3e}")
    assert e32 <= TOL and e64 <= TOL


@pytest.mark.parametrize("L", [1, 3, 4, 16, 63, 64, 96, 100, 256, 257, 1024, 1028, 1500, 4096])
@pytest.mark.parametrize("offset", [0, 1])
def test_norm_row_lengths(ssm, orc, L, offset):
    case = ssm_inputs.make_norm_case(37, 1, L, 900 + L, eps=1e-5, name=f"norm_L{L}")
    say(f"norm L={L} offset={offset}")
    out = run_norm_gpu(case, offset_floats=offset)
    e = rel_err(out, orc.norm_case(case))
    say(f"  max rel err {e:.3e}")
    assert np.all(np.isfinite(out)) and e <= TOL


def test_norm_eps_edges(ssm, orc):
    """eps = 0 on nonzero rows, and all-zero rows with eps > 0 (zeros out)."""
    case = ssm_inputs.make_norm_case(50, 8, 64, 950, eps=0.0, name="norm_eps0")
    out = run_norm_gpu(case)
    assert rel_err(out, orc.norm_case(case)) <= TOL
    case.y[:] = 0.0
    case.eps = 1e-5
    assert np.array_equal(run_norm_gpu(case), np.zeros_like(case.y))


def test_norm_scale_invariance_is_exact(ssm):
    """With eps = 0 the norm of 2y equals the norm of y bit for bit: the mean
    square takes an exact factor 4, its square root an exact factor 2."""
    import dataclasses
    case = ssm_inputs.make_norm_case(64, 8, 256, 977, eps=0.0, name="norm_scale")
    twice = dataclasses.replace(case, y=case.y * np.float32(2))
    assert np.array_equal(run_norm_gpu(case), run_norm_gpu(twice))


# ------------------------------------------------------------------ sweeps
@pytest.mark.parametrize("seed", range(12))
def test_conv_random_sweep(ssm, orc, seed):
    """Seeded random conv batches: channel count, taps, 1-40 sequences of
    0-300 tokens (empty ones included), fresh and resumed, scattered slots,
    the prefill or decode entry, vector or scalar path, with or without
    snapshots (prefill only)."""
    rng = np.random.Generator(np.random.PCG64(97500 + seed))
    K = int(rng.integers(1, 5))
    D = int(rng.choice([int(rng.integers(1, 3000)), 4 * int(rng.integers(1, 1600))]))
    mode = "decode" if seed % 3 == 2 else "prefill"
    n = int(rng.integers(1, 41))
    lengths = [1] * n if mode == "decode" else [int(v) for v in rng.integers(0, 301, size=n)]
    if mode == "prefill" and rng.random() < 0.5:
        lengths[int(rng.integers(0, n))] = 0
    snapshots = K > 1 and rng.random() < 0.3 and mode == "prefill"   # the decode entry takes none
    offset = int(rng.random() < 0.3)
    case = ssm_inputs.make_conv_case(D, K, lengths, [int(v) for v in rng.integers(0, 2, size=n)],
                                     97600 + seed, slots=rng.permutation(n + 3)[:n].astype(np.int32),
                                     n_slots=n + 3, poison_fresh=True, sentinel_unused=True,
                                     name=f"conv_sweep{seed}_{mode}_D{D}_K{K}_{n}seqs_{sum(lengths)}tok"
                                          f"{'_snapshots' if snapshots else ''}{'_scalar' if offset else ''}")
    say(case.name)
    res = run_conv_gpu(case, mode, offset_floats=offset, snapshots=snapshots)
    ref = orc.conv_case(case, snapshots=snapshots)
    assert_conv_parity(case, res[0], res[1], ref[0], ref[1])
    if snapshots:
        assert np.array_equal(res[2], ref[2]), "snapshots differ"


@pytest.mark.parametrize("seed", range(8))
def test_norm_random_sweep(ssm, orc, seed):
    """Seeded random gated RMSNorm shapes: rows, heads, row length (odd ones
    included), scaled inputs, vector or scalar path."""
    rng = np.random.Generator(np.random.PCG64(97800 + seed))
    T, H = int(rng.integers(1, 300)), int(rng.integers(1, 9))
    L = int(rng.choice([int(rng.integers(1, 2000)), 4 * int(rng.integers(1, 600))]))
    case = ssm_inputs.make_norm_case(T, H, L, 97900 + seed, eps=float(rng.choice([1e-5, 1e-6, 0.0])),
                                     y_std=float(rng.choice([1.0, 1e-3, 30.0])),
                                     name=f"norm_sweep{seed}_T{T}_H{H}_L{L}")
    offset = int(rng.random() < 0.3)
    say(f"{case.name} eps={case.eps} offset={offset}")
    out = run_norm_gpu(case, offset_floats=offset)
    e = rel_err(out, orc.norm_case(case))
    say(f"  max rel err {e:.3e}")
    assert np.all(np.isfinite(out)) and e <= TOL
