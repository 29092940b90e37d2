"""GPU parity for the gated delta rule over seeded random batches: the
per-token prefill, the chunked prefill (or its per-token fallback where the
shape does not take chunks) and decode, against the fp32 oracle.

Each draw picks the head counts (value heads a multiple of key heads), key and
value widths, 1-4 sequences of 0-500 tokens with empty ones, fresh and
resumed starts, scattered slots (fresh ones NaN-poisoned, unused ones
sentinel-filled), and half the time q and k rows of length U[0.25, 1.4] with
drawn, 0, 1/2 or 1 write strengths.  Bar as everywhere: max |gpu - ref| /
(1 + |ref|) <= 1e-4 on y and on the final state of every used slot.
"""
import numpy as np
import pytest

import oracle
import ssm_inputs
from gpu_helpers import TOL, run_gdn_gpu, say
from test_gpu_gdn import assert_gdn_parity

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


def _gdn_sweep_case(seed):
    rng = np.random.Generator(np.random.PCG64(95000 + seed))
    Hk = int(rng.integers(1, 5))
    Hv = Hk * int(rng.integers(1, 4))
    if seed % 2 == 0:                            # shapes the chunked form takes
        Dk = int(rng.choice([64, 128]))
        Dv = 16 * int(rng.integers(1, 9))
    else:
        Dk = int(rng.integers(1, 129))
        Dv = int(rng.integers(1, 129))
    n = int(rng.integers(1, 5))
    lengths = [int(v) for v in rng.integers(0, 501, size=n)]
    if rng.random() < 0.3:
        lengths[int(rng.integers(0, n))] = 0
    fresh = [int(v) for v in rng.integers(0, 2, size=n)]
    slots = [int(v) for v in rng.permutation(n + 2)[:n]]
    normed = rng.random() < 0.5
    beta = [None, 0.0, 0.5, 1.0][int(rng.integers(0, 4))] if normed else None
    case = ssm_inputs.make_gdn_case(Hv, Hk, Dk, Dv, lengths, fresh, 96000 + seed, slots=slots,
                                    n_slots=n + 2, poison_fresh=True, sentinel_unused=True,
                                    qk_norm=(0.25, 1.4) if normed else None, beta=beta,
                                    name=f"gdn_sweep{seed}_Hv{Hv}_Hk{Hk}_Dk{Dk}_Dv{Dv}_{lengths}"
                                         f"{'_normed' if normed else ''}_beta{beta}")
    return case


@pytest.mark.parametrize("seed", range(16))
def test_gdn_random_shape_sweep(ssm, orc, seed):
    case = _gdn_sweep_case(seed)
    ws = ssm.gdn_workspace_size(case.Hv, case.Hk, case.Dk, case.Dv, case.n_seqs,
                                int(case.lengths.max()))
    say(f"{case.name}: chunked workspace {ws} bytes")
    y32, s32 = orc.gdn_case(case)
    y, st = run_gdn_gpu(case, "prefill")
    assert_gdn_parity(case, y, st, y32, s32, label=f"{case.name} per token")
    y, st = run_gdn_gpu(case, "prefill_ws")
    assert_gdn_parity(case, y, st, y32, s32, label=f"{case.name} chunked")
    # decode at the same shape: 1..40 one-token sequences, scattered slots
    rng = np.random.Generator(np.random.PCG64(97000 + seed))
    n = int(rng.integers(1, 41))
    dec = ssm_inputs.make_gdn_case(case.Hv, case.Hk, case.Dk, case.Dv, [1] * n,
                                   [int(v) for v in rng.integers(0, 2, size=n)], 98000 + seed,
                                   slots=[int(v) for v in rng.permutation(n + 3)[:n]],
                                   n_slots=n + 3, poison_fresh=True, sentinel_unused=True,
                                   name=f"gdn_sweep{seed}_decode{n}")
    y32, s32 = orc.gdn_case(dec)
    y, st = run_gdn_gpu(dec, "decode")
    assert_gdn_parity(dec, y, st, y32, s32)


@pytest.mark.parametrize("seed", range(12))
def test_gdn_random_option_sweep(ssm, orc, seed):
    """Seeded random delta-rule batches with snapshots or arrays off 16-byte
    alignment (the scalar path), through the per-token prefill or decode:
    y and state against the fp32 oracle, snapshots too, and each sequence's
    last snapshot bit for bit the state written to its slot."""
    rng = np.random.Generator(np.random.PCG64(99000 + seed))
    mode = "decode" if seed % 3 == 2 else "prefill"
    Hk = int(rng.integers(1, 4))
    Hv = Hk * int(rng.integers(1, 3))
    Dk, Dv = int(rng.integers(1, 129)), int(rng.integers(1, 97))
    n = int(rng.integers(1, 25)) if mode == "decode" else int(rng.integers(1, 4))
    lengths = [1] * n if mode == "decode" else [int(v) for v in rng.integers(0, 120, size=n)]
    snapshots = bool(seed % 2 == 0)
    offset = int(rng.random() < 0.5)
    case = ssm_inputs.make_gdn_case(Hv, Hk, Dk, Dv, lengths, [int(v) for v in rng.integers(0, 2, size=n)],
                                    99500 + seed, slots=[int(v) for v in rng.permutation(n + 2)[:n]],
                                    n_slots=n + 2, poison_fresh=True, sentinel_unused=True,
                                    name=f"gdn_option_sweep{seed}_{mode}_Hv{Hv}_Hk{Hk}_Dk{Dk}_Dv{Dv}_"
                                         f"{n}seqs{'_snapshots' if snapshots else ''}"
                                         f"{'_scalar' if offset else ''}")
    say(case.name)
    res = run_gdn_gpu(case, mode, offset_floats=offset, snapshots=snapshots)
    ref = orc.gdn_case(case, snapshots=snapshots)
    assert_gdn_parity(case, res[0], res[1], ref[0], ref[1])
    if snapshots:
        sn, st = res[2], res[1]
        err = np.abs(sn - ref[2]) / (1 + np.abs(ref[2]))
        assert err.size == 0 or err.max() <= TOL
        for s in range(case.n_seqs):
            if case.lengths[s] > 0:
                assert np.array_equal(sn[int(case.cu_seqlens[s + 1]) - 1], st[case.slot[s]]), s


@pytest.mark.parametrize("seed", range(4))
def test_gdn_random_batch_sweep(ssm, orc, seed):
    """Seeded random batches of 8-48 sequences (mostly short, a few long) at
    the model geometry (Hv 32, Hk 16, Dk = Dv = 128), so the chunked scan runs
    more workgroups than CUs (two per CU) and the per-token kernel a large
    grid; both prefills and the fp32 oracle."""
    rng = np.random.Generator(np.random.PCG64(99300 + seed))
    n = int(rng.integers(8, 49))
    long = rng.random(n) < 0.1
    lengths = [int(v) for v in np.where(long, rng.integers(100, 500, size=n), rng.integers(0, 60, size=n))]
    case = ssm_inputs.make_gdn_case(32, 16, 128, 128, lengths, [int(v) for v in rng.integers(0, 2, size=n)],
                                    99400 + seed, slots=[int(v) for v in rng.permutation(n + 3)[:n]],
                                    n_slots=n + 3, poison_fresh=True, sentinel_unused=True,
                                    name=f"gdn_batch_sweep{seed}_{n}seqs_{sum(lengths)}tok")
    say(case.name)
    y32, s32 = orc.gdn_case(case)
    for mode in ("prefill", "prefill_ws"):
        y, st = run_gdn_gpu(case, mode)
        assert_gdn_parity(case, y, st, y32, s32, label=f"{case.name} {mode}")


@pytest.mark.parametrize("mode", ["prefill", "prefill_ws", "decode"])
def test_gdn_scaling_by_two_is_exact(ssm, mode):
    """The delta rule is linear in (v, the start state) -- the keys enter
    only through the decayed, rank-1 transition -- and doubling is exact, so
    doubling v and every start state doubles y and the final states bit for
    bit, per token, in the chunked matrix form and in decode."""
    import dataclasses
    if mode == "decode":
        case = ssm_inputs.make_gdn_case(8, 4, 128, 64, [1] * 10, [i % 2 for i in range(10)], 97050)
    else:
        case = ssm_inputs.make_gdn_case(8, 4, 128, 64, [300, 33, 0, 130], [0, 1, 0, 1], 97051)
    twice = dataclasses.replace(case, v=case.v * np.float32(2), state=case.state * np.float32(2))
    y1, s1 = run_gdn_gpu(case, mode)
    y2, s2 = run_gdn_gpu(twice, mode)
    used = np.unique(case.slot)
    assert np.array_equal(y2, 2 * y1)
    assert np.array_equal(s2[used], 2 * s1[used])
