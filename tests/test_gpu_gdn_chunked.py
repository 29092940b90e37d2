"""GPU parity for the chunked (matrix-core) gated delta-rule prefill,
``ssm_gdn_prefill_ws``, against the CPU oracle.

Bar: max |gpu - ref| / (1 + |ref|) <= 1e-4 on y and on the final state of
every used slot against the fp32 oracle (and the fp64 oracle on the long
workload); unused slots bit for bit unchanged.  The chunked form regroups the
recurrence's sums over 32-token chunks, so it agrees with the oracle and with
the per-token kernel to rounding, not bit for bit.
"""
import numpy as np
import pytest

import oracle
import ssm_inputs
from gpu_helpers import TOL, rel_err, run_gdn_gpu, say
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


def test_gdn_chunked_headline(ssm, orc):
    """1 x 4096, Hv 32 Hk 16 Dk = Dv = 128: the chunked form is taken (128
    chunks of 32 tokens, one 1680-float workspace unit per chunk and value head)."""
    case = ssm_inputs.gdn_workload("prefill4096")
    need = ssm.gdn_workspace_size(case.Hv, case.Hk, case.Dk, case.Dv, 1, 4096)
    assert need == 128 * 32 * 1680 * 4, need
    say(f"gdn chunked prefill 1x4096: workspace {need} bytes")
    y, st = run_gdn_gpu(case, "prefill_ws")
    y32, s32 = orc.gdn_case(case)
    assert_gdn_parity(case, y, st, y32, s32, label="chunked 1x4096 vs fp32 oracle")
    y64, s64 = orc.gdn_case(case, precision="f64")
    assert_gdn_parity(case, y, st, y64, s64, label="chunked 1x4096 vs fp64 oracle")


@pytest.mark.parametrize("Dk,Dv,Hv,Hk", [(128, 128, 4, 2), (64, 32, 3, 1), (128, 16, 2, 2),
                                         (64, 64, 4, 4)])
def test_gdn_chunked_varlen(ssm, orc, Dk, Dv, Hv, Hk):
    """Lengths around the chunk size and its 16-token tiles (0, 1, 15, 16, 17,
    31, 32, 33, 100, 250), fresh and resuming sequences, NaN-poisoned fresh
    slots, sentinel unused slots."""
    lengths = [0, 1, 15, 16, 17, 31, 32, 33, 100, 250]
    fresh = [1, 0, 1, 0, 0, 1, 0, 1, 0, 1]
    case = ssm_inputs.make_gdn_case(Hv, Hk, Dk, Dv, lengths, fresh, seed=700 + Dk + Dv,
                                    slots=[3, 9, 0, 5, 7, 1, 8, 2, 11, 12], n_slots=14,
                                    poison_fresh=True, sentinel_unused=True,
                                    name=f"gdn_chunked_Dk{Dk}_Dv{Dv}_Hv{Hv}_Hk{Hk}")
    assert ssm.gdn_workspace_size(Hv, Hk, Dk, Dv, len(lengths), 250) > 0
    y, st = run_gdn_gpu(case, "prefill_ws")
    y32, s32 = orc.gdn_case(case)
    assert_gdn_parity(case, y, st, y32, s32, label=case.name)


def test_gdn_chunked_decay_regimes(ssm, orc):
    """Eight value heads in four decay regimes over a long and a short sequence
    (one resumed): almost none (g = -0.001), moderate (-0.5), steep (-20: the
    decay from a chunk's start underflows fp32 within the chunk, so every
    factor the chunked form uses must come from differences of running sums,
    never a quotient of two decays) and bursts (-30 on 5% of the tokens, -0.01
    elsewhere)."""
    import dataclasses
    case = ssm_inputs.make_gdn_case(8, 4, 64, 32, [300, 130], [1, 0], seed=751,
                                    name="gdn_decay_regimes")
    rng = np.random.Generator(np.random.PCG64(7511))
    g = case.g.copy()
    T = g.shape[0]
    g[:, 0:2] = -0.001
    g[:, 2:4] = -0.5
    g[:, 4:6] = -20.0
    g[:, 6:8] = np.where(rng.uniform(size=(T, 2)) < 0.05, -30.0, -0.01)
    case = dataclasses.replace(case, g=g.astype(np.float32))
    y, st = run_gdn_gpu(case, "prefill_ws")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(st))
    y32, s32 = orc.gdn_case(case)
    assert_gdn_parity(case, y, st, y32, s32, label=case.name)


def test_gdn_chunked_matches_per_token(ssm, orc):
    """The chunked and the per-token kernels on the same batch agree within the bar."""
    case = ssm_inputs.make_gdn_case(8, 4, 128, 64, [300, 77, 160], [1, 0, 0], seed=733,
                                    name="gdn_chunked_vs_token")
    yc, sc = run_gdn_gpu(case, "prefill_ws")
    yt, st_ = run_gdn_gpu(case, "prefill")
    used = np.unique(case.slot)
    e_y, e_s = rel_err(yc, yt), rel_err(sc[used], st_[used])
    say(f"  chunked vs per-token: y {e_y:.3e} state {e_s:.3e}")
    assert e_y <= TOL and e_s <= TOL


def test_gdn_chunked_split_resume(ssm, orc):
    """T tokens in one call equal the same tokens in two calls with the state
    carried (cut inside a chunk and on a chunk boundary), within the bar, and
    a sequence alone equals itself inside a batch, bit for bit."""
    case = ssm_inputs.make_gdn_case(4, 2, 128, 32, [200], [1], seed=741, name="gdn_split")
    y_all, st_all = run_gdn_gpu(case, "prefill_ws")

    def part(a, b, state, fresh):
        return ssm_inputs.GdnCase(Hv=case.Hv, Hk=case.Hk, Dk=case.Dk, Dv=case.Dv,
                                  lengths=np.array([b - a], np.int32),
                                  cu_seqlens=np.array([0, b - a], np.int32), slot=case.slot,
                                  fresh=np.array([fresh], np.uint8), q=case.q[a:b],
                                  k=case.k[a:b], v=case.v[a:b], g=case.g[a:b],
                                  beta=case.beta[a:b], state=state, scale=case.scale)
    for cut in (37, 64, 150):
        y1, s1 = run_gdn_gpu(part(0, cut, case.state, 1), "prefill_ws")
        y2, s2 = run_gdn_gpu(part(cut, 200, s1, 0), "prefill_ws")
        e = max(rel_err(np.concatenate([y1, y2]), y_all), rel_err(s2, st_all))
        say(f"  split at {cut}: {e:.3e}")
        assert e <= TOL, cut
    batch = ssm_inputs.make_gdn_case(4, 2, 128, 32, [90, 200, 41], [0, 1, 0], seed=742,
                                     name="gdn_batch")
    yb, sb = run_gdn_gpu(batch, "prefill_ws", max_seqlen=200)
    a, b = int(batch.cu_seqlens[1]), int(batch.cu_seqlens[2])
    one = ssm_inputs.GdnCase(Hv=4, Hk=2, Dk=128, Dv=32, lengths=batch.lengths[1:2],
                             cu_seqlens=np.array([0, b - a], np.int32), slot=batch.slot[1:2],
                             fresh=batch.fresh[1:2], q=batch.q[a:b], k=batch.k[a:b],
                             v=batch.v[a:b], g=batch.g[a:b], beta=batch.beta[a:b],
                             state=batch.state, scale=batch.scale)
    y1, s1 = run_gdn_gpu(one, "prefill_ws", max_seqlen=200)
    assert np.array_equal(y1, yb[a:b])
    assert np.array_equal(s1[batch.slot[1]], sb[batch.slot[1]])


def test_gdn_chunked_short_batch_uses_per_token(ssm, orc):
    """Below 32 tokens (or with Dk outside {64, 128}) the entry point runs the
    per-token kernel: no workspace, same results as ssm_gdn_prefill."""
    assert ssm.gdn_workspace_size(4, 2, 128, 64, 3, 31) == 0
    assert ssm.gdn_workspace_size(4, 2, 100, 64, 3, 500) == 0
    case = ssm_inputs.make_gdn_case(4, 2, 128, 64, [31, 5, 20], [1, 0, 1], seed=751,
                                    name="gdn_short")
    y, st = run_gdn_gpu(case, "prefill_ws")
    yt, stt = run_gdn_gpu(case, "prefill")
    assert np.array_equal(y, yt) and np.array_equal(st, stt)
