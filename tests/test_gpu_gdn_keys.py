"""GPU parity for the gated delta-rule kernels with queries and keys that are
not unit length.

The recurrence takes q and k as given (the page normalises them in a kernel of
its own before the recurrence); its update row <- row (I - beta k k^T) + ...
is a contraction while 0 <= beta |k|^2 <= 2.  These cases draw q and k rows of
length U[0.25, 1.4] and write strengths drawn, 0, 1/2 and 1 (so beta |k|^2
reaches 1.96), and run them through the per-token prefill, the chunked
matrix-core prefill (whose (I + A)^-1 and K K^T scale with |k|^2) and decode,
against the fp32 and fp64 oracle.  Bar as everywhere: max |gpu - ref| /
(1 + |ref|) <= 1e-4 on y and on the final state of every used slot.
"""
import pytest

import oracle
import ssm_inputs
from gpu_helpers import TOL, rel_err, run_gdn_gpu, say
from test_gpu_gdn import assert_gdn_parity

pytestmark = pytest.mark.gpu

NORMS = (0.25, 1.4)


@pytest.fixture(scope="module")
def ssm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mamba2_selective_scan_amd as m
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _check(case, y, st, orc, label):
    y32, s32 = orc.gdn_case(case)
    assert_gdn_parity(case, y, st, y32, s32, label=f"{label} vs fp32 oracle")
    y64, s64 = orc.gdn_case(case, precision="f64")
    assert_gdn_parity(case, y, st, y64, s64, label=f"{label} vs fp64 oracle")


@pytest.mark.parametrize("beta", [None, 0.0, 0.5, 1.0])
def test_gdn_keys_per_token_mixed(ssm, orc, beta):
    """The mixed batch's geometry (Dk 100, Dv 96, varlen, fresh and resumed,
    poisoned fresh slots, sentinel unused slots) through ssm_gdn_prefill."""
    case = ssm_inputs.make_gdn_case(
        8, 4, 100, 96, [1, 7, 25, 26, 64, 100, 150, 150], [1 - (i % 2) for i in range(8)],
        900 + int(10 * (beta or 0.3)), slots=[3, 9, 0, 5, 7, 1, 8, 2], n_slots=10,
        poison_fresh=True, sentinel_unused=True, qk_norm=NORMS, beta=beta,
        name=f"gdn_keys_mixed_beta{beta}")
    say(f"{case.name}: per-token prefill")
    y, st = run_gdn_gpu(case, "prefill")
    _check(case, y, st, orc, case.name)


@pytest.mark.parametrize("beta", [None, 0.0, 0.5, 1.0])
@pytest.mark.parametrize("Dk,Dv,Hv,Hk", [(128, 128, 4, 2), (64, 32, 3, 1)])
def test_gdn_keys_chunked(ssm, orc, beta, Dk, Dv, Hv, Hk):
    """ssm_gdn_prefill_ws in chunked matrix form: lengths around the 16-token
    chunk, fresh and resumed, with keys of any length."""
    lengths = [0, 1, 15, 16, 17, 33, 100, 250]
    fresh = [1, 0, 1, 0, 0, 1, 0, 1]
    case = ssm_inputs.make_gdn_case(Hv, Hk, Dk, Dv, lengths, fresh,
                                    910 + Dk + Dv + int(10 * (beta or 0.3)),
                                    slots=[3, 9, 0, 5, 7, 1, 8, 2], n_slots=11,
                                    poison_fresh=True, sentinel_unused=True, qk_norm=NORMS,
                                    beta=beta, name=f"gdn_keys_chunked_Dk{Dk}_beta{beta}")
    assert ssm.gdn_workspace_size(Hv, Hk, Dk, Dv, len(lengths), 250) > 0
    say(f"{case.name}: chunked prefill")
    y, st = run_gdn_gpu(case, "prefill_ws")
    _check(case, y, st, orc, case.name)


def test_gdn_keys_chunked_long(ssm, orc):
    """A 2048-token sequence at the model geometry (Hv 32, Hk 16, D 128) with
    keys of any length, chunked form."""
    case = ssm_inputs.make_gdn_case(32, 16, 128, 128, [2048], [0], 930, qk_norm=NORMS,
                                    name="gdn_keys_chunked_1x2048")
    say(f"{case.name}: chunked prefill")
    y, st = run_gdn_gpu(case, "prefill_ws")
    _check(case, y, st, orc, case.name)


@pytest.mark.parametrize("beta", [None, 1.0])
def test_gdn_keys_decode(ssm, orc, beta):
    """16 sequences x 1 token at the model geometry through ssm_gdn_decode,
    and the same batch as one-token prefill (its row sums split over another
    lane count, so the two agree within the bar, not bit for bit)."""
    case = ssm_inputs.make_gdn_case(32, 16, 128, 128, [1] * 16, [0] * 8 + [1] * 8,
                                    940 + int(beta or 0), qk_norm=NORMS, beta=beta,
                                    name=f"gdn_keys_decode16_beta{beta}")
    say(f"{case.name}: decode")
    y, st = run_gdn_gpu(case, "decode")
    _check(case, y, st, orc, case.name)
    yp, stp = run_gdn_gpu(case, "prefill")
    assert rel_err(st, stp) <= TOL and rel_err(y, yp) <= TOL
