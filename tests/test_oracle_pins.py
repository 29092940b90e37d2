"""The oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import ssm_inputs
import oracle_pins
from oracle_pins import rel_err


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("name", ["tiny", "decode16", "mixed", "decode256", "prefill4096"])
def test_f32_against_f64(orc, name):
    """fp32 oracle within the parity bound of the fp64 oracle on every workload."""
    case = ssm_inputs.workload(name)
    y32, st32 = orc.scan_case(case, precision="f32")
    y64, st64 = orc.scan_case(case, precision="f64")
    used = np.unique(case.slot)
    assert np.all(np.isfinite(y32)) and np.all(np.isfinite(st32[used]))
    assert rel_err(y32, y64) <= 1e-4
    assert rel_err(st32[used], st64[used]) <= 1e-4


@pytest.mark.parametrize("name", ["tiny", "decode16", "mixed", "decode256", "prefill4096"])
def test_conv_f32_against_f64(orc, name):
    """conv1d + SiLU: fp32 oracle within the parity bound of the fp64 oracle."""
    case = ssm_inputs.conv_workload(name)
    o32, s32 = orc.conv_case(case, precision="f32")
    o64, s64 = orc.conv_case(case, precision="f64")
    used = np.unique(case.slot)
    assert np.all(np.isfinite(o32))
    assert rel_err(o32, o64) <= 1e-4
    assert np.array_equal(s32[used], s64[used].astype(np.float32))   # raw inputs, copied


@pytest.mark.parametrize("name", ["tiny", "decode16", "mixed", "decode256", "prefill4096"])
def test_norm_f32_against_f64(orc, name):
    case = ssm_inputs.norm_workload(name)
    assert rel_err(orc.norm_case(case, precision="f32"), orc.norm_case(case, precision="f64")) <= 1e-4


@pytest.mark.parametrize("name", ["tiny", "decode16", "mixed", "decode256", "prefill4096"])
def test_gdn_f32_against_f64(orc, name):
    """Gated delta rule: fp32 oracle within the parity bound of the fp64 oracle."""
    case = ssm_inputs.gdn_workload(name)
    y32, s32 = orc.gdn_case(case, precision="f32")
    y64, s64 = orc.gdn_case(case, precision="f64")
    used = np.unique(case.slot)
    assert np.all(np.isfinite(y32)) and np.all(np.isfinite(s32[used]))
    assert rel_err(y32, y64) <= 1e-4
    assert rel_err(s32[used], s64[used]) <= 1e-4
