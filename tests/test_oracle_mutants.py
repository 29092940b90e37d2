"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (CPU only).  The committed oracle source is never changed: the
test copies it to a temporary directory, edits the copy's fp32 function, builds
it with the oracle's own flags and runs all pins against that build."""
import os
import shutil

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

SRC = oracle_build.SRC

# (name, text in the fp32 function, replacement)
MUTANTS = [
    ("y_reads_state_before_update",
     "                    h_p[n] = h_p[n] * dA + B_t[n] * x_dt;\n"
     "                    acc += h_p[n] * C_t[n];",
     "                    acc += h_p[n] * C_t[n];\n"
     "                    h_p[n] = h_p[n] * dA + B_t[n] * x_dt;"),
    ("interleaved_group_map", "const int64_t g = hd / heads_per_group;",
     "const int64_t g = hd % G;"),
    ("decay_sign_flipped", "expf(dt_t * A[hd])", "expf(-dt_t * A[hd])"),
    ("decay_dropped", "h_p[n] = h_p[n] * dA + B_t[n] * x_dt;",
     "h_p[n] = h_p[n] + B_t[n] * x_dt;"),
    ("dt_not_applied_to_x", "x[(t * H + hd) * P + p] * dt_t;", "x[(t * H + hd) * P + p];"),
    ("B_and_C_swapped", "h_p[n] = h_p[n] * dA + B_t[n] * x_dt;\n                    acc += h_p[n] * C_t[n];",
     "h_p[n] = h_p[n] * dA + C_t[n] * x_dt;\n                    acc += h_p[n] * B_t[n];"),
    ("fresh_flag_ignored", "        if (fresh[s])\n            memset(", "        if (0)\n            memset("),
    ("first_token_skipped", "for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {\n            const float",
     "for (int64_t t = cu_seqlens[s] + 1; t < cu_seqlens[s + 1]; ++t) {\n            const float"),
    ("rows_reversed_in_x", "x[(t * H + hd) * P + p] * dt_t;", "x[(t * H + hd) * P + (P - 1 - p)] * dt_t;"),
    ("slot_index_ignored", "float *h = state + ((int64_t)slot[s] * H + hd) * P * N;",
     "float *h = state + ((int64_t)s * H + hd) * P * N;"),
    ("state_index_transposed", "float *h_p = h + p * N;", "float *h_p = h + p;"),
    ("dt_head_index_wrong", "const float dt_t = dt[t * H + hd];", "const float dt_t = dt[t * H + (H - 1 - hd)];"),
    ("y_not_reset_per_row", "                float acc = 0.0f;\n                for (int64_t n = 0; n < N; ++n) {\n                    h_p[n] = h_p[n] * dA",
     "                float acc = (float)p;\n                for (int64_t n = 0; n < N; ++n) {\n                    h_p[n] = h_p[n] * dA"),
]


def _f32_part(src):
    i = src.index("int ssm_oracle_scan_f32(")
    j = src.index("int ssm_oracle_scan_f64(")
    return i, j


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    i, j = _f32_part(src)
    part = src[i:j]
    assert part.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = src[:i] + part.replace(old, new) + src[j:]
    msrc = tmp_path / "ssm_oracle_mutant.c"
    msrc.write_text(mutated)
    lib = oracle_build.build(str(msrc), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
