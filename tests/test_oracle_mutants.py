"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one (CPU only).  The committed oracle source is never changed: the
test copies it to a temporary directory, edits the copy's fp32 code, builds it
with the oracle's own flags and runs all pins against that build."""
import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

SRC = oracle_build.SRC

# (name, text of the fp32 code, replacement); each text occurs once in the file
MUTANTS = [
    ("y_reads_state_before_update",
     "                    h_p[n] = h_p[n] * dA_n + B_t[n] * x_dt;\n"
     "                    acc += h_p[n] * C_t[n];",
     "                    acc += h_p[n] * C_t[n];\n"
     "                    h_p[n] = h_p[n] * dA_n + B_t[n] * x_dt;"),
    ("interleaved_group_map", "const int64_t g = hd / heads_per_group;\n        /* h is",
     "const int64_t g = hd % G;\n        /* h is"),
    ("decay_sign_flipped", "expf(dt_t * A[hd])", "expf(-dt_t * A[hd])"),
    ("decay_dropped", "h_p[n] = h_p[n] * dA_n + B_t[n] * x_dt;",
     "h_p[n] = h_p[n] + B_t[n] * x_dt;"),
    ("dt_not_applied_to_x", "x[(t * H + hd) * P + p] * dt_t;\n                float *h_p",
     "x[(t * H + hd) * P + p];\n                float *h_p"),
    ("B_and_C_swapped",
     "h_p[n] = h_p[n] * dA_n + B_t[n] * x_dt;\n                    acc += h_p[n] * C_t[n];",
     "h_p[n] = h_p[n] * dA_n + C_t[n] * x_dt;\n                    acc += h_p[n] * B_t[n];"),
    ("fresh_flag_ignored", "        if (fresh[s])\n            memset(", "        if (0)\n            memset("),
    ("first_token_skipped",
     "for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {\n            const float dt_t",
     "for (int64_t t = cu_seqlens[s] + 1; t < cu_seqlens[s + 1]; ++t) {\n            const float dt_t"),
    ("rows_reversed_in_x", "x[(t * H + hd) * P + p] * dt_t;\n                float *h_p",
     "x[(t * H + hd) * P + (P - 1 - p)] * dt_t;\n                float *h_p"),
    ("slot_index_ignored", "float *h = state + ((int64_t)slot[s] * H + hd) * P * N;",
     "float *h = state + ((int64_t)s * H + hd) * P * N;"),
    ("state_index_transposed", "float *h_p = h + p * N;", "float *h_p = h + p;"),
    ("dt_head_index_wrong", "dt_eff_f32(dt[t * H + hd],", "dt_eff_f32(dt[t * H + (H - 1 - hd)],"),
    ("y_not_reset_per_row", "                float acc = 0.0f;\n                for (int64_t n = 0;",
     "                float acc = (float)p;\n                for (int64_t n = 0;"),
    # options
    ("softplus_cutoff_reversed", "if (softplus && v <= 20.0f)", "if (softplus && v > 20.0f)"),
    ("softplus_not_applied", "        v = log1pf(expf(v));", "        v = v;"),
    ("bias_ignored", "float v = dt_bias ? dt + dt_bias[hd] : dt;", "float v = dt;"),
    ("per_state_A_transposed", "expf(dt_t * A[hd * N + n])", "expf(dt_t * A[n * H + hd])"),
    ("per_state_A_ignored", "const float dA_n = a_per_state ? expf(dt_t * A[hd * N + n]) : dA;",
     "const float dA_n = a_per_state ? expf(dt_t * A[hd * N]) : dA;"),
    ("snapshot_of_previous_token",
     "memcpy(snapshots + (t * H + hd) * P * N, h,",
     "memcpy(snapshots + ((t > cu_seqlens[s] ? t - 1 : t) * H + hd) * P * N, h,"),
    # conv1d + SiLU
    ("silu_sign_flipped", "static float silu_f32(float v) { return v / (1.0f + expf(-v)); }",
     "static float silu_f32(float v) { return v / (1.0f + expf(v)); }"),
    ("conv_taps_reversed", "            for (int64_t i = 0; i < km1; ++i)\n"
     "                acc += hist[i] * wc[i];\n            out[t * D + c] = silu_f32(acc);",
     "            for (int64_t i = 0; i < km1; ++i)\n"
     "                acc += hist[i] * wc[km1 - 1 - i];\n            out[t * D + c] = silu_f32(acc);"),
    ("conv_own_tap_wrong", "float acc = xv * wc[km1];", "float acc = xv * wc[0];"),
    ("conv_no_silu", "out[t * D + c] = silu_f32(acc);", "out[t * D + c] = acc;"),
    ("conv_history_not_rolled", "                hist[i] = hist[i + 1];\n            if (km1 > 0)\n"
     "                hist[km1 - 1] = xv;\n            if (snapshots)\n                for (int64_t i = 0; i < km1; ++i)\n"
     "                    snapshots[(t * D + c) * km1 + i] = hist[i];\n        }\n    }\n    return 0;\n}\n\n/* The same in double",
     "                hist[i] = hist[i];\n            if (km1 > 0)\n"
     "                hist[km1 - 1] = xv;\n            if (snapshots)\n                for (int64_t i = 0; i < km1; ++i)\n"
     "                    snapshots[(t * D + c) * km1 + i] = hist[i];\n        }\n    }\n    return 0;\n}\n\n/* The same in double"),
    ("conv_fresh_not_zeroed", "        if (fresh[s])\n            for (int64_t i = 0; i < km1; ++i)\n"
     "                hist[i] = 0.0f;",
     "        if (0)\n            for (int64_t i = 0; i < km1; ++i)\n                hist[i] = 0.0f;"),
    ("conv_slot_ignored", "float *hist = conv_state + ((int64_t)slot[s] * D + c) * km1;",
     "float *hist = conv_state + ((int64_t)s * D + c) * km1;"),
    ("conv_snapshot_reversed", "snapshots[(t * D + c) * km1 + i] = hist[i];\n        }\n    }\n"
     "    return 0;\n}\n\n/* The same in double",
     "snapshots[(t * D + c) * km1 + i] = hist[km1 - 1 - i];\n        }\n    }\n"
     "    return 0;\n}\n\n/* The same in double"),
    # gated RMSNorm
    ("norm_sum_not_mean", "sqrtf(sum_sq / (float)L + eps)", "sqrtf(sum_sq + eps)"),
    ("norm_no_sqrt", "1.0f / sqrtf(sum_sq / (float)L + eps)", "1.0f / (sum_sq / (float)L + eps)"),
    ("norm_eps_outside_sqrt", "1.0f / sqrtf(sum_sq / (float)L + eps)",
     "1.0f / (sqrtf(sum_sq / (float)L) + eps)"),
    ("norm_weight_reversed", "out[r * L + d] = yr[d] * inv_rms * w[d] * silu_f32(zr[d]);",
     "out[r * L + d] = yr[d] * inv_rms * w[L - 1 - d] * silu_f32(zr[d]);"),
    ("norm_gate_not_silu", "out[r * L + d] = yr[d] * inv_rms * w[d] * silu_f32(zr[d]);",
     "out[r * L + d] = yr[d] * inv_rms * w[d] * zr[d];"),
    ("norm_gate_from_y", "out[r * L + d] = yr[d] * inv_rms * w[d] * silu_f32(zr[d]);",
     "out[r * L + d] = yr[d] * inv_rms * w[d] * silu_f32(yr[d]);"),
    ("norm_abs_not_square", "sum_sq += yr[d] * yr[d];", "sum_sq += fabsf(yr[d]);"),
    # gated delta rule
    ("gdn_decay_not_exp", "const float decay = expf(g[t * Hv + vh]);",
     "const float decay = g[t * Hv + vh];"),
    ("gdn_decay_after_retrieval",
     "                for (int64_t i = 0; i < Dk; ++i)\n                    row[i] = row[i] * decay;\n"
     "                float pred = 0.0f;\n                for (int64_t i = 0; i < Dk; ++i)\n"
     "                    pred += row[i] * kt[i];\n",
     "                float pred = 0.0f;\n                for (int64_t i = 0; i < Dk; ++i)\n"
     "                    pred += row[i] * kt[i];\n                for (int64_t i = 0; i < Dk; ++i)\n"
     "                    row[i] = row[i] * decay;\n"),
    ("gdn_delta_sign", "const float delta = (v[(t * Hv + vh) * Dv + j] - pred) * b;",
     "const float delta = (pred - v[(t * Hv + vh) * Dv + j]) * b;"),
    ("gdn_beta_ignored", "const float delta = (v[(t * Hv + vh) * Dv + j] - pred) * b;",
     "const float delta = (v[(t * Hv + vh) * Dv + j] - pred);"),
    ("gdn_write_with_query", "row[i] = row[i] + kt[i] * delta;\n                float acc = 0.0f;",
     "row[i] = row[i] + qt[i] * delta;\n                float acc = 0.0f;"),
    ("gdn_y_before_write",
     "                for (int64_t i = 0; i < Dk; ++i)\n                    row[i] = row[i] + kt[i] * delta;\n"
     "                float acc = 0.0f;\n                for (int64_t i = 0; i < Dk; ++i)\n"
     "                    acc += row[i] * qt[i];\n",
     "                float acc = 0.0f;\n                for (int64_t i = 0; i < Dk; ++i)\n"
     "                    acc += row[i] * qt[i];\n                for (int64_t i = 0; i < Dk; ++i)\n"
     "                    row[i] = row[i] + kt[i] * delta;\n"),
    ("gdn_gqa_contiguous", "        const int64_t kh = vh % Hk;\n        float *st",
     "        const int64_t kh = vh / (Hv / Hk);\n        float *st"),
    ("gdn_scale_missing", "acc += row[i] * qt[i];\n                y[(t * Hv + vh) * Dv + j] = scale * acc;",
     "acc += row[i] * qt[i];\n                y[(t * Hv + vh) * Dv + j] = acc;"),
    ("gdn_rows_overlap", "float *row = st + j * Dk;", "float *row = st + j;"),
    ("gdn_fresh_ignored", "        if (fresh[s])\n            for (int64_t e = 0; e < block; ++e)\n"
     "                st[e] = 0.0f;",
     "        if (0)\n            for (int64_t e = 0; e < block; ++e)\n                st[e] = 0.0f;"),
    ("gdn_value_index_wrong", "const float delta = (v[(t * Hv + vh) * Dv + j] - pred) * b;",
     "const float delta = (v[(t * Hv + vh) * Dv + (Dv - 1 - j)] - pred) * b;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    msrc = tmp_path / "ssm_oracle_mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = oracle_build.build(str(msrc), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
