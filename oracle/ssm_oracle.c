/*
 * ssm_oracle.c -- plain, sequential CPU oracle for the Mamba2 selective-state scan.
 *
 * TEST INFRASTRUCTURE.  This file is the correctness reference the GPU library
 * is compared against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it.  It shares no code, header or constant with the GPU
 * library and the GPU library never calls it.
 *
 * What it computes (the definition, written out):
 *   "The llama journey", Day 12: ggml's CPU reference loops over sequences,
 *   then tokens, then heads, then head-dim rows, then state elements, updates
 *   each state element and reads y out as the row's dot product with C.
 *   "The llama journey", Day 14 (the rewritten group kernel): per token the
 *   decay is exp(dt * A[head]) with one scalar A per head, x is scaled by dt,
 *   each state element becomes state * dA + B * (x * dt), y sums state * C
 *   over the state index using the state *after* the update, and heads map to
 *   B/C groups contiguously: group = head / (n_head / n_group).
 *   "perf(cuda): keep the Mamba2 scan state in registers, stage tokens by
 *   chunk #90" (Why / What changes / Testing): a batch mixes sequences that
 *   start from zero with sequences that resume from their state slot, and the
 *   state is left in that slot at the end.
 *
 * Readings where the pages leave a step open (each is listed with its reason
 * in the design notes): by default dt is used as given; B enters as dt*B
 * (not the zero-order-hold form); the final state goes back to the slot it was
 * read from; a fresh sequence never reads its slot; a zero-length sequence
 * leaves a resuming slot unchanged and zeroes a fresh one.
 *
 * Options (the _opt entry points; the plain ones are the defaults):
 *   dt_bias, dt_softplus -- dt_eff = dt + bias[head], then, with softplus on,
 *     softplus(v) = log1p(exp(v)) for v <= 20 and v itself above: the rule of
 *     ggml's scan kernels ("The llama journey", Day 11 and Day 14, the
 *     dt_soft_plus lines) and of Foundry's decay gate ("ssm_gated_delta.cu",
 *     fc_ssm_decay_gate, softplus of a bias plus dt).
 *   a_per_state -- A holds one value per (head, state index), [H][N], and each
 *     element decays by exp(dt * A[head][n]): the Mamba1 form of ggml's CPU
 *     table (Day 12, A as [d_state][n_head]) and of its Mamba1 kernel (Day 11).
 *   snapshots -- the state after every token, [T][H][P][N] in packed token
 *     order: the per-position snapshots Foundry keeps for speculative-decoding
 *     rollback ("ssm_gated_delta.cu", the snaps argument of the scan kernels).
 *
 * Arithmetic: plain C, compiled with -O2 -ffp-contract=off and no fast-math,
 * so every multiply and add rounds on its own, in the order written.  The f32
 * oracle uses expf; the f64 oracle takes the same fp32 inputs, widens them and
 * runs the identical loop nest in double with exp.
 *
 * Heads of one sequence are independent (nothing couples them), so the
 * (sequence, head) pairs may run on several threads; the result is bitwise the
 * same for any thread count because each pair owns its own slot rows and outputs.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

int ssm_oracle_version(void) { return 2; }

/* dt after the optional bias and softplus (see the header). */
static float dt_eff_f32(float dt, const float *dt_bias, int64_t hd, int32_t softplus)
{
    float v = dt_bias ? dt + dt_bias[hd] : dt;
    if (softplus && v <= 20.0f)
        v = log1pf(expf(v));
    return v;
}

static double dt_eff_f64(double dt, const float *dt_bias, int64_t hd, int32_t softplus)
{
    double v = dt_bias ? dt + (double)dt_bias[hd] : dt;
    if (softplus && v <= 20.0)
        v = log1p(exp(v));
    return v;
}

/* Returns 0, or -1 for bad dimensions. */
int ssm_oracle_scan_opt_f32(int32_t H, int32_t P, int32_t N, int32_t G, int32_t n_seqs,
                            const int32_t *cu_seqlens, const int32_t *slot,
                            const uint8_t *fresh, const float *x, const float *dt,
                            const float *A, const float *B, const float *C,
                            float *state, float *y, int32_t n_threads,
                            const float *dt_bias, int32_t dt_softplus, int32_t a_per_state,
                            float *snapshots)
{
    if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || n_seqs < 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t heads_per_group = H / G;
    const int64_t pairs = (int64_t)n_seqs * H;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t k = 0; k < pairs; ++k) {
        const int64_t s = k / H;
        const int64_t hd = k % H;
        const int64_t g = hd / heads_per_group;
        /* h is this (sequence, head)'s [P][N] block of its state slot. */
        float *h = state + ((int64_t)slot[s] * H + hd) * P * N;
        if (fresh[s])
            memset(h, 0, sizeof(float) * (size_t)P * (size_t)N);
        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const float dt_t = dt_eff_f32(dt[t * H + hd], dt_bias, hd, dt_softplus);
            const float dA = expf(dt_t * A[hd]);          /* one A per head */
            const float *B_t = B + (t * G + g) * N;
            const float *C_t = C + (t * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                const float x_dt = x[(t * H + hd) * P + p] * dt_t;
                float *h_p = h + p * N;
                float acc = 0.0f;
                for (int64_t n = 0; n < N; ++n) {
                    const float dA_n = a_per_state ? expf(dt_t * A[hd * N + n]) : dA;
                    h_p[n] = h_p[n] * dA_n + B_t[n] * x_dt;
                    acc += h_p[n] * C_t[n];
                }
                y[(t * H + hd) * P + p] = acc;
            }
            if (snapshots)
                memcpy(snapshots + (t * H + hd) * P * N, h, sizeof(float) * (size_t)P * (size_t)N);
        }
    }
    return 0;
}

int ssm_oracle_scan_f32(int32_t H, int32_t P, int32_t N, int32_t G, int32_t n_seqs,
                        const int32_t *cu_seqlens, const int32_t *slot,
                        const uint8_t *fresh, const float *x, const float *dt,
                        const float *A, const float *B, const float *C,
                        float *state, float *y, int32_t n_threads)
{
    return ssm_oracle_scan_opt_f32(H, P, N, G, n_seqs, cu_seqlens, slot, fresh, x, dt, A, B, C,
                                   state, y, n_threads, NULL, 0, 0, NULL);
}

/* The same loop nest in double.  Inputs stay fp32 (the bits both sides see);
 * the state, y and snapshots are double. */
int ssm_oracle_scan_opt_f64(int32_t H, int32_t P, int32_t N, int32_t G, int32_t n_seqs,
                            const int32_t *cu_seqlens, const int32_t *slot,
                            const uint8_t *fresh, const float *x, const float *dt,
                            const float *A, const float *B, const float *C,
                            double *state, double *y, int32_t n_threads,
                            const float *dt_bias, int32_t dt_softplus, int32_t a_per_state,
                            double *snapshots)
{
    if (H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || n_seqs < 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t heads_per_group = H / G;
    const int64_t pairs = (int64_t)n_seqs * H;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t k = 0; k < pairs; ++k) {
        const int64_t s = k / H;
        const int64_t hd = k % H;
        const int64_t g = hd / heads_per_group;
        double *h = state + ((int64_t)slot[s] * H + hd) * P * N;
        if (fresh[s])
            for (int64_t i = 0; i < (int64_t)P * N; ++i)
                h[i] = 0.0;
        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const double dt_t = dt_eff_f64((double)dt[t * H + hd], dt_bias, hd, dt_softplus);
            const double dA = exp(dt_t * (double)A[hd]);
            const float *B_t = B + (t * G + g) * N;
            const float *C_t = C + (t * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                const double x_dt = (double)x[(t * H + hd) * P + p] * dt_t;
                double *h_p = h + p * N;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double dA_n = a_per_state ? exp(dt_t * (double)A[hd * N + n]) : dA;
                    h_p[n] = h_p[n] * dA_n + (double)B_t[n] * x_dt;
                    acc += h_p[n] * (double)C_t[n];
                }
                y[(t * H + hd) * P + p] = acc;
            }
            if (snapshots)
                for (int64_t i = 0; i < (int64_t)P * N; ++i)
                    snapshots[(t * H + hd) * P * N + i] = h[i];
        }
    }
    return 0;
}

int ssm_oracle_scan_f64(int32_t H, int32_t P, int32_t N, int32_t G, int32_t n_seqs,
                        const int32_t *cu_seqlens, const int32_t *slot,
                        const uint8_t *fresh, const float *x, const float *dt,
                        const float *A, const float *B, const float *C,
                        double *state, double *y, int32_t n_threads)
{
    return ssm_oracle_scan_opt_f64(H, P, N, G, n_seqs, cu_seqlens, slot, fresh, x, dt, A, B, C,
                                   state, y, n_threads, NULL, 0, 0, NULL);
}
