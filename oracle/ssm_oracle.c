/*
 * ssm_oracle.c -- plain, sequential CPU oracle for the Mamba2 selective-state scan
 * and the two steps beside it in a layer (causal conv1d + SiLU with a rolling
 * history, gated RMSNorm), and the gated delta-rule recurrence (the second
 * workload on the same register design); each section cites its source.
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

int ssm_oracle_version(void) { return 4; }

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

/* ------------------------------------------------------------------------
 * The two steps on either side of the scan in a Mamba2-style layer.
 *
 * SiLU: silu(v) = v * sigmoid(v), written as v / (1 + exp(-v)) as in the
 * fc_ssm_silu helper of "ssm_gated_delta.cu".
 * ------------------------------------------------------------------------ */
static float silu_f32(float v) { return v / (1.0f + expf(-v)); }
static double silu_f64(double v) { return v / (1.0 + exp(-v)); }

/*
 * Causal depthwise conv1d + SiLU with a rolling per-channel history, over a
 * packed batch ("ssm_gated_delta.cu": fc_ssm_conv1d_silu for one token,
 * fc_ssm_conv1d_silu_seq for a run of positions, fc_ssm_conv1d_silu_slots for
 * one token of several users).  For channel c the window at each token is the
 * K-1 previous raw inputs, oldest first, followed by the token's own input;
 *     out[t][c] = silu( x[t][c] * w[c][K-1] + sum_{i<K-1} hist[i] * w[c][i] )
 * accumulated in that order (the token's own tap first, then the history from
 * oldest to newest), after which the history drops its oldest value and
 * appends x[t][c].
 *
 * Layouts: x and out [T][D] token-major (tokens of all sequences packed as for
 * the scan), w [D][K], conv_state [n_slots][D][K-1] with each channel's
 * history oldest..newest, snapshots (optional) [T][D][K-1] = the history after
 * each token.  Sequence s reads its history from slot[s] unless fresh[s] (then
 * it starts from zeros and never reads the slot) and leaves it there.
 * Channels and sequences are independent, so (sequence, channel) pairs may run
 * on several threads with bitwise the same result.
 */
int ssm_oracle_conv1d_silu_f32(int32_t D, int32_t K, int32_t n_seqs,
                               const int32_t *cu_seqlens, const int32_t *slot,
                               const uint8_t *fresh, const float *x, const float *w,
                               float *conv_state, float *out, float *snapshots,
                               int32_t n_threads)
{
    if (D <= 0 || K < 1 || n_seqs < 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t km1 = K - 1;
    const int64_t pairs = (int64_t)n_seqs * D;

#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t k = 0; k < pairs; ++k) {
        const int64_t s = k / D;
        const int64_t c = k % D;
        float *hist = conv_state + ((int64_t)slot[s] * D + c) * km1;
        const float *wc = w + c * K;
        if (fresh[s])
            for (int64_t i = 0; i < km1; ++i)
                hist[i] = 0.0f;
        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const float xv = x[t * D + c];
            float acc = xv * wc[km1];
            for (int64_t i = 0; i < km1; ++i)
                acc += hist[i] * wc[i];
            out[t * D + c] = silu_f32(acc);
            for (int64_t i = 0; i + 1 < km1; ++i)
                hist[i] = hist[i + 1];
            if (km1 > 0)
                hist[km1 - 1] = xv;
            if (snapshots)
                for (int64_t i = 0; i < km1; ++i)
                    snapshots[(t * D + c) * km1 + i] = hist[i];
        }
    }
    return 0;
}

/* The same in double (inputs fp32; history, output and snapshots double). */
int ssm_oracle_conv1d_silu_f64(int32_t D, int32_t K, int32_t n_seqs,
                               const int32_t *cu_seqlens, const int32_t *slot,
                               const uint8_t *fresh, const float *x, const float *w,
                               double *conv_state, double *out, double *snapshots,
                               int32_t n_threads)
{
    if (D <= 0 || K < 1 || n_seqs < 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t km1 = K - 1;
    const int64_t pairs = (int64_t)n_seqs * D;

#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t k = 0; k < pairs; ++k) {
        const int64_t s = k / D;
        const int64_t c = k % D;
        double *hist = conv_state + ((int64_t)slot[s] * D + c) * km1;
        const float *wc = w + c * K;
        if (fresh[s])
            for (int64_t i = 0; i < km1; ++i)
                hist[i] = 0.0;
        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const double xv = (double)x[t * D + c];
            double acc = xv * (double)wc[km1];
            for (int64_t i = 0; i < km1; ++i)
                acc += hist[i] * (double)wc[i];
            out[t * D + c] = silu_f64(acc);
            for (int64_t i = 0; i + 1 < km1; ++i)
                hist[i] = hist[i + 1];
            if (km1 > 0)
                hist[km1 - 1] = xv;
            if (snapshots)
                for (int64_t i = 0; i < km1; ++i)
                    snapshots[(t * D + c) * km1 + i] = hist[i];
        }
    }
    return 0;
}

/*
 * Gated RMSNorm ("ssm_gated_delta.cu", fc_ssm_gated_norm): each row of L
 * values (one head of one token) is divided by its root mean square, then
 * scaled by a weight that all rows share and by silu of the gate:
 *     rms      = sqrt( (sum_d y[d]^2) / L + eps )
 *     out[d]   = y[d] * (1 / rms) * w[d] * silu(z[d])
 * multiplied left to right in that order.  y, z, out [n_rows][L]; w [L].
 */
int ssm_oracle_gated_rmsnorm_f32(int64_t n_rows, int32_t L, const float *y, const float *z,
                                 const float *w, float eps, float *out, int32_t n_threads)
{
    if (n_rows < 0 || L <= 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;

#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t r = 0; r < n_rows; ++r) {
        const float *yr = y + r * L;
        const float *zr = z + r * L;
        float sum_sq = 0.0f;
        for (int64_t d = 0; d < L; ++d)
            sum_sq += yr[d] * yr[d];
        const float inv_rms = 1.0f / sqrtf(sum_sq / (float)L + eps);
        for (int64_t d = 0; d < L; ++d)
            out[r * L + d] = yr[d] * inv_rms * w[d] * silu_f32(zr[d]);
    }
    return 0;
}

int ssm_oracle_gated_rmsnorm_f64(int64_t n_rows, int32_t L, const float *y, const float *z,
                                 const float *w, double eps, double *out, int32_t n_threads)
{
    if (n_rows < 0 || L <= 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;

#pragma omp parallel for schedule(static) num_threads(n_threads)
    for (int64_t r = 0; r < n_rows; ++r) {
        const float *yr = y + r * L;
        const float *zr = z + r * L;
        double sum_sq = 0.0;
        for (int64_t d = 0; d < L; ++d)
            sum_sq += (double)yr[d] * (double)yr[d];
        const double inv_rms = 1.0 / sqrt(sum_sq / (double)L + eps);
        for (int64_t d = 0; d < L; ++d)
            out[r * L + d] = (double)yr[d] * inv_rms * (double)w[d] * silu_f64((double)zr[d]);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Gated delta-rule recurrence ("ssm_gated_delta.cu": fc_ssm_recurrence for one
 * token, fc_ssm_recurrence_seq for a run of positions with optional
 * snapshots, fc_ssm_recurrence_slots for one token of several users).
 *
 * Per value head vh the state is Dv rows of Dk values, stored transposed as on
 * that page: row j (one value coordinate) is contiguous over the key
 * coordinate i.  Queries and keys come per key head kh; value heads map to key
 * heads interleaved, kh = vh % Hk (the page's GQA tiling vh = r*Hk + kh).  Per
 * token, for every row j, in this order:
 *     row[i] = row[i] * exp(g)                          (decay)
 *     pred   = sum_i row[i] * k[i]                      (retrieval)
 *     delta  = (v[j] - pred) * beta
 *     row[i] = row[i] + k[i] * delta                    (rank-1 write)
 *     y[j]   = scale * sum_i row[i] * q[i]              (read after the write)
 * Layouts: q, k [T][Hk][Dk]; v, y [T][Hv][Dv]; g (log decay, exp'd here) and
 * beta [T][Hv]; state [n_slots][Hv][Dv][Dk]; snapshots [T][Hv][Dv][Dk].  Slot,
 * fresh and zero-length rules are the scan's.  (sequence, value head) pairs
 * are independent and may run on several threads.
 * ------------------------------------------------------------------------ */
int ssm_oracle_gdn_f32(int32_t Hv, int32_t Hk, int32_t Dk, int32_t Dv, int32_t n_seqs,
                       const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                       const float *q, const float *k, const float *v, const float *g,
                       const float *beta, float scale, float *state, float *y,
                       float *snapshots, int32_t n_threads)
{
    if (Hv <= 0 || Hk <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0 || n_seqs < 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t pairs = (int64_t)n_seqs * Hv;
    const int64_t block = (int64_t)Dv * Dk;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t w = 0; w < pairs; ++w) {
        const int64_t s = w / Hv;
        const int64_t vh = w % Hv;
        const int64_t kh = vh % Hk;
        float *st = state + ((int64_t)slot[s] * Hv + vh) * block;
        if (fresh[s])
            for (int64_t e = 0; e < block; ++e)
                st[e] = 0.0f;
        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const float decay = expf(g[t * Hv + vh]);
            const float b = beta[t * Hv + vh];
            const float *kt = k + (t * Hk + kh) * Dk;
            const float *qt = q + (t * Hk + kh) * Dk;
            for (int64_t j = 0; j < Dv; ++j) {
                float *row = st + j * Dk;
                for (int64_t i = 0; i < Dk; ++i)
                    row[i] = row[i] * decay;
                float pred = 0.0f;
                for (int64_t i = 0; i < Dk; ++i)
                    pred += row[i] * kt[i];
                const float delta = (v[(t * Hv + vh) * Dv + j] - pred) * b;
                for (int64_t i = 0; i < Dk; ++i)
                    row[i] = row[i] + kt[i] * delta;
                float acc = 0.0f;
                for (int64_t i = 0; i < Dk; ++i)
                    acc += row[i] * qt[i];
                y[(t * Hv + vh) * Dv + j] = scale * acc;
            }
            if (snapshots)
                memcpy(snapshots + (t * Hv + vh) * block, st, sizeof(float) * (size_t)block);
        }
    }
    return 0;
}

/* The same in double (inputs fp32; state, y and snapshots double). */
int ssm_oracle_gdn_f64(int32_t Hv, int32_t Hk, int32_t Dk, int32_t Dv, int32_t n_seqs,
                       const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                       const float *q, const float *k, const float *v, const float *g,
                       const float *beta, double scale, double *state, double *y,
                       double *snapshots, int32_t n_threads)
{
    if (Hv <= 0 || Hk <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0 || n_seqs < 0)
        return -1;
    if (n_threads < 1)
        n_threads = 1;
    const int64_t pairs = (int64_t)n_seqs * Hv;
    const int64_t block = (int64_t)Dv * Dk;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t w = 0; w < pairs; ++w) {
        const int64_t s = w / Hv;
        const int64_t vh = w % Hv;
        const int64_t kh = vh % Hk;
        double *st = state + ((int64_t)slot[s] * Hv + vh) * block;
        if (fresh[s])
            for (int64_t e = 0; e < block; ++e)
                st[e] = 0.0;
        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const double decay = exp((double)g[t * Hv + vh]);
            const double b = (double)beta[t * Hv + vh];
            const float *kt = k + (t * Hk + kh) * Dk;
            const float *qt = q + (t * Hk + kh) * Dk;
            for (int64_t j = 0; j < Dv; ++j) {
                double *row = st + j * Dk;
                for (int64_t i = 0; i < Dk; ++i)
                    row[i] = row[i] * decay;
                double pred = 0.0;
                for (int64_t i = 0; i < Dk; ++i)
                    pred += row[i] * (double)kt[i];
                const double delta = ((double)v[(t * Hv + vh) * Dv + j] - pred) * b;
                for (int64_t i = 0; i < Dk; ++i)
                    row[i] = row[i] + (double)kt[i] * delta;
                double acc = 0.0;
                for (int64_t i = 0; i < Dk; ++i)
                    acc += row[i] * (double)qt[i];
                y[(t * Hv + vh) * Dv + j] = scale * acc;
            }
            if (snapshots)
                for (int64_t e = 0; e < block; ++e)
                    snapshots[(t * Hv + vh) * block + e] = st[e];
        }
    }
    return 0;
}
