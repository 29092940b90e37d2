/*
 * ssm_conv_norm.h -- the two steps on either side of the Mamba2 scan in a
 * layer, for AMD Instinct MI355X (gfx950), in the same library as ssm_scan.h.
 *
 *   ssm_conv1d_silu_prefill / ssm_conv1d_silu_decode
 *     Causal depthwise conv1d followed by SiLU, with a rolling per-channel
 *     history of the last K-1 raw inputs kept in a state slot.  Defined by
 *     Foundry's kernels in "ssm_gated_delta.cu": fc_ssm_conv1d_silu (one
 *     token), fc_ssm_conv1d_silu_seq (a run of positions, optional per-position
 *     snapshots) and fc_ssm_conv1d_silu_slots (one token for each of several
 *     users).  For channel c at each token, with hist the history oldest first:
 *         out[t][c] = silu( x[t][c] * w[c][K-1] + sum_{i<K-1} hist[i] * w[c][i] )
 *     then the history drops its oldest value and appends x[t][c].
 *     silu(v) = v / (1 + exp(-v)).  "The llama journey" (Day 11) names the
 *     same step in ggml as ssm_conv.
 *
 *   ssm_gated_rmsnorm
 *     Foundry's fc_ssm_gated_norm ("ssm_gated_delta.cu"): every row of L
 *     values (one head of one token) is divided by its root mean square
 *     sqrt(sum(y^2)/L + eps), multiplied by a weight of length L that all rows
 *     share, and by silu of the gate z.
 *
 * Conventions are those of ssm_scan.h: every array is DEVICE memory owned by
 * the caller, dense row-major fp32 (int32 / uint8 for metadata); the library
 * allocates nothing, never synchronizes and enqueues one kernel on `stream`
 * (a hipStream_t; NULL = the null stream).  Return value: SSM_OK or a negative
 * SSM_ERR_* code from ssm_scan.h, detected on the host before anything is
 * enqueued; ssm_scan_last_hip_error() explains an SSM_ERR_LAUNCH.  Arrays need
 * 4-byte alignment; with D (or L) a multiple of 4 and 16-byte aligned arrays
 * the kernels move float4s, otherwise single floats (same results).  The
 * packed-batch metadata (cu_seqlens, slot, fresh) means what it means for
 * ssm_scan_prefill, and ssm_scan_check_metadata checks it.
 */
#ifndef SSM_CONV_NORM_H
#define SSM_CONV_NORM_H

#include <stddef.h>
#include <stdint.h>

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_CONV_MAX_KERNEL 4

typedef struct ssm_conv_dims {
    int32_t channels;   /* D >= 1: depthwise channels (a Mamba2 layer: H*P + 2*G*N)      */
    int32_t kernel;     /* K in [1, SSM_CONV_MAX_KERNEL]: taps; the history holds K-1     */
} ssm_conv_dims;

/*
 * Causal conv1d + SiLU over a packed batch of n_seqs sequences, n_tokens
 * tokens in all.
 *   cu_seqlens  [n_seqs+1]   token offsets: cu[0] = 0, nondecreasing, cu[n_seqs] = n_tokens
 *   slot        [n_seqs]     history slot of each sequence, distinct, in [0, n_slots)
 *   fresh       [n_seqs]     1 = start from a zero history and never read the slot
 *   x           [n_tokens][D]  raw inputs, token-major
 *   weight      [D][K]       taps of each channel; tap K-1 multiplies the current token
 *   conv_state  [n_slots][D][K-1]  history, oldest first; read unless fresh, written
 *                            for every named sequence; slots not named are untouched.
 *                            May be NULL when K == 1 (there is no history).
 *   out         [n_tokens][D]  silu of the convolution; must not alias any input
 *   snapshots   [n_tokens][D][K-1] or NULL: the history after each token, for
 *                            rolling back a partly accepted run of draft tokens
 *                            (fc_ssm_conv1d_silu_seq's snaps).
 * A zero-length sequence leaves a resuming slot unchanged and zeroes a fresh
 * one.  n_seqs == 0 is a no-op; with n_tokens == 0, x, out and snapshots may
 * be NULL.  Errors: SSM_ERR_NULL (a needed pointer is
 * NULL), SSM_ERR_DIMS (D < 1, K < 1, n_seqs or n_tokens < 0, n_slots < 1 with
 * n_seqs > 0), SSM_ERR_UNSUPPORTED (K > SSM_CONV_MAX_KERNEL), SSM_ERR_ALIGN,
 * SSM_ERR_LAUNCH.
 */
int ssm_conv1d_silu_prefill(const ssm_conv_dims *dims, int32_t n_seqs, int32_t n_tokens,
                            const int32_t *cu_seqlens, const int32_t *slot,
                            const uint8_t *fresh, const float *x, const float *weight,
                            float *conv_state, int32_t n_slots, float *out, float *snapshots,
                            void *stream);

/*
 * One token for each of n_seqs sequences (the slot form of multi-user decode,
 * fc_ssm_conv1d_silu_slots): the same as ssm_conv1d_silu_prefill with every
 * length 1 and no cu_seqlens.  x, out [n_seqs][D]; the rest as above.
 */
int ssm_conv1d_silu_decode(const ssm_conv_dims *dims, int32_t n_seqs, const int32_t *slot,
                           const uint8_t *fresh, const float *x, const float *weight,
                           float *conv_state, int32_t n_slots, float *out, void *stream);

/*
 * Gated RMSNorm over n_rows rows of row_len values:
 *   out[r][d] = y[r][d] * (1 / sqrt(sum_d' y[r][d']^2 / row_len + eps)) * weight[d] * silu(z[r][d])
 * y, z, out [n_rows][row_len]; weight [row_len], shared by all rows (for y of
 * shape [T][H][P] normalised per head: n_rows = T*H, row_len = P).  out must
 * not alias y or z.  n_rows == 0 is a no-op.  Errors: SSM_ERR_NULL,
 * SSM_ERR_DIMS (n_rows < 0, row_len < 1, eps negative or not finite),
 * SSM_ERR_ALIGN, SSM_ERR_LAUNCH.
 */
int ssm_gated_rmsnorm(int64_t n_rows, int32_t row_len, const float *y, const float *z,
                      const float *weight, float eps, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CONV_NORM_H */
