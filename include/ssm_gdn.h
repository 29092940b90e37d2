/*
 * ssm_gdn.h -- the gated delta-rule recurrence for AMD Instinct MI355X
 * (gfx950), in the same library as ssm_scan.h, on the same register-resident
 * design as the Mamba2 scan.
 *
 * Defined by Foundry's kernels in "ssm_gated_delta.cu" (fc_ssm_recurrence for
 * one token, fc_ssm_recurrence_seq for a run of positions with optional
 * snapshots, fc_ssm_recurrence_slots for one token of several users).  Per
 * value head vh the state is Dv rows of Dk values, stored transposed as on that
 * page: row j (a value coordinate) contiguous over the key coordinate i.  Value
 * heads read the queries and keys of key head vh % Hk (the page's interleaved
 * GQA tiling).  Per token, for every row j:
 *     row   = row * exp(g)
 *     pred  = row . k
 *     delta = (v[j] - pred) * beta
 *     row   = row + k * delta
 *     y[j]  = scale * (row . q)
 * q and k are used as given, at any length (the page L2-normalises them in
 * a kernel of its own before the recurrence); no kernel here assumes unit
 * rows.  The update row <- row (I - beta k k^T) + beta v k^T is a contraction
 * while 0 <= beta |k|^2 <= 2, which unit keys with beta in [0, 1] satisfy;
 * beyond that the state can grow without bound, in the recurrence itself.
 * g is the log decay and beta the write strength, both per (token, value
 * head).  The kernel forms y as scale * (row_decayed . q +
 * delta * (k . q)), which equals the above in exact arithmetic.
 *
 * Conventions are those of ssm_scan.h: DEVICE arrays owned by the caller,
 * dense row-major fp32 (int32 / uint8 metadata), no allocation, no
 * synchronisation, one kernel on `stream`; SSM_OK or a negative SSM_ERR_* code
 * from ssm_scan.h, detected on the host before anything is enqueued.  With Dk
 * and Dv multiples of 4 and 16-byte aligned float arrays the kernels move
 * float4s, otherwise single floats (same results).  The packed-batch metadata
 * means what it means for ssm_scan_prefill (ssm_scan_check_metadata checks it):
 * a fresh sequence starts from a zero state without reading its slot, the
 * final state goes back to the slot, a zero-length sequence leaves a resuming
 * slot unchanged and zeroes a fresh one, slots not named are untouched.
 */
#ifndef SSM_GDN_H
#define SSM_GDN_H

#include <stddef.h>
#include <stdint.h>

#include "ssm_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_GDN_MAX_DK 256

typedef struct ssm_gdn_dims {
    int32_t n_v_heads;   /* Hv >= 1                                          */
    int32_t n_k_heads;   /* Hk >= 1, Hv % Hk == 0                            */
    int32_t d_k;         /* Dk in [1, SSM_GDN_MAX_DK]: key / query width     */
    int32_t d_v;         /* Dv >= 1: value width (state rows per head)       */
} ssm_gdn_dims;

/*
 * The recurrence over a packed batch of n_seqs sequences, n_tokens in all.
 *   cu_seqlens [n_seqs+1], slot [n_seqs], fresh [n_seqs]   as for ssm_scan_prefill
 *   q, k       [n_tokens][Hk][Dk]
 *   v          [n_tokens][Hv][Dv]
 *   g, beta    [n_tokens][Hv]   log decay (exp'd here) and write strength
 *   scale      multiplies y (the page uses 1/sqrt(Dk))
 *   state      [n_slots][Hv][Dv][Dk], updated in place
 *   y          [n_tokens][Hv][Dv]; must not alias any input
 *   snapshots  [n_tokens][Hv][Dv][Dk] or NULL: the state after every token
 * n_seqs == 0 is a no-op; with n_tokens == 0 the token arrays may be NULL.
 * Errors: SSM_ERR_NULL, SSM_ERR_DIMS (a size < 1, Hv % Hk != 0, n_seqs or
 * n_tokens < 0, n_slots < 1 with n_seqs > 0), SSM_ERR_UNSUPPORTED
 * (Dk > SSM_GDN_MAX_DK, or the grid would exceed 2^31-1 workgroups),
 * SSM_ERR_ALIGN, SSM_ERR_LAUNCH.
 */
int ssm_gdn_prefill(const ssm_gdn_dims *dims, int32_t n_seqs, int32_t n_tokens,
                    const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                    const float *q, const float *k, const float *v, const float *g,
                    const float *beta, float scale, float *state, int32_t n_slots, float *y,
                    float *snapshots, void *stream);

/*
 * The same recurrence over a packed batch, with the prefill of long sequences
 * in chunked matrix form on the matrix cores.  Over a chunk of 32 tokens the
 * per-token updates regroup into dense products ("ssm_gated_delta.cu" runs
 * them one token at a time; the regrouping is exact in real arithmetic, so
 * results agree with ssm_gdn_prefill to rounding):
 *     Delta = T diag(beta) (V - diag(gamma) K S0^T),  T = (I + A)^-1,
 *     A[t][s] = beta_t (gamma_t / gamma_s) (k_t . k_s) for s < t,
 *     y = scale (diag(gamma) Q S0^T + M Delta),  S' = gamma_31 S0 + Delta^T diag(gamma_31/gamma) K,
 * with gamma the running product of exp(g) from the chunk start and M the
 * decayed q . k for s <= t.  Two kernels on `stream`: per (sequence, chunk, key
 * head) T, M and the weights go to the workspace; then the chunks are scanned.
 *   max_seqlen  host int >= every sequence's length (precondition: chunks past
 *               ceil(max_seqlen/32) are not run, and no memory outside the
 *               arrays and the workspace is touched)
 *   workspace   DEVICE memory of at least ssm_gdn_prefill_workspace_size()
 *               bytes, 16-byte aligned, owned by the caller; its contents are
 *               scratch between calls.  Two calls in flight at once need two.
 * The chunked form runs for Dk in {64, 128}, Dv a multiple of 16, max_seqlen
 * >= 32 and 16-byte aligned float arrays; otherwise (and then the workspace
 * may be NULL) this is ssm_gdn_prefill without snapshots.  Errors as for
 * ssm_gdn_prefill, plus SSM_ERR_NULL for a missing workspace the chunked form
 * needs, SSM_ERR_DIMS for max_seqlen < 0 or a workspace below the size.
 */
int ssm_gdn_prefill_ws(const ssm_gdn_dims *dims, int32_t n_seqs, int32_t n_tokens,
                       const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                       const float *q, const float *k, const float *v, const float *g,
                       const float *beta, float scale, float *state, int32_t n_slots, float *y,
                       int32_t max_seqlen, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * Bytes of workspace ssm_gdn_prefill_ws needs for n_seqs sequences of at most
 * max_seqlen tokens (0 when it would not use the chunked form).  Host only.
 * Errors: SSM_ERR_NULL, SSM_ERR_DIMS (sizes as for ssm_gdn_prefill, n_seqs or
 * max_seqlen < 0).
 */
int ssm_gdn_prefill_workspace_size(const ssm_gdn_dims *dims, int32_t n_seqs, int32_t max_seqlen,
                                   size_t *bytes);

/*
 * One token for each of n_seqs sequences (fc_ssm_recurrence_slots): the same
 * as ssm_gdn_prefill with every length 1 and no cu_seqlens; the token arrays
 * are indexed by sequence.
 */
int ssm_gdn_decode(const ssm_gdn_dims *dims, int32_t n_seqs, const int32_t *slot,
                   const uint8_t *fresh, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, float scale, float *state,
                   int32_t n_slots, float *y, float *snapshots, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_GDN_H */
