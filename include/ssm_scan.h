/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) Mamba2 selective-state scan.
 *
 * The operation.  For every sequence s of a packed token batch, every head h,
 * head-dim row p and state index n, tokens strictly in order:
 *
 *     dA       = exp(dt[t][h] * A[h])
 *     st[p][n] = st[p][n] * dA + B[t][g][n] * (x[t][h][p] * dt[t][h])
 *     y[t][h][p] = sum over n of st[p][n] * C[t][g][n]    (after the update)
 *
 * with g = h / (n_heads / n_groups): heads share B and C by contiguous group.
 * This is the recurrence of ggml's CPU scan and of its rewritten Mamba2 group
 * kernel ("The llama journey", Day 12 operand table and loop nest, Day 14
 * kernel), over a batch that mixes sequences starting from zero with
 * sequences resuming from their state slot ("perf(cuda): keep the Mamba2 scan
 * state in registers, stage tokens by chunk #90", What changes and Testing).
 * dt is used as given (no softplus is applied) and B enters as dt*B.
 *
 * Conventions shared by every entry point:
 *  - All array pointers are DEVICE pointers, dense and row-major in the
 *    layouts written beside each argument, owned by the caller.  float arrays
 *    are fp32 and must be 4-byte aligned; 16-byte alignment together with
 *    d_state % 4 == 0 and head_dim % 4 == 0 selects the vector (float4) path.
 *  - The library allocates nothing and never synchronizes (the one exception
 *    is the debugging aid ssm_scan_check_metadata, which waits for its
 *    copies).  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns as soon as it is enqueued.
 *  - Return value: SSM_OK (0) or a negative SSM_ERR_* code.  Argument errors
 *    are detected on the host before anything is enqueued; then nothing on the
 *    device has been touched.  No C++ exception crosses the ABI.
 *  - The state slots named by `slot` are updated in place: read when the
 *    sequence resumes (fresh[s] == 0), never read when it is fresh, and always
 *    written with the state after the sequence's last token.  A zero-length
 *    resuming sequence leaves its slot unchanged; a zero-length fresh one
 *    zeroes it.  Slots no sequence names are not touched.
 *  - y must not alias any input or the state.  Inputs may alias each other.
 *  - Preconditions on device-array CONTENTS are not checked on the hot path:
 *    cu_seqlens[0] == 0, non-decreasing, cu_seqlens[n_seqs] == n_tokens; slots
 *    distinct and in [0, n_slots).  Breaking them is undefined behaviour (two
 *    sequences writing one slot race); ssm_scan_check_metadata() checks them.
 *  - The library holds no state; calls on different streams may run
 *    concurrently if they touch disjoint slots and outputs.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_SCAN_ABI_VERSION 2
#define SSM_SCAN_MAX_D_STATE 1024

enum ssm_scan_status {
    SSM_OK = 0,
    SSM_ERR_NULL = -1,        /* a required pointer is NULL                        */
    SSM_ERR_DIMS = -2,        /* a size is <= 0 (or < 0 where 0 is allowed), or
                                 n_heads % n_groups != 0                            */
    SSM_ERR_UNSUPPORTED = -3, /* d_state > SSM_SCAN_MAX_D_STATE or the grid would
                                 exceed the launch limits                           */
    SSM_ERR_ALIGN = -4,       /* a float or int array is not 4-byte aligned         */
    SSM_ERR_LAUNCH = -5,      /* the HIP runtime refused the launch                 */
    SSM_ERR_METADATA = -6,    /* ssm_scan_check_metadata found a violation          */
    SSM_ERR_SCRATCH = -7      /* the call needs more than the static scratch holds  */
};

/* H, P, N, G: heads, head-dim rows per head, state size, B/C groups. */
typedef struct ssm_scan_dims {
    int32_t n_heads;
    int32_t head_dim;
    int32_t d_state;
    int32_t n_groups;
} ssm_scan_dims;

/*
 * Prefill: scan a packed batch of n_seqs sequences, n_tokens tokens in all.
 *   cu_seqlens [n_seqs+1] int32  token offsets; sequence s owns tokens
 *                                 cu_seqlens[s] .. cu_seqlens[s+1]-1
 *   slot       [n_seqs]   int32  state slot of each sequence
 *   fresh      [n_seqs]   uint8  1 = start from the zero state (slot not read)
 *   x          [n_tokens][H][P]  input
 *   dt         [n_tokens][H]     step size (final; no softplus)
 *   A          [H]               one decay rate per head (normally < 0)
 *   B, C       [n_tokens][G][N]  input and output projections
 *   state      [n_slots][H][P][N] read (resume) and written in place
 *   y          [n_tokens][H][P]  output, fully overwritten
 * n_seqs == 0 is a no-op returning SSM_OK.  With n_tokens == 0 the token
 * arrays (x, dt, B, C, y) may be NULL.
 */
int ssm_scan_prefill(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                     const int32_t *cu_seqlens, const int32_t *slot,
                     const uint8_t *fresh, const float *x, const float *dt,
                     const float *A, const float *B, const float *C, float *state,
                     int32_t n_slots, float *y, void *stream);

/*
 * Prefill that may split long sequences over time, for batches too small to
 * fill the GPU (few sequences, long prompts).  Same arguments and meaning as
 * ssm_scan_prefill, plus:
 *   max_seqlen      host-side upper bound on every sequence's length (a longer
 *                   sequence is still scanned correctly, its last segment just
 *                   runs to its end)
 *   n_segments      0 = let the library decide, 1 = never split, k > 1 = cut
 *                   each sequence into about k segments
 *   workspace       device scratch of at least the size that
 *                   ssm_scan_prefill_workspace_size() reports for the same
 *                   arguments; owned by the caller, contents need no
 *                   initialisation and are garbage afterwards.  With NULL or
 *                   too small a workspace the call runs unsplit.
 * A split sequence is cut into segments that run in parallel, in one of two
 * forms (three kernels each):
 *   - d_state <= 128 (a multiple of 4), head_dim a multiple of 16, 16-byte
 *     aligned arrays: the chunked matrix form on the matrix cores.  A state
 *     pass computes every segment's end state but the last (segment 0 from
 *     the true start state, later ones from zero); a second kernel chains
 *     them, carry <- prod(dA over the segment) * carry + end, into the state
 *     carried into each segment; a third scans every segment from its
 *     carried-in state in 16-token chunks, writing final y and, for the last
 *     segment, the slot.  Automatic planning keeps segments of at least 128
 *     tokens (shorter batches run unsplit).
 *   - otherwise: the register scan of every segment (segment 0 from the true
 *     start state, later ones from zero), the same chaining, which also writes
 *     the final state to the slot, and a correction of each later segment's y:
 *     y[t] += prod(dA from the segment start through t) * (C_t . carry).
 *     Automatic planning keeps segments of at least 256 tokens.
 * Real arithmetic equals the sequential recurrence exactly; in floating point
 * only the association changes (the time-split form of the scan that "perf(cuda):
 * keep the Mamba2 scan state in registers ... #90" leaves for later).
 * Three kernels are enqueued on `stream`; no allocation, no synchronization.
 */
int ssm_scan_prefill_ws(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                        int32_t max_seqlen, int32_t n_segments, const int32_t *cu_seqlens,
                        const int32_t *slot, const uint8_t *fresh, const float *x,
                        const float *dt, const float *A, const float *B, const float *C,
                        float *state, int32_t n_slots, float *y, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * ssm_scan_prefill_ws with the library's own scratch in place of the caller's
 * workspace.  Same arguments, meaning and results (bit for bit the same
 * kernels and plan), minus workspace and workspace_bytes.
 *   - The scratch is one static device array of SSM_SCAN_STATIC_SCRATCH_BYTES
 *     on each GPU the library runs on, held until the process ends.  The
 *     first call on a GPU looks up its address there (a runtime query, no
 *     allocation); make that first call outside graph capture.
 *   - A call whose split needs more than SSM_SCAN_STATIC_SCRATCH_BYTES
 *     (ssm_scan_prefill_workspace_size tells) returns SSM_ERR_SCRATCH before
 *     anything is enqueued; ask for fewer segments or use ssm_scan_prefill_ws.
 *     The 1 x 4096-token prefill at H 64, P 64, N 128 (16 segments) needs 33 MB.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (nothing in it needs clearing).  Calls that overlap on
 *     one GPU (on concurrent streams, or from several host threads) race on it
 *     and give wrong results: the caller serialises them.
 * Never calls hipMalloc, hipFree or any allocating library routine.  Errors as
 * for ssm_scan_prefill_ws, plus SSM_ERR_SCRATCH, and SSM_ERR_LAUNCH if the
 * scratch's address cannot be found (ssm_scan_last_hip_error tells why).
 */
#define SSM_SCAN_STATIC_SCRATCH_BYTES ((size_t)48 << 20)
int ssm_scan_prefill_static(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                            int32_t max_seqlen, int32_t n_segments, const int32_t *cu_seqlens,
                            const int32_t *slot, const uint8_t *fresh, const float *x,
                            const float *dt, const float *A, const float *B, const float *C,
                            float *state, int32_t n_slots, float *y, void *stream);

/* Workspace bytes ssm_scan_prefill_ws needs for these sizes (0 if it would not
 * split).  Touches no device.  The same size serves ssm_scan_prefill_opt, which
 * ignores the workspace when its options force a whole-sequence scan. */
int ssm_scan_prefill_workspace_size(const ssm_scan_dims *dims, int32_t n_seqs, int32_t n_tokens,
                                    int32_t max_seqlen, int32_t n_segments, size_t *bytes);

/*
 * Options of ssm_scan_prefill_opt / ssm_scan_decode_opt (a NULL pointer to
 * this struct, or a zeroed one, is the plain scan):
 *   dt_bias      [H] device array or NULL: dt_eff = dt + dt_bias[head]
 *   dt_softplus  1: dt_eff = softplus(dt_eff) = log1p(exp(dt_eff)) for
 *                dt_eff <= 20 and dt_eff itself above -- the rule of ggml's scan
 *                kernels ("The llama journey", Day 11 and Day 14) and of
 *                Foundry's decay gate ("ssm_gated_delta.cu", fc_ssm_decay_gate)
 *   a_per_state  1: A is [H][N] and element n of a head decays by
 *                exp(dt_eff * A[head][n]) -- the Mamba1 form of ggml's CPU
 *                table (Day 12) and kernel (Day 11); 0: A is [H]
 *   snapshots    [n_tokens][H][P][N] device array or NULL: receives the state
 *                after every token, in packed token order, for rolling back a
 *                partly accepted speculative draft ("ssm_gated_delta.cu", the
 *                snaps argument of the scan kernels)
 * dt_eff replaces dt everywhere (decay and input scaling).  a_per_state or
 * snapshots make ssm_scan_prefill_opt scan whole sequences (no time split).
 * Pointers must be 4-byte aligned (16 for the vector path), like the others.
 */
typedef struct ssm_scan_options {
    const float *dt_bias;
    int32_t dt_softplus;
    int32_t a_per_state;
    float *snapshots;
} ssm_scan_options;

/* ssm_scan_prefill_ws with options (opts may be NULL). */
int ssm_scan_prefill_opt(const ssm_scan_dims *dims, const ssm_scan_options *opts, int32_t n_seqs,
                         int32_t n_tokens, int32_t max_seqlen, int32_t n_segments,
                         const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                         const float *x, const float *dt, const float *A, const float *B,
                         const float *C, float *state, int32_t n_slots, float *y, void *workspace,
                         size_t workspace_bytes, void *stream);

/* ssm_scan_decode with options (opts may be NULL; snapshots then has one
 * entry per sequence, equal to the state written to its slot). */
int ssm_scan_decode_opt(const ssm_scan_dims *dims, const ssm_scan_options *opts, int32_t n_seqs,
                        const int32_t *slot, const uint8_t *fresh, const float *x,
                        const float *dt, const float *A, const float *B, const float *C,
                        float *state, int32_t n_slots, float *y, void *stream);

/*
 * Decode: one token for each of n_seqs sequences (token s belongs to sequence
 * s).  Identical in meaning to ssm_scan_prefill with every length equal to 1;
 * it exists so a decode step needs no cu_seqlens.
 *   x [n_seqs][H][P], dt [n_seqs][H], B and C [n_seqs][G][N], y [n_seqs][H][P];
 *   slot, fresh, A, state as for prefill.
 */
int ssm_scan_decode(const ssm_scan_dims *dims, int32_t n_seqs, const int32_t *slot,
                    const uint8_t *fresh, const float *x, const float *dt,
                    const float *A, const float *B, const float *C, float *state,
                    int32_t n_slots, float *y, void *stream);

/* Static text for a status code (never NULL). */
const char *ssm_scan_strerror(int code);

/* SSM_SCAN_ABI_VERSION of the built library. */
int ssm_scan_version(void);

/*
 * The hipError_t of the last HIP runtime call that failed inside this library
 * on the calling thread (0 if none has), and the runtime's text for it.  Lets
 * a caller that got SSM_ERR_LAUNCH see why.  The text pointer is static.
 */
int ssm_scan_last_hip_error(void);
const char *ssm_scan_last_hip_error_string(void);

/*
 * Debug / test helper on the DEVICE metadata a prefill or decode call would
 * take: copies cu_seqlens (n_seqs + 1 entries; NULL to check the slots of a
 * decode batch only) and slot (n_seqs entries) to the host on `stream`, waits
 * for the stream, then checks what ssm_scan_check_metadata_host checks.  It
 * synchronizes, so it is for tests and debugging, never for the hot path
 * (the scans themselves do not check array contents).  Returns SSM_OK,
 * SSM_ERR_NULL (slot NULL with n_seqs > 0), SSM_ERR_DIMS (a negative count),
 * SSM_ERR_METADATA, or SSM_ERR_LAUNCH if a copy failed (then
 * ssm_scan_last_hip_error() tells why).  n_seqs == 0 returns SSM_OK at once.
 */
int ssm_scan_check_metadata(int32_t n_seqs, int32_t n_tokens, const int32_t *cu_seqlens,
                            const int32_t *slot, int32_t n_slots, void *stream);

/*
 * The same checks on HOST arrays: cu_seqlens[0] == 0, non-decreasing,
 * cu_seqlens[n_seqs] == n_tokens, every slot in [0, n_slots) and no slot
 * named twice.  Returns SSM_OK, SSM_ERR_NULL, SSM_ERR_DIMS or
 * SSM_ERR_METADATA.  cu_seqlens may be NULL to check the slots of a decode
 * batch only.  Touches no device.
 */
int ssm_scan_check_metadata_host(int32_t n_seqs, int32_t n_tokens, const int32_t *cu_seqlens,
                                 const int32_t *slot, int32_t n_slots);

/* The launch shape the library picks for a call (for logs and tests). */
typedef struct ssm_scan_geometry {
    int32_t lanes_per_row;     /* R: adjacent wavefront lanes that share one row   */
    int32_t elems_per_lane;    /* E: state elements each lane keeps in registers  */
    int32_t rows_per_block;    /* RB: head-dim rows one workgroup covers           */
    int32_t chunk_tokens;      /* CT: tokens staged in LDS per chunk               */
    int32_t threads_per_block;
    int32_t lds_bytes;         /* dynamic LDS per workgroup                         */
    int64_t blocks;            /* workgroups in the grid                            */
    int32_t vector_path;       /* 1 = float4 loads and stores; 0 = scalar + LDS tile */
    int32_t segments;          /* time segments per sequence (1 = not split)        */
    int32_t segment_tokens;    /* tokens per segment when split                      */
} ssm_scan_geometry;

/*
 * Fill *out with the geometry a prefill (decode == 0) or decode (decode != 0)
 * call with these sizes would launch.  `aligned` says whether the caller's
 * pointers are all 16-byte aligned.  Touches no device.
 */
int ssm_scan_query_geometry(const ssm_scan_dims *dims, int32_t n_seqs, int32_t decode,
                            int32_t aligned, ssm_scan_geometry *out);

/* The geometry of the segment-scan kernel ssm_scan_prefill_ws would launch
 * (segments = 1: it would run unsplit).  Touches no device. */
int ssm_scan_query_prefill_plan(const ssm_scan_dims *dims, int32_t n_seqs, int32_t max_seqlen,
                                int32_t n_segments, int32_t aligned, ssm_scan_geometry *out);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
