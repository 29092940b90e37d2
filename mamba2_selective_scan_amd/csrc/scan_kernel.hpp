// scan_kernel.hpp -- the gfx950 kernel of the Mamba2 selective-state scan.
//
// One kernel template serves prefill and decode.  A workgroup of 256 lanes
// (four 64-wide wavefronts) owns one (sequence, head, run of RB head-dim rows)
// and walks that sequence's tokens in order.  Per token and row it computes
//     dA = exp(dt*A[h]);  st[n] = st[n]*dA + B[n]*(x*dt);  y = sum_n st[n]*C[n]
// -- the recurrence of ggml's Mamba2 group kernel ("The llama journey", Day 14)
// with the state kept in registers and a row split over adjacent lanes, as in
// "perf(cuda): keep the Mamba2 scan state in registers, stage tokens by chunk
// #90" (What changes).  Where this layout departs from that page's CUDA one:
//
//  * Register layout.  A row of N state elements is split over R adjacent
//    lanes of one wavefront.  Lane r owns the 4-element groups r, r+R, r+2R,
//    ... (J groups, E = 4J elements).  Within a 16-lane row of the wavefront,
//    consecutive lanes therefore touch consecutive 16-byte pieces of memory,
//    so (a) LDS reads of B and C are 128-bit and conflict-free with no padding,
//    and (b) with N % 4 == 0 the state moves between HBM and registers with
//    plain float4 loads that already cover whole cache lines: every wavefront
//    instruction reads 64/R complete R*16-byte runs.  The page's contiguous
//    32-element slices needed a padded LDS layout and an LDS state tile to
//    get the same two properties.  When N or P is not a multiple of 4 (rows
//    are then not 16-byte aligned) the state goes through a coalesced LDS tile
//    instead: one linear dword sweep of the workgroup's contiguous rows.
//  * y is a butterfly over the R lanes of the row with DPP row permutations
//    (quad_perm, row_half_mirror, row_mirror; a lane shuffle only past 16
//    lanes).  Every lane of the row ends with the same sum, so no barrier and
//    no atomic is needed per token.
//  * Prefill: B, C, x and dt of CT tokens are staged in LDS per chunk, double-buffered:
//    the next chunk's global loads are issued into registers before the
//    current chunk is computed and written to the other buffer after it, so
//    there is one barrier per chunk.  dA = exp(dt*A) is computed once per
//    token at staging time, not per lane.  y of the chunk is collected in an
//    LDS tile (each lane keeps the y of every R-th token in a register and
//    stores it once per group of tokens) and written out coalesced during the
//    next chunk.
//  * Decode (one token per sequence) reads the lane's B/C groups, x and dt
//    straight into registers: no LDS, no barrier.
//  * The grid is one-dimensional.  Workgroup ids are remapped so that the
//    blocks the hardware sends to one XCD (id % 8) are consecutive in
//    (sequence, head, row-block) order: heads of one B/C group share an L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "buffer_io.hpp"

namespace ssm {

using f4 = float __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;

struct ScanArgs {
    const int32_t *cu_seqlens;   // [n_seqs+1]; unused by decode
    const int32_t *slot;         // [n_seqs]
    const uint8_t *fresh;        // [n_seqs]
    const float *x;              // [T][H][P]
    const float *dt;             // [T][H]
    const float *A;              // [H]
    const float *B;              // [T][G][N]
    const float *C;              // [T][G][N]
    float *state;                // [n_slots][H][P][N]
    float *y;                    // [T][H][P]
    int32_t H, P, N, G;
    int32_t heads_per_group;
    int32_t n_row_blocks;        // ceil(P / RB)
    int32_t n_blocks;            // n_seqs * n_segs * H * n_row_blocks
    // Time-parallel prefill (n_segs > 1): each sequence is cut into segments
    // of seg_len tokens (the last one runs to the sequence end).
    int32_t n_segs;              // segments per sequence in the grid (1 = none)
    int32_t seg_len;
    float *ws_state;             // [n_seqs][n_segs][H][P][N] segment end / carried-in states
    float *ws_dtot;              // [n_seqs][n_segs][H] product of dA over each segment
    float *ws_dcum;              // [T][H] product of dA from the segment start through t
    // Options.  dt_eff = dt + dt_bias[h] (if given), then softplus (identity
    // above 20) if dt_softplus; with OPT_A_PER_STATE A is [H][N]; with
    // OPT_SNAPSHOTS the state after every token goes to snapshots.
    const float *dt_bias;        // [H] or null
    int32_t dt_softplus;
    float *snapshots;            // [T][H][P][N]
};

// Compile-time option bits of a prefill/decode kernel instance.
constexpr int OPT_A_PER_STATE = 1;
constexpr int OPT_SNAPSHOTS = 2;

// dt after the optional bias and softplus: log1p(exp(v)) up to 20, v above.
__device__ __forceinline__ float dt_transform(float v, float bias, int softplus) {
    v += bias;
    if (softplus && v <= 20.0f) v = log1pf(expf(v));
    return v;
}

enum class Mode { kPrefill, kSegScan, kDecode, kCorrect };

// Compile-time shape of one kernel instance.
template <int R_, int J_, int CT_>
struct Shape {
    static constexpr int R = R_;                    // lanes per row
    static constexpr int J = J_;                    // float4 groups per lane
    static constexpr int E = 4 * J;                 // state elements per lane
    static constexpr int CT = CT_;                  // tokens per staged chunk
    static constexpr int NP = 4 * R * J;            // staged (zero-padded) state width
    static constexpr int ROWS_PER_WAVE = 64 / R;
    static constexpr int RB = kWaves * ROWS_PER_WAVE;   // rows per workgroup
    static constexpr int NPT = NP + 4;              // LDS state-tile row stride
    // One staging buffer, in floats: B[CT][NP] C[CT][NP] x[CT][RB] y[CT][YR] dt[CT] dA[CT]
    static constexpr int OFF_B = 0;
    static constexpr int OFF_C = OFF_B + CT * NP;
    static constexpr int OFF_X = OFF_C + CT * NP;
    // y tile rows padded: lane r of a row stores token r's y at row r, so with
    // a row stride of RB lanes r and r + 64/RB hit one bank.  Measured on gfx950
    // (plain LDS probes): a 32-bit store goes 32 lanes at a time over 32 banks,
    // and with R = 16 (16 tokens x 2 rows per half) it is conflict-free for a
    // row stride of 2 mod 4 floats (4 mod 8 is 2-way, 0 mod 8 worse), so those
    // rows take 18 floats and the flush reads them as float pairs (8-byte
    // aligned); the other widths keep 16-byte aligned rows for a float4 flush.
    static constexpr int YR = R == 4 ? 80 : R == 8 ? 40 : R == 16 ? 18 : 12;
    static constexpr int YV = YR % 4 == 0 ? 4 : 2;   // floats per flush read
    static constexpr int OFF_Y = OFF_X + CT * RB;
    static constexpr int OFF_DT = OFF_Y + CT * YR;
    static constexpr int OFF_DA = OFF_DT + CT;
    // the decay is deferred over sub-chunks of SUB tokens (one 16-lane DPP row
    // of prefix products each), whatever the staging chunk, so a chunk of 32
    // and two of 16 give the same bits
    static constexpr int SUB = CT < 16 ? CT : 16;
    static constexpr int NSUB = CT / SUB;
    static constexpr int OFF_LAZY = OFF_DA + CT;    // [NSUB] 1: the sub-chunk runs with the decay deferred
    static constexpr int BUF = ((OFF_LAZY + NSUB) + 3) / 4 * 4;
    static constexpr int TILE = RB * NPT;           // state tile (scalar path), floats
    // register prefetch units per thread
    static constexpr int U_BC = (CT * NP / 4 + kThreads - 1) / kThreads;    // float4 of B (and of C)
    static constexpr int U_X = (CT * RB / 4 + kThreads - 1) / kThreads;     // float4 of x
    static_assert(R == 4 || R == 8 || R == 16 || R == 32 || R == 64, "R must be a power of two in [4, 64]");
    static_assert(CT <= 64, "one lane of wave 0 stages each token's dt");
    static_assert(RB % 4 == 0, "rows per block must be a multiple of 4");

    static constexpr int lds_floats(Mode mode, bool vec) {
        const int staging = mode == Mode::kDecode ? 0 : 2 * BUF;   // decode reads from global
        return (!vec && TILE > staging) ? TILE : staging;
    }
};

// DPP lane permutations within a 16-lane row.  `old` = 0 is the identity of
// the add that consumes them, which lets the backend fuse each into v_add_f32_dpp.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;   // lane l <- lane 7-l within 8
constexpr int kMirror = 0x140;       // lane l <- lane 15-l within 16

// Sum over the R adjacent lanes that hold one row.  Every step adds a value
// and its partner's (commutative), so all R lanes end with identical bits.
template <int R>
__device__ __forceinline__ float row_allreduce(float v) {
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    if constexpr (R >= 8) v += dpp<kHalfMirror>(v);
    if constexpr (R >= 16) v += dpp<kMirror>(v);
    if constexpr (R >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (R >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Reduce-scatter of KY per-token partials over KY adjacent lanes (KY = 4, 8
// or 16, inside one DPP row): lane l ends with the sum over the KY lanes of
// partial l % KY.  Each stage pairs every lane with one whose index differs in
// the stage's bit (row_mirror, row_half_mirror, quad xor 2, quad xor 1): the
// lane keeps the half of its values whose index has the lane's bit and adds
// the partner's copy of that half.  KY sums cost (KY/2 + KY/4 + ... + 1) DPP
// adds and twice as many selects, against KY full butterflies of log2(KY)
// dependent steps.
template <int CTRL, int BIT, int NV>
__device__ __forceinline__ void scatter_stage(const float (&in)[NV], float (&out)[NV / 2]) {
    const bool up = (threadIdx.x & BIT) != 0;
#pragma unroll
    for (int j = 0; j < NV / 2; ++j) {
        const float keep = up ? in[j + NV / 2] : in[j];
        const float send = up ? in[j] : in[j + NV / 2];
        out[j] = keep + dpp<CTRL>(send);
    }
}
template <int KY>
__device__ __forceinline__ float row_reduce_scatter(const float (&p)[KY]) {
    static_assert(KY == 4 || KY == 8 || KY == 16, "KY lanes inside one DPP row");
    float q8[8], q4[4], q2[2], q1[1];
    if constexpr (KY == 16) {
        scatter_stage<kMirror, 8, 16>(p, q8);
        scatter_stage<kHalfMirror, 4, 8>(q8, q4);
    } else if constexpr (KY == 8) {
        scatter_stage<kHalfMirror, 4, 8>(p, q4);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) q4[j] = p[j];
    }
    scatter_stage<kQuadXor2, 2, 4>(q4, q2);
    scatter_stage<kQuadXor1, 1, 2>(q2, q1);
    return q1[0];
}

// Inclusive running product over the 16 lanes of each DPP row (lanes past a
// row's start multiply by 1).  Used on one token's dA per lane.
template <int CTRL>
__device__ __forceinline__ float dpp_or_one(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(v), CTRL,
                                                      0xF, 0xF, false));
}
__device__ __forceinline__ float row_prefix_product(float v) {
    v *= dpp_or_one<0x111>(v);     // row_shr:1
    v *= dpp_or_one<0x112>(v);     // row_shr:2
    v *= dpp_or_one<0x114>(v);     // row_shr:4
    v *= dpp_or_one<0x118>(v);     // row_shr:8
    return v;
}

// Deferred decay.  Within a sub-chunk of at most 16 tokens (Shape::SUB) the
// row is kept as h / sigma_t, with sigma_t the product of dA from the
// sub-chunk start through token t; then
//     h / sigma_t = h / sigma_{t-1} + b * (x * dt / sigma_t)
// is one fused multiply-add per element instead of a multiply and an FMA, y is
// sigma_t times the row's dot with C, and the sub-chunk ends by multiplying
// the row by its sigma.  A sub-chunk whose sigma would fall below this floor
// (so that 1/sigma could overflow the stored row) runs the direct update
// instead.  Sub-chunks start every 16 tokens of a sequence (every chunk for
// chunks of fewer tokens), so the rounding does not depend on the staging
// chunk.
constexpr float kLazyFloor = 0x1p-40f;

// Load 4 consecutive floats, the ones at index >= n_valid read as 0.
template <bool VEC>
__device__ __forceinline__ f4 load4(const float *p, int n_valid) {
    if constexpr (VEC) {
        return n_valid > 0 ? *reinterpret_cast<const f4 *>(p) : f4{0.f, 0.f, 0.f, 0.f};
    } else {
        f4 v;
        v.x = n_valid > 0 ? p[0] : 0.f;
        v.y = n_valid > 1 ? p[1] : 0.f;
        v.z = n_valid > 2 ? p[2] : 0.f;
        v.w = n_valid > 3 ? p[3] : 0.f;
        return v;
    }
}

__device__ __forceinline__ int clamp4(int v) { return v < 0 ? 0 : (v > 4 ? 4 : v); }

// One state element: h <- h*dA + b*x_dt, with the rounding spelled out (one
// product rounded, then a fused multiply-add) so every caller gets the same bits.
__device__ __forceinline__ float step(float h, float dA, float b, float x_dt) {
    return __builtin_fmaf(b, x_dt, h * dA);
}

// One token of the recurrence for the lane's E = 4J state elements, given the
// lane's J 4-groups of B and C for the token.  Returns the lane's partial y.
// Prefill and decode both go through here, so their arithmetic is identical.
template <int J>
__device__ __forceinline__ float update_token(float (&h)[4 * J], const f4 (&b)[J], const f4 (&c)[J],
                                              float dA, float x_dt) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float *hj = h + 4 * j;
        hj[0] = step(hj[0], dA, b[j].x, x_dt);
        hj[1] = step(hj[1], dA, b[j].y, x_dt);
        hj[2] = step(hj[2], dA, b[j].z, x_dt);
        hj[3] = step(hj[3], dA, b[j].w, x_dt);
        acc0 = __builtin_fmaf(hj[0], c[j].x, acc0);
        acc1 = __builtin_fmaf(hj[1], c[j].y, acc1);
        acc0 = __builtin_fmaf(hj[2], c[j].z, acc0);
        acc1 = __builtin_fmaf(hj[3], c[j].w, acc1);
    }
    return acc0 + acc1;
}

// The same with a decay per state element (A per (head, n)): dA[e] for the
// lane's E elements.
template <int J>
__device__ __forceinline__ float update_token_pe(float (&h)[4 * J], const f4 (&b)[J], const f4 (&c)[J],
                                                 const float (&dA)[4 * J], float x_dt) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float *hj = h + 4 * j;
        const float *dj = dA + 4 * j;
        hj[0] = step(hj[0], dj[0], b[j].x, x_dt);
        hj[1] = step(hj[1], dj[1], b[j].y, x_dt);
        hj[2] = step(hj[2], dj[2], b[j].z, x_dt);
        hj[3] = step(hj[3], dj[3], b[j].w, x_dt);
        acc0 = __builtin_fmaf(hj[0], c[j].x, acc0);
        acc1 = __builtin_fmaf(hj[1], c[j].y, acc1);
        acc0 = __builtin_fmaf(hj[2], c[j].z, acc0);
        acc1 = __builtin_fmaf(hj[3], c[j].w, acc1);
    }
    return acc0 + acc1;
}

// One token with the decay deferred: h <- h + b * xs (xs = x*dt/sigma);
// returns the lane's partial dot of the stored row with C, one fused chain
// over the lane's elements in order.  (Two chains and an add, as the direct
// update takes them, cost the one-pass prefill 3.5% more cycles at one
// wavefront per SIMD: the extra add per token outweighs the shorter chain.)
template <int J>
__device__ __forceinline__ float update_token_lazy(float (&h)[4 * J], const f4 (&b)[J],
                                                   const f4 (&c)[J], float xs) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float *hj = h + 4 * j;
        hj[0] = __builtin_fmaf(b[j].x, xs, hj[0]);
        hj[1] = __builtin_fmaf(b[j].y, xs, hj[1]);
        hj[2] = __builtin_fmaf(b[j].z, xs, hj[2]);
        hj[3] = __builtin_fmaf(b[j].w, xs, hj[3]);
        acc = __builtin_fmaf(hj[0], c[j].x, acc);
        acc = __builtin_fmaf(hj[1], c[j].y, acc);
        acc = __builtin_fmaf(hj[2], c[j].z, acc);
        acc = __builtin_fmaf(hj[3], c[j].w, acc);
    }
    return acc;
}

// The lane's J 4-groups of one token's B (or C) row in LDS; p points at the
// lane's first group, groups are 4*R floats apart.
template <int R, int J>
__device__ __forceinline__ void lds_groups(f4 (&v)[J], const float *p) {
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = *reinterpret_cast<const f4 *>(p + 4 * R * j);
}

// The tokens [t_begin, t_end) that time segment k of sequence s covers, and
// how many segments the sequence really has.  With n_segs == 1 the segment is
// the whole sequence.
struct SegRange {
    int t_begin, t_end, n_real;
};
__device__ __forceinline__ SegRange segment_range(const ScanArgs &a, int s, int k) {
    const int c0 = a.cu_seqlens[s], c1 = a.cu_seqlens[s + 1];
    if (a.n_segs == 1) return SegRange{c0, c1, 1};
    const int len = c1 - c0;
    int n_real = (len + a.seg_len - 1) / a.seg_len;
    n_real = n_real < 1 ? 1 : (n_real > a.n_segs ? a.n_segs : n_real);
    const int tb = c0 + k * a.seg_len;
    return SegRange{tb, k == n_real - 1 ? c1 : tb + a.seg_len, n_real};
}

// MODE kPrefill: scan whole sequences and write y and the end state (slot).
// MODE kSegScan: scan one time segment of a sequence cut into n_segs pieces
//   (segment 0 from the true start state, later ones from zero) and write y;
//   the end state goes to ws_state (to the slot if the sequence was too short
//   to be cut), with the segment's running and total decay products.
// MODE kDecode: one token per sequence, B/C/x/dt read straight into registers.
// MODE kCorrect: for a time segment k >= 1, add the carried-in state's
//   contribution dcum[t] * (C_t . carry) to the y the segment scan wrote.
template <class S, bool VEC, Mode MODE, int OPT = 0>
__global__ void __launch_bounds__(kThreads) scan_kernel(ScanArgs a) {
    extern __shared__ float4 lds_raw[];
    float *const lds = reinterpret_cast<float *>(lds_raw);

    constexpr int R = S::R, J = S::J, E = S::E, CT = S::CT, NP = S::NP, RB = S::RB;
    constexpr bool DECODE = MODE == Mode::kDecode;
    constexpr bool CORRECT = MODE == Mode::kCorrect;
    constexpr bool SEGMENTED = MODE == Mode::kSegScan || CORRECT;   // grid has a segment axis
    constexpr bool A_PER_STATE = (OPT & OPT_A_PER_STATE) != 0;
    constexpr bool SNAPSHOTS = (OPT & OPT_SNAPSHOTS) != 0;
    // the deferred-decay update (see kLazyFloor) for plain prefill and segment scans
    constexpr bool LAZY = (MODE == Mode::kPrefill || MODE == Mode::kSegScan) && OPT == 0;
    static_assert(OPT == 0 || MODE == Mode::kPrefill || MODE == Mode::kDecode,
                  "options are built for whole-sequence prefill and decode only");

    // ---- workgroup -> (sequence, segment, head, row block).  XCD-contiguous
    // order (consecutive ids dealt round-robin over the XCDs take consecutive
    // runs of the grid, so the heads of a B/C group share an L2) -- except a
    // whole-sequence prefill of several sequences, which takes the plain order:
    // there a sequence's workgroups are spread over every XCD, so one long
    // sequence of a ragged batch does not pile onto a few CUs while the others
    // idle (measured on the mixed batch, 8 sequences of 1..150 tokens at H 16,
    // P 96, N 100: 33.7 us XCD-contiguous, 25.2 us plain; a single 1 x 4096
    // sequence keeps the L2 sharing, 455 against 462 us).
    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    const bool plain_order = MODE == Mode::kPrefill && nb > a.n_row_blocks * a.H;
    const int L = plain_order ? bid
                : (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int rb = L % a.n_row_blocks;
    const int hd = (L / a.n_row_blocks) % a.H;
    const int seg = SEGMENTED ? (L / (a.n_row_blocks * a.H)) % a.n_segs : 0;
    const int s = L / (a.n_row_blocks * a.H * (SEGMENTED ? a.n_segs : 1));

    const int H = a.H, P = a.P, N = a.N, G = a.G;
    const int g = hd / a.heads_per_group;
    int t_begin, t_end, n_real = 1;
    if constexpr (DECODE) {
        t_begin = s;
        t_end = s + 1;
    } else if constexpr (!SEGMENTED) {
        t_begin = a.cu_seqlens[s];
        t_end = a.cu_seqlens[s + 1];
    } else {
        const SegRange sr = segment_range(a, s, seg);
        t_begin = sr.t_begin;
        t_end = sr.t_end;
        n_real = sr.n_real;
    }
    if (seg >= n_real) return;                       // the sequence is shorter
    if (CORRECT && seg == 0) return;                 // segment 0 started from the true state
    const int n_tok = t_end - t_begin;
    const bool split = SEGMENTED && n_real > 1;
    // Only the first segment of a sequence sees the slot; later ones start at 0.
    const bool fresh = CORRECT ? false : (seg > 0 || a.fresh[s] != 0);
    if (!CORRECT && !split && !fresh && n_tok <= 0) return;   // empty resume: slot unchanged

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = (tid >> 6) * S::ROWS_PER_WAVE + lane / R;   // row within the block
    const int r = lane % R;                                    // lane within the row
    const int p0 = rb * RB;
    const int rows_valid = min(RB, P - p0);
    const bool row_ok = i < rows_valid;
    const int64_t hpn = int64_t(H) * P * N;
    // rows p0.. of this head in the slot, and in this segment's workspace entry
    float *const st_block = a.state + ((int64_t(a.slot[s]) * H + hd) * P + p0) * int64_t(N);
    float *const ws_block = SEGMENTED
        ? a.ws_state + (int64_t(s) * a.n_segs + seg) * hpn + (int64_t(hd) * P + p0) * N
        : nullptr;
    // where the state comes from: the slot; for a correction, the state carried
    // into this segment (the combine pass left it in the previous entry)
    float *const src_block = CORRECT ? ws_block - hpn : st_block;
    const float A_h = A_PER_STATE ? 0.f : a.A[hd];
    const float bias_h = a.dt_bias ? a.dt_bias[hd] : 0.f;
    // A per state element: this lane's E values of A[hd][n] (0 past N)
    float Ae[A_PER_STATE ? E : 1];
    if constexpr (A_PER_STATE) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            const f4 v = load4<false>(a.A + int64_t(hd) * N + n0, clamp4(N - n0));
            Ae[4 * j + 0] = v.x; Ae[4 * j + 1] = v.y; Ae[4 * j + 2] = v.z; Ae[4 * j + 3] = v.w;
        }
    }
    float h[E];
#pragma unroll
    for (int e = 0; e < E; ++e) h[e] = 0.f;
    // the state after token t, to the snapshot buffer
    auto snapshot = [&](int t) __attribute__((always_inline)) {
        float *dst = a.snapshots + (int64_t(t) * H + hd) * P * int64_t(N) + int64_t(p0 + i) * N;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            const int nv = row_ok ? clamp4(N - n0) : 0;
            if constexpr (VEC) {
                if (nv > 0) *reinterpret_cast<f4 *>(dst + n0) = f4{h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
            } else {
                if (nv > 0) dst[n0 + 0] = h[4 * j + 0];
                if (nv > 1) dst[n0 + 1] = h[4 * j + 1];
                if (nv > 2) dst[n0 + 2] = h[4 * j + 2];
                if (nv > 3) dst[n0 + 3] = h[4 * j + 3];
            }
        }
    };

    // ---- state -> registers
    if (!fresh) {
        if constexpr (VEC) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int n0 = 4 * (j * R + r);
                if (row_ok && n0 < N) {
                    const f4 v = __builtin_nontemporal_load(
                        reinterpret_cast<const f4 *>(src_block + int64_t(i) * N + n0));
                    h[4 * j + 0] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
                }
            }
        } else {
            // coalesced LDS tile: one linear sweep over the block's contiguous rows
            const int total = rows_valid * N;
            for (int q = tid; q < total; q += kThreads) {
                const int row = q / N;
                lds[row * S::NPT + (q - row * N)] = src_block[q];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int n0 = 4 * (j * R + r);
                const f4 v = *reinterpret_cast<const f4 *>(lds + i * S::NPT + n0);
                const int nv = row_ok ? clamp4(N - n0) : 0;
                h[4 * j + 0] = nv > 0 ? v.x : 0.f;
                h[4 * j + 1] = nv > 1 ? v.y : 0.f;
                h[4 * j + 2] = nv > 2 ? v.z : 0.f;
                h[4 * j + 3] = nv > 3 ? v.w : 0.f;
            }
            __syncthreads();                        // the tile area is reused below
        }
    }

    if constexpr (DECODE) {
        // One token: read the lane's slices of B and C, its row's x and the
        // head's dt straight into registers; no LDS and no barrier.
        const int64_t bc = (int64_t(s) * G + g) * N;
        f4 bl[J], cl[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            const int nv = clamp4(N - n0);
            bl[j] = load4<VEC>(a.B + bc + n0, nv);
            cl[j] = load4<VEC>(a.C + bc + n0, nv);
        }
        const float dt = dt_transform(a.dt[int64_t(s) * H + hd], bias_h, a.dt_softplus);
        const float x = row_ok ? a.x[(int64_t(s) * H + hd) * P + p0 + i] : 0.f;
        float part;
        if constexpr (A_PER_STATE) {
            float dAe[E];
#pragma unroll
            for (int e = 0; e < E; ++e) dAe[e] = __expf(dt * Ae[e]);
            part = update_token_pe<J>(h, bl, cl, dAe, x * dt);
        } else {
            part = update_token<J>(h, bl, cl, expf(dt * A_h), x * dt);
        }
        const float yv = row_allreduce<R>(part);
        if (r == 0 && row_ok) a.y[(int64_t(s) * H + hd) * P + p0 + i] = yv;
        if constexpr (SNAPSHOTS) snapshot(s);
    } else {
        // All state loads are complete before the chunk pipeline starts, so the
        // token loop never waits on the next chunk's prefetch.
        __builtin_amdgcn_s_waitcnt(0);

        // ---- chunk staging: global -> registers -> LDS.  The x slot carries x
        // (prefill) or the segment scan's y (correction); the dt slot carries dt
        // (prefill) or, for a correction, the running product of dA from the
        // segment start through each token.  Time segments keep that running
        // product in wave 0 (`run`), chunk after chunk: a 16-lane DPP prefix
        // product per chunk (chunks of a segmented launch are <= 16 tokens).
        // Chunks are loaded PF ahead: chunk k lands in register set k % PF and
        // is committed to LDS buffer k & 1 one step before it is computed.  On
        // the vector path the loads go through buffer descriptors that cover
        // the chunk's tokens only (none at all for a chunk past the end): every
        // step issues the same loads with no branch, so the wait before a
        // commit is for that chunk's loads alone, never the newer chunk's.
        constexpr int PF = VEC ? 2 : 1;
        constexpr int kNone = 0x7ffffff0;                   // a byte offset past every descriptor
        struct Stage {
            f4 pb[S::U_BC], pc[S::U_BC], px[S::U_X];
            float pdt;
        };
        Stage stg[PF];
        const float *xsrc = CORRECT ? a.y : a.x;
        // the vector path's fixed byte offsets into a chunk
        int vo_bc[VEC ? S::U_BC : 1], vo_x[VEC ? S::U_X : 1];
        int vo_dt = kNone;
        if constexpr (VEC) {
#pragma unroll
            for (int u = 0; u < S::U_BC; ++u) {
                const int q = u * kThreads + tid;             // unit = (token, 4-group)
                const int tt = q / (NP / 4);
                const int n0 = 4 * (q - tt * (NP / 4));
                vo_bc[u] = q < CT * NP / 4 && n0 < N ? ((tt * G + g) * N + n0) * int(sizeof(float)) : kNone;
            }
#pragma unroll
            for (int u = 0; u < S::U_X; ++u) {
                const int q = u * kThreads + tid;             // unit = (token, 4 rows)
                const int tt = q / (RB / 4);
                const int pi = 4 * (q - tt * (RB / 4));
                vo_x[u] = q < CT * RB / 4 && pi < rows_valid ? ((tt * H + hd) * P + p0 + pi) * int(sizeof(float)) : kNone;
            }
            vo_dt = tid < CT ? (tid * H + hd) * int(sizeof(float)) : kNone;
        }

        auto issue_loads = [&](Stage &sg, int t0, int nt) __attribute__((always_inline)) {
            if constexpr (VEC) {
                const int nb = nt;                          // 0 past the last chunk
                const __amdgpu_buffer_rsrc_t rbd = buffer_of(a.B + int64_t(t0) * G * N, nb * G * N * int(sizeof(float)));
                const __amdgpu_buffer_rsrc_t rcd = buffer_of(a.C + int64_t(t0) * G * N, nb * G * N * int(sizeof(float)));
                const __amdgpu_buffer_rsrc_t rxd = buffer_of(xsrc + int64_t(t0) * H * P, nb * H * P * int(sizeof(float)));
                const __amdgpu_buffer_rsrc_t rdd = buffer_of(a.dt + int64_t(t0) * H, nb * H * int(sizeof(float)));
#pragma unroll
                for (int u = 0; u < S::U_BC; ++u) {
                    if constexpr (!CORRECT) sg.pb[u] = buffer_load<4>(rbd, vo_bc[u], 0);
                    sg.pc[u] = buffer_load<4>(rcd, vo_bc[u], 0);
                }
#pragma unroll
                for (int u = 0; u < S::U_X; ++u) sg.px[u] = buffer_load<4>(rxd, vo_x[u], 0);
                // raw dt: its transform waits until the commit
                sg.pdt = buffer_load<1>(rdd, vo_dt, 0);
            } else {
#pragma unroll
                for (int u = 0; u < S::U_BC; ++u) {
                    const int q = u * kThreads + tid;             // unit = (token, 4-group)
                    const int tt = q / (NP / 4);
                    const int n0 = 4 * (q - tt * (NP / 4));
                    const bool ok = (q < CT * NP / 4) && (tt < nt);
                    const int64_t off = (int64_t(t0 + tt) * G + g) * N + n0;
                    const int nv = ok ? clamp4(N - n0) : 0;
                    if constexpr (!CORRECT) sg.pb[u] = load4<VEC>(a.B + off, nv);
                    sg.pc[u] = load4<VEC>(a.C + off, nv);
                }
#pragma unroll
                for (int u = 0; u < S::U_X; ++u) {
                    const int q = u * kThreads + tid;             // unit = (token, 4 rows)
                    const int tt = q / (RB / 4);
                    const int pi = 4 * (q - tt * (RB / 4));
                    const bool ok = (q < CT * RB / 4) && (tt < nt);
                    const int nv = ok ? clamp4(rows_valid - pi) : 0;
                    sg.px[u] = load4<VEC>(xsrc + (int64_t(t0 + tt) * H + hd) * P + p0 + pi, nv);
                }
                // raw dt: its transform waits until the commit, so nothing here
                // waits for a load to arrive
                sg.pdt = (tid < nt) ? a.dt[int64_t(t0 + tid) * H + hd] : 0.f;
            }
        };

        float run = 1.f;                                    // wave 0: dA product so far
        auto commit = [&](int buf, const Stage &sg, int t0, int nt) __attribute__((always_inline)) {
            float *base = lds + buf * S::BUF;
            // the chunk's dt after bias and softplus (0 past its tokens)
            auto dt_eff = [&] { return (tid < nt) ? dt_transform(sg.pdt, bias_h, a.dt_softplus) : 0.f; };
            f4 *Bs4 = reinterpret_cast<f4 *>(base + S::OFF_B);
            f4 *Cs4 = reinterpret_cast<f4 *>(base + S::OFF_C);
            f4 *Xs4 = reinterpret_cast<f4 *>(base + S::OFF_X);
#pragma unroll
            for (int u = 0; u < S::U_BC; ++u) {
                const int q = u * kThreads + tid;
                if (q < CT * NP / 4) {
                    if constexpr (!CORRECT) Bs4[q] = sg.pb[u];
                    Cs4[q] = sg.pc[u];
                }
            }
#pragma unroll
            for (int u = 0; u < S::U_X; ++u) {
                const int q = u * kThreads + tid;
                if (q < CT * RB / 4) Xs4[q] = sg.px[u];
            }
            if constexpr (SEGMENTED || LAZY) {
                if (tid < 64) {                              // wave 0, all lanes active
                    const float dtv = dt_eff();
                    const float dA = (tid < nt) ? expf(dtv * A_h) : 1.f;
                    // from the start of the token's sub-chunk (its DPP row; for
                    // chunks of at most 16 tokens, the chunk)
                    const float loc = row_prefix_product(dA);
                    const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(loc), S::SUB - 1));
                    if constexpr (SEGMENTED) {
                        const float cum = run * loc;                     // from the segment start
                        if constexpr (CORRECT) {
                            if (tid < CT) {
                                base[S::OFF_DT + tid] = cum;
                                base[S::OFF_DA + tid] = dA;
                            }
                        }
                        // a split sequence's segment scan also leaves the running
                        // product for the matrix-core correction (one row block per head)
                        if (MODE == Mode::kSegScan && split && rb == 0 && tid < nt)
                            a.ws_dcum[int64_t(t0 + tid) * H + hd] = cum;
                        run *= total;
                    }
                    if constexpr (LAZY) {
                        // per sub-chunk; one-token sub-chunks keep the direct
                        // update, so a lone token gives the same bits as decode
                        bool lazy_k[S::NSUB];
#pragma unroll
                        for (int k = 0; k < S::NSUB; ++k) {
                            const float tot = __int_as_float(
                                __builtin_amdgcn_readlane(__float_as_int(loc), S::SUB * k + S::SUB - 1));
                            lazy_k[k] = nt - S::SUB * k > 1 && tot >= kLazyFloor;
                        }
                        bool lazy = lazy_k[0];
#pragma unroll
                        for (int k = 1; k < S::NSUB; ++k) lazy = (tid / S::SUB == k) ? lazy_k[k] : lazy;
                        if (tid < CT) {
                            base[S::OFF_DT + tid] = lazy ? dtv / loc : dtv;
                            base[S::OFF_DA + tid] = lazy ? loc : dA;
                        }
                        // sub-chunk k's flag, written by lane k (not lane k's own
                        // sub-chunk's: lanes 0 .. NSUB-1 all sit in sub-chunk 0)
                        bool flag = lazy_k[0];
#pragma unroll
                        for (int k = 1; k < S::NSUB; ++k) flag = (tid == k) ? lazy_k[k] : flag;
                        if (tid < S::NSUB) base[S::OFF_LAZY + tid] = flag ? 1.f : 0.f;
                    }
                }
            } else {
                if (tid < CT) {
                    const float dtv = dt_eff();
                    base[S::OFF_DT + tid] = dtv;
                    base[S::OFF_DA + tid] = expf(dtv * A_h);
                }
            }
        };

        // Tokens go in groups of KY.  Every lane of a row ends a token with the
        // row's y; lane r keeps the y of the group's token r % KY and stores it
        // once per group, so the per-token cost is one select.  Inside a group
        // the token index is a compile-time constant: LDS offsets fold into the
        // instructions and the keep-select needs no runtime compare.
        constexpr int KY = R < 16 ? R : 16;
        const int rk = r % KY;
        int chunk_t0 = 0;                                   // first token of the chunk in compute
        // The lane's partial of token tt's y (prefill / segment scan): the row
        // sum of these, times y_scale(tt), is y.
        // One token's operands out of LDS: the lane's B and C groups, its row's
        // x and the token's dt and dA (deferred form: dt / sigma and sigma).
        struct TokIn {
            f4 b[J], c[J];
            float x, dt, dA;
        };
        auto token_load = [&](const float *base, int tt) __attribute__((always_inline)) {
            TokIn in;
            lds_groups<R, J>(in.c, base + S::OFF_C + 4 * r + tt * NP);
            lds_groups<R, J>(in.b, base + S::OFF_B + 4 * r + tt * NP);
            in.x = base[S::OFF_X + tt * RB + i];
            in.dt = base[S::OFF_DT + tt];
            in.dA = base[S::OFF_DA + tt];
            return in;
        };
        // The lane's partial of token tt's y (prefill / segment scan) from its
        // operands: the row sum of these, times y_scale(tt), is y.
        auto token_part_in = [&](TokIn &in, int tt, auto lazy_tag) -> float __attribute__((always_inline)) {
            if constexpr (decltype(lazy_tag)::value) {
                return update_token_lazy<J>(h, in.b, in.c, in.x * in.dt);
            } else {
                const float x_dt = in.x * in.dt;
                float part;
                if constexpr (A_PER_STATE) {
                    float dAe[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) dAe[e] = __expf(in.dt * Ae[e]);
                    part = update_token_pe<J>(h, in.b, in.c, dAe, x_dt);
                } else {
                    part = update_token<J>(h, in.b, in.c, in.dA, x_dt);
                }
                if constexpr (SNAPSHOTS) snapshot(chunk_t0 + tt);
                return part;
            }
        };
        // The same operands for token t0 + kk of a group, from pointers formed
        // once per group (kk a compile-time constant: its offsets fold into the
        // LDS instructions instead of a per-token address computation).
        struct GroupPtr {
            const float *c, *x, *s;
        };
        auto group_ptr = [&](const float *base, int t0) __attribute__((always_inline)) {
            return GroupPtr{base + S::OFF_C + 4 * r + t0 * NP, base + S::OFF_X + t0 * RB + i, base + t0};
        };
        auto token_load_g = [&](const GroupPtr &g, int kk) __attribute__((always_inline)) {
            TokIn in;
            lds_groups<R, J>(in.c, g.c + kk * NP);
            lds_groups<R, J>(in.b, g.c + (S::OFF_B - S::OFF_C) + kk * NP);
            in.x = g.x[kk * RB];
            in.dt = g.s[S::OFF_DT + kk];
            in.dA = g.s[S::OFF_DA + kk];
            return in;
        };
        auto token_part = [&](const float *base, int tt, auto lazy_tag) -> float __attribute__((always_inline)) {
            TokIn in = token_load(base, tt);
            return token_part_in(in, tt, lazy_tag);
        };
        auto y_scale = [&](const float *base, int tt, auto lazy_tag) -> float __attribute__((always_inline)) {
            if constexpr (decltype(lazy_tag)::value) return base[S::OFF_DA + tt];
            else return 1.f;
        };
        auto token_y = [&](const float *base, int tt, auto lazy_tag) -> float __attribute__((always_inline)) {
            if constexpr (CORRECT) {
                // y += dcum[t] * (C_t . carry): the carry decayed to token t
                f4 cv[J];
                lds_groups<R, J>(cv, base + S::OFF_C + 4 * r + tt * NP);
                float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    acc0 += h[4 * j + 0] * cv[j].x;
                    acc1 += h[4 * j + 1] * cv[j].y;
                    acc0 += h[4 * j + 2] * cv[j].z;
                    acc1 += h[4 * j + 3] * cv[j].w;
                }
                const float yc = row_allreduce<R>(acc0 + acc1);
                return base[S::OFF_X + tt * RB + i] + base[S::OFF_DT + tt] * yc;
            } else {
                return y_scale(base, tt, lazy_tag) * row_allreduce<R>(token_part(base, tt, lazy_tag));
            }
        };
        // tokens tb .. tb + nt - 1 of the staged chunk
        auto run_tokens = [&](const float *base, float *Ys, int tb, int nt, auto lazy_tag) __attribute__((always_inline)) {
            int t0 = tb;
            nt += tb;
            float y_keep = 0.f;
            if constexpr (!CORRECT && !SNAPSHOTS) {
                // KY tokens at a time: their partials reduce-scattered over the
                // row, so lane r ends with token r % KY's y and stores it.
                // (Snapshot kernels keep the per-token sums: holding KY partials
                // beside the snapshot stores costs them occupancy.)
                // Software-pipelined: token kk + 1's operands are read out of
                // LDS before token kk's arithmetic, so their latency is under it.
                for (; t0 + KY <= nt; t0 += KY) {
                    float part[KY];
                    TokIn in[2];
                    const GroupPtr gp = group_ptr(base, t0);
                    in[0] = token_load_g(gp, 0);
#pragma unroll
                    for (int kk = 0; kk < KY; ++kk) {
                        if (kk + 1 < KY) in[(kk + 1) & 1] = token_load_g(gp, kk + 1);
                        __builtin_amdgcn_sched_barrier(0);
                        part[kk] = token_part_in(in[kk & 1], t0 + kk, lazy_tag);
                    }
                    float yv = row_reduce_scatter<KY>(part);
                    if constexpr (R >= 32) yv += __shfl_xor(yv, 16, 64);
                    if constexpr (R >= 64) yv += __shfl_xor(yv, 32, 64);
                    Ys[(t0 + rk) * S::YR] = y_scale(base, t0 + rk, lazy_tag) * yv;
                }
            } else {
                for (; t0 + KY <= nt; t0 += KY) {
#pragma unroll
                    for (int kk = 0; kk < KY; ++kk) {
                        const float yv = token_y(base, t0 + kk, lazy_tag);
                        y_keep = (rk == kk) ? yv : y_keep;
                    }
                    Ys[(t0 + rk) * S::YR] = y_keep;
                }
            }
            if (t0 < nt) {
                for (int tt = t0; tt < nt; ++tt) {
                    const float yv = token_y(base, tt, lazy_tag);
                    y_keep = (rk == tt - t0) ? yv : y_keep;
                }
                if (rk < nt - t0) Ys[(t0 + rk) * S::YR] = y_keep;
            }
        };
        auto compute = [&](int buf, int nt) __attribute__((always_inline)) {
            const float *base = lds + buf * S::BUF;
            float *Ys = lds + buf * S::BUF + S::OFF_Y + i;
            if constexpr (LAZY) {
#pragma unroll 1
                for (int k = 0; k < S::NSUB; ++k) {
                    const int tb = S::SUB * k;
                    const int n = min(S::SUB, nt - tb);
                    if (n <= 0) break;
                    if (base[S::OFF_LAZY + k] != 0.f) {         // sub-chunk-uniform
                        run_tokens(base, Ys, tb, n, std::true_type{});
                        const float sigma = base[S::OFF_DA + tb + n - 1];
#pragma unroll
                        for (int e = 0; e < E; ++e) h[e] *= sigma;
                    } else {
                        // a direct sub-chunk (one token, or a decay below the floor)
                        run_tokens(base, Ys, tb, n, std::false_type{});
                    }
                }
            } else {
                run_tokens(base, Ys, 0, nt, std::false_type{});
            }
        };

        auto flush_y = [&](int buf, int t0, int nt) __attribute__((always_inline)) {
            const float *Ys = lds + buf * S::BUF + S::OFF_Y;
            if constexpr (VEC) {
                constexpr int YV = S::YV;
                using fy = float __attribute__((ext_vector_type(YV)));
                for (int q = tid; q < nt * (RB / YV); q += kThreads) {
                    const int tt = q / (RB / YV);
                    const int pi = YV * (q - tt * (RB / YV));
                    if (pi < rows_valid)
                        *reinterpret_cast<fy *>(a.y + (int64_t(t0 + tt) * H + hd) * P + p0 + pi) =
                            *reinterpret_cast<const fy *>(Ys + tt * S::YR + pi);
                }
            } else {
                for (int q = tid; q < nt * RB; q += kThreads) {
                    const int tt = q / RB;
                    const int pi = q - tt * RB;
                    if (pi < rows_valid) a.y[(int64_t(t0 + tt) * H + hd) * P + p0 + pi] = Ys[tt * S::YR + pi];
                }
            }
        };

        // ---- token loop, chunk by chunk, double-buffered.  Chunk c's y tile is
        // written out during chunk c+1, after that chunk's prefetch is issued and
        // before its token loop: the stores then drain under the compute, and
        // the registers that carried them are free again by the time they are
        // reused (vector-memory counters on this chip count stores too).
        const int n_chunks = (n_tok + CT - 1) / CT;
        // chunk k's loads (none past the last chunk)
        auto issue_chunk = [&](Stage &sg, int k) __attribute__((always_inline)) {
            const int t0 = t_begin + k * CT;
            issue_loads(sg, k < n_chunks ? t0 : t_begin, k < n_chunks ? min(CT, t_end - t0) : 0);
        };
        // vector-memory instructions of one issue_loads (vector path)
        constexpr int kLoadsPerChunk = (CORRECT ? 1 : 2) * S::U_BC + S::U_X + 1;
        if (n_chunks > 0) {
            // chunk 0's loads all before chunk 1's, so its commit waits for them alone
#pragma unroll
            for (int k = 0; k < PF; ++k) {
                issue_chunk(stg[k], k);
                __builtin_amdgcn_sched_barrier(0);
            }
            commit(0, stg[0], t_begin, min(CT, n_tok));
            if constexpr (PF > 1) {
                // chunk 0 is in LDS on every path through the commit: only
                // chunk 1's loads may still be in flight at the loop head
                constexpr int n = kLoadsPerChunk;
                static_assert(n < 64, "vmcnt field");
                __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
            }
        }
        __syncthreads();
        // chunk c: the loads of chunk c + PF into the register set chunk c
        // left, the previous chunk's y out, chunk c's tokens, then chunk c + 1
        // to LDS
        auto step = [&](int c, auto setc) __attribute__((always_inline)) {
            constexpr int st = decltype(setc)::value;
            const int buf = c & 1;
            const int t0 = t_begin + c * CT;
            const int nt = min(CT, t_end - t0);
            issue_chunk(stg[st], c + PF);
            if (c > 0) flush_y(buf ^ 1, t0 - CT, CT);    // previous chunk, always full
            chunk_t0 = t0;
            compute(buf, nt);
            if (c + 1 < n_chunks) commit(buf ^ 1, stg[(st + 1) % PF], t0 + CT, min(CT, t_end - t0 - CT));
            __syncthreads();
        };
        // (a pair cut short leaves the loop at once, so the loop head's wait
        // counts only the loads of a whole pair)
        for (int c = 0; c < n_chunks; c += PF) {
            step(c, std::integral_constant<int, 0>{});
            if constexpr (PF > 1) {
                if (c + 1 >= n_chunks) break;
                step(c + 1, std::integral_constant<int, 1>{});
            }
        }
        if (n_chunks > 0) {
            const int c = n_chunks - 1;
            flush_y(c & 1, t_begin + c * CT, n_tok - c * CT);
        }
        // a split sequence's segment records its total decay once per head
        if constexpr (MODE == Mode::kSegScan)
            if (split && rb == 0 && tid == 0) a.ws_dtot[(int64_t(s) * a.n_segs + seg) * H + hd] = run;
    }

    if constexpr (CORRECT) return;                   // the state is not changed here

    // ---- registers -> state slot (or this segment's workspace entry)
    float *const dst_block = (SEGMENTED && split) ? ws_block : st_block;
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            if (row_ok && n0 < N) {
                const f4 v = {h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
                __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(dst_block + int64_t(i) * N + n0));
            }
        }
    } else {
        __syncthreads();                             // the last y tile may overlap the state tile
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            *reinterpret_cast<f4 *>(lds + i * S::NPT + n0) =
                f4{h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
        }
        __syncthreads();
        const int total = rows_valid * N;
        for (int q = tid; q < total; q += kThreads) {
            const int row = q / N;
            dst_block[q] = lds[row * S::NPT + (q - row * N)];
        }
    }
}

// Combine pass of the time-parallel prefill, one thread per 4 (VEC) or 1 state
// elements of one (sequence, head, row): walk the sequence's segments in order,
//     carry <- dtot[k] * carry + local_end[k]
// starting from segment 0's (true) end state, and leave the state carried INTO
// segment k in entry k-1.  With into_slot, every segment's end state is in the
// workspace and the final carry goes to the sequence's slot (the register
// segment scan, followed by the corrections).  Without it the last segment's
// end state is not there yet: the walk stops at the carry into the last
// segment, which then runs from it (the matrix-core scan pass).
template <bool VEC>
__global__ void __launch_bounds__(kThreads) combine_kernel(ScanArgs a, int64_t n_units,
                                                           int into_slot) {
    const int64_t u = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (u >= n_units) return;
    constexpr int W = VEC ? 4 : 1;
    const int64_t per_seq = int64_t(a.H) * a.P * a.N / W;
    const int s = int(u / per_seq);
    const int64_t e = (u - int64_t(s) * per_seq) * W;          // element within [H][P][N]
    const int hd = int(e / (int64_t(a.P) * a.N));
    const SegRange sr = segment_range(a, s, 0);
    if (sr.n_real == 1) return;                                // not split: the scan wrote the slot
    const int64_t hpn = int64_t(a.H) * a.P * a.N;
    float *w = a.ws_state + int64_t(s) * a.n_segs * hpn + e;
    float *dst = a.state + int64_t(a.slot[s]) * hpn + e;
    const int k_end = into_slot ? sr.n_real : sr.n_real - 1;   // local end states folded in
    if constexpr (VEC) {
        f4 carry = *reinterpret_cast<const f4 *>(w);
        for (int k = 1; k < k_end; ++k) {
            if (k > 1) *reinterpret_cast<f4 *>(w + (k - 1) * hpn) = carry;
            const float d = a.ws_dtot[(int64_t(s) * a.n_segs + k) * a.H + hd];
            const f4 loc = *reinterpret_cast<const f4 *>(w + k * hpn);
            carry = d * carry + loc;
        }
        if (into_slot)
            __builtin_nontemporal_store(carry, reinterpret_cast<f4 *>(dst));
        else if (k_end > 1)
            *reinterpret_cast<f4 *>(w + (k_end - 1) * hpn) = carry;
    } else {
        float carry = w[0];
        for (int k = 1; k < k_end; ++k) {
            if (k > 1) w[(k - 1) * hpn] = carry;
            const float d = a.ws_dtot[(int64_t(s) * a.n_segs + k) * a.H + hd];
            carry = d * carry + w[k * hpn];
        }
        if (into_slot)
            dst[0] = carry;
        else if (k_end > 1)
            w[(k_end - 1) * hpn] = carry;
    }
}

}  // namespace ssm
