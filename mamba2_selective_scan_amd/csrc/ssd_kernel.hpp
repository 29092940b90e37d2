// ssd_kernel.hpp -- the segment scan of the time-split prefill in chunked
// matrix form, on the matrix cores.
//
// "perf(cuda): keep the Mamba2 scan state in registers, stage tokens by chunk
// #90" (Not in this PR) names the chunked matrix-multiply (SSD) rewrite as the
// next step for long prefills.  Over a chunk of 16 tokens t (inclusive running
// log-decay S_t = sum of dt*A from the chunk start, u_s = dt_s * x_s), with the
// chunk's carried-in state h (rows p, state index n):
//     y[t][p]  = e^{S_t} (C_t . h[p])  +  sum_{s<=t} (C_t . B_s) e^{S_t - S_s} dt_s x_s[p]
//     h'[p][n] = e^{S_15} h[p][n]     +  sum_s B_s[n] e^{S_15 - S_s} dt_s x_s[p]
// which is the recurrence of the scan kernel regrouped: in real arithmetic the
// same numbers, only association changes.  Each of the four products is a
// dense fp32 contraction on v_mfma_f32_16x16x4f32:
//     G^T = B C^T            (16 x 16, over n)       per chunk
//     Y  += C h^T            (16 t x 16 p, over n)   carried-in state
//     Y  += G' X             (16 t x 16 p, over s)   G' = masked, scaled G
//     h^T += B^T (w X)       (n x 16 p, over s)      state update
// Operand layouts (checked on gfx950): A[i][k] is lane i + 16k, B[k][j] is
// lane j + 16k, and accumulator register v of lane l holds D[4(l/16) + v][l%16].
// The state is kept transposed, h^T[n][p], in accumulators: with the
// contraction index of C h^T permuted as n = 16*tile + 4*(lane/16) + step,
// register `step` of a state tile is exactly the B operand the next product
// needs, and likewise G^T's registers are the A operand of G' X.  So no
// accumulator ever goes through LDS to be transposed.  The emulation of this
// scheme with these lane rules reproduced the fp64 oracle to rounding.
//
// Two kernels here serve the time-split prefill.  The state pass
// (ssd_state_kernel) runs every segment but the last of a cut sequence and
// leaves only the segment's end state and total decay (segment 0 from the
// sequence's start state, later ones from zero); the combine pass turns those
// into the state carried into each segment; the scan pass (ssd_scan_kernel)
// then runs every segment from its true carried-in state, so the y it writes
// is final and the last segment's end state is the sequence's.  No y is ever
// read back.  The scan pass runs one workgroup per (sequence, time segment,
// window of 64 TW rows of a B/C group): its four wavefronts own TW 16-row
// tiles each.  B, C and x of a chunk are staged in LDS, double-buffered (rows
// of B, C and x padded, each for the way it is read), the per-token
// scalars of each head are formed once in wave 0, and G^T, the same for the
// four wavefronts, is formed a quarter by each and summed through LDS.  G^T
// only feeds the chunk's own y (never the state), so a chunk's y is finished
// during the next chunk, after the one barrier per chunk that the staging
// needs anyway.
#pragma once

#include "buffer_io.hpp"
#include "scan_kernel.hpp"

namespace ssm {

using f4m = float __attribute__((ext_vector_type(4)));

// LDS layout and staging of the scan pass: a workgroup owns RBW = 64 TW rows
// of the flattened (head, row) space, TW 16-row tiles per wave.
template <int NT, int TW>               // N = 16 NT state elements; TW tiles per wave
struct SsdScanShape {
    static constexpr int N = 16 * NT;
    static constexpr int CT = 16;                   // tokens per chunk
    static constexpr int RBW = 64 * TW;             // rows per workgroup (4 waves x 16 TW)
    static constexpr int MH = 4;                    // heads per workgroup at most (16 TW | P)
    // Padded LDS rows of B and C.  Measured on gfx950 (SQ_LDS_BANK_CONFLICT of
    // plain probes): float reads at rows 4 (l/16) + v, column l%16 are free of
    // conflicts for a row stride of 4 mod 16 floats and 2-way at 8 mod 16; float4
    // reads at row l%16, columns 4 (l/16) .. + 3 cost 4 conflict cycles for 4 mod
    // 16 and none for 8 mod 16.  B is read both ways (the state update's B^T
    // the first, G^T the second), C only the second (C h^T, G^T), so B is
    // staged twice: at N + 4 for the first way and, beside C, at N + 8 for the
    // second.
    static constexpr int LDN = N + 4;               // B rows, read down columns
    static constexpr int LDC = N + 8;               // C rows and B's row-read copy
    // x rows padded by 4 floats: a lane reads row 4 (l/16) + v, column l % 16
    // (+ a wave offset), so with RBW a multiple of the bank count the four
    // l/16 groups would share banks; 4 more floats per row put them 16 banks
    // apart (conflict-free for 32 and for 64 banks)
    static constexpr int XR = RBW + 4;
    static constexpr int OFF_C = 0;
    static constexpr int OFF_BR = OFF_C + CT * LDC;  // B rows at stride LDC (G^T)
    static constexpr int OFF_B = OFF_BR + CT * LDC;
    static constexpr int OFF_X = OFF_B + CT * LDN;  // x[CT][XR]
    static constexpr int OFF_S = OFF_X + CT * XR;   // [MH][CT] S_t
    static constexpr int OFF_DT = OFF_S + MH * CT;  // [MH][CT] dt_t (0 past the segment)
    static constexpr int OFF_ES = OFF_DT + MH * CT; // [MH][CT] e^{S_t} (times sigma when deferred)
    static constexpr int OFF_W = OFF_ES + MH * CT;  // [MH][CT] the update's weights
    static constexpr int OFF_E15 = OFF_W + MH * CT; // [MH] e^{S_15} (exact chunks), else 1
    static constexpr int OFF_PRE = OFF_E15 + MH;    // [MH] factor the state takes before the chunk
    static constexpr int OFF_MODE = OFF_PRE + MH;   // [MH] 1: deferred-decay chunk, 0: exact chunk
    static constexpr int BUF = (OFF_MODE + MH + 3) / 4 * 4;
    static constexpr int U_BC = (CT * N / 4 + kThreads - 1) / kThreads;    // float4 units of B (and of C)
    static constexpr int U_X = CT * RBW / 4 / kThreads;                    // float4 units of x
    static constexpr int PF = TW == 1 ? 2 : 1;      // chunks loaded ahead (register sets)
    static constexpr int OFF_GX = 2 * BUF;          // G^T parts [2 chunk parities][4 waves][64 lanes][4]
    static constexpr int GX = kWaves * 64 * 4;
    static constexpr int OFF_SIG = OFF_GX + 2 * GX; // [MH] sigma at the end
    static constexpr int lds_floats() { return OFF_SIG + MH; }
    static_assert(TW == 1 || TW == 2, "one or two tiles per wave");
    static_assert(CT * RBW / 4 % kThreads == 0, "whole x units per thread");
};

// Sum over lanes 0..l of each 16-lane DPP row (lanes past a row's start add 0).
__device__ __forceinline__ float row_prefix_sum(float v) {
    v += dpp<0x111>(v);     // row_shr:1
    v += dpp<0x112>(v);     // row_shr:2
    v += dpp<0x114>(v);     // row_shr:4
    v += dpp<0x118>(v);     // row_shr:8
    return v;
}

__device__ __forceinline__ f4m mfma16(float a, float b, f4m c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Running sum over the 64 lanes of a wavefront (inclusive): within each
// 16-lane DPP row, then row r adds the running total that the last lane of
// row r - 1 holds by then (rows in order, so each adds every earlier row once).
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
    v = row_prefix_sum(v);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float before = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r - 1));
        if ((lane >> 4) == r) v += before;
    }
    return v;
}

// The state pass: the end state of every segment but a sequence's last, and
// its total decay, with no y.  Over a window of up to kSsdWindow tokens (S_t
// the inclusive running log-decay from the window start)
//     h^T <- e^{S_last} h^T + B^T (w X),   w_t = e^{S_last - S_t} dt_t,
// a plain contraction over the window's tokens on v_mfma_f32_16x16x4f32.
// The workgroup first turns the window's dt into the weights w (an LDS array,
// summed from the window end); after that each wavefront streams its operands
// from global memory straight into registers, with no LDS staging and no
// barrier per chunk.  A wavefront owns two 16-row tiles (rows p0 + 16 t + i)
// and E*16 state columns, so one B load feeds both tiles' products.  To make
// that load one contiguous vector per lane the columns are taken in a
// permuted order: lane l%16 = i reads B[t][n_base + E i .. + E - 1] and uses
// its element e for column tile e, which holds columns n_base + E i + e; the
// accumulators then hold h[p0 + 16 t + l%16][n_base + E (4 (l/16) + v) + e].
// The four wavefronts of a workgroup cover 64 rows x 2 column parts; with
// NS > 1 the grid splits the columns further.  Segment 0 of a resumed
// sequence starts from the slot, the others from zero.  Grid: n_seqs x
// (n_segs - 1) x H x ceil(P / 64) x NS workgroups, XCD-contiguous order.
constexpr int kSsdWindow = 512;          // tokens whose weights one pass of the prologue forms
constexpr float kSsdFastDecay = 40.f;    // a scan chunk decaying less than e^-40 runs deferred
constexpr float kSsdFloor = 0x1p-30f;    // the deferred factor is folded in before passing this
template <int NT, int NS, int IT>        // N = 16 NT; NS column parts; IT tokens per load group
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
ssd_state_kernel(ScanArgs a) {
    // High wave priority until the products start: a workgroup placed on a
    // CU whose SIMDs already run other workgroups' products otherwise waits
    // out most of their loops before its weight prologue gets issue slots
    // (3.75 workgroups per CU at 1 x 4096: -2.5% cycles).
    __builtin_amdgcn_s_setprio(3);
    constexpr int N = 16 * NT;
    constexpr int NW = N / (2 * NS);                 // state columns per wavefront
    constexpr int E = NW / 16;                       // columns per lane = column tiles per wave
    constexpr int KS = IT / 4;                       // MFMA steps per load group
    constexpr int TPT = kSsdWindow / kThreads;       // prologue tokens per thread
    static_assert(NW % 16 == 0 && (E == 1 || E == 2 || E == 4 || E == 8) && IT % 4 == 0 &&
                  kSsdWindow % IT == 0 && (kSsdWindow / IT) % 2 == 0, "state pass shape");
    using fE = typename VecT<E>::type;
    __shared__ float w_lds[kSsdWindow];
    __shared__ float wave_tot[kWaves];

    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    const int L = (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int segs = a.n_segs - 1;
    const int part = L % NS;
    const int rbw = (L / NS) % a.n_row_blocks;
    const int hd = (L / (NS * a.n_row_blocks)) % a.H;
    const int seg = (L / (NS * a.n_row_blocks * a.H)) % segs;
    const int s = L / (NS * a.n_row_blocks * a.H * segs);

    const int H = a.H, P = a.P, G = a.G;
    const int Nr = a.N;                              // state columns in memory (N rounds it up)
    const int g = hd / a.heads_per_group;
    const SegRange sr = segment_range(a, s, seg);
    if (seg >= sr.n_real - 1) return;                // the last segment needs no pass
    const int t_begin = sr.t_begin, t_end = sr.t_end; // at least one token
    const bool from_slot = seg == 0 && a.fresh[s] == 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: offsets in SGPRs
    const int tl = lane & 15, kq = lane >> 4;
    const int p0 = rbw * 64 + 32 * (w & 1);          // the wave's two row tiles: p0, p0 + 16
    const bool tile_ok[2] = {p0 < P, p0 + 16 < P};   // P % 16 == 0: whole tiles
    const int n_base = (2 * part + (w >> 1)) * NW;
    const int64_t hpn = int64_t(H) * P * Nr;
    const float A_h = a.A[hd];
    const float bias_h = a.dt_bias ? a.dt_bias[hd] : 0.f;

    // hacc[t][e] register v of lane l: h[p0 + 16 t + l%16][n_base + E (4 (l/16) + v) + e]
    f4m hacc[2][E];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) hacc[t][e] = f4m{0.f, 0.f, 0.f, 0.f};
    // columns at Nr and past (N > Nr: padding to whole 16-column tiles) hold
    // zeros: their B reads as zero and they are neither loaded nor stored.
    // Nr % 4 == 0 and E <= 4 or Nr % 8 == 0, so a lane's E columns are all in
    // or all out.
    const int64_t head_off = int64_t(hd) * P * Nr;
    if (from_slot) {
        const float *src = a.state + int64_t(a.slot[s]) * hpn + head_off + n_base;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (!tile_ok[t]) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if (n_base + E * (4 * kq + v) >= Nr) continue;
                const fE h = *reinterpret_cast<const fE *>(src + int64_t(p0 + 16 * t + tl) * Nr + E * (4 * kq + v));
#pragma unroll
                for (int e = 0; e < E; ++e) hacc[t][e][v] = vget<E>(h, e);
            }
        }
    }

    // operand registers of one load group: step k covers tokens 4 k + l/16.
    // Buffer descriptors cover the window's tokens; the lane's byte offsets
    // are fixed, the group and step advance in the scalar offset.  (A tile
    // past P reads rows of the next head or zeros: it is never stored.)
    float xg[2][KS][2];
    fE bg[2][KS];
    constexpr int kNone = 0x7ffffff0;                // a byte offset past every descriptor
    const int x_tok = H * P * int(sizeof(float)), b_tok = G * Nr * int(sizeof(float));
    const int vo_x = (kq * H * P + hd * P + p0 + tl) * int(sizeof(float));
    const int vo_b = n_base + E * tl < Nr ? (kq * G * Nr + g * Nr + n_base + E * tl) * int(sizeof(float)) : kNone;
    __amdgpu_buffer_rsrc_t rx, rb;
    auto load_group = [&](int r, int j0) {           // j0: first token of the group in the window
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            xg[r][k][0] = buffer_load<1>(rx, vo_x, (j0 + 4 * k) * x_tok);
            xg[r][k][1] = buffer_load<1>(rx, vo_x + 16 * int(sizeof(float)), (j0 + 4 * k) * x_tok);
            bg[r][k] = buffer_load<E>(rb, vo_b, (j0 + 4 * k) * b_tok);
        }
    };
    auto mma_group = [&](int r, int w0) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const float wk = w_lds[w0 + 4 * k + kq];
            const float wx0 = wk * xg[r][k][0], wx1 = wk * xg[r][k][1];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                hacc[0][e] = mfma16(vget<E>(bg[r][k], e), wx0, hacc[0][e]);
                hacc[1][e] = mfma16(vget<E>(bg[r][k], e), wx1, hacc[1][e]);
            }
        }
    };

    float run = 1.f;                                   // product of dA over the segment
    for (int tw = t_begin; tw < t_end; tw += kSsdWindow) {
        const int m = min(kSsdWindow, t_end - tw);
        rx = buffer_of(a.x + int64_t(tw) * H * P, m * x_tok);
        rb = buffer_of(a.B + int64_t(tw) * G * Nr, m * b_tok);
        if (tile_ok[0]) load_group(0, 0);              // first operands in flight during the prologue
        // ---- prologue: w_t = e^{S_last - S_t} dt_t for the window's tokens.  The
        // exponent is summed from the window end backwards (thread 0 takes the
        // last tokens), so it is exact to rounding of its own size where the
        // weight matters; a difference of two long running sums would not be.
        __syncthreads();                               // the previous window's weights are read
        float d[TPT], c[TPT];
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int j = kSsdWindow - 1 - (TPT * tid + i);
            d[i] = j < m ? dt_transform(a.dt[int64_t(tw + j) * H + hd], bias_h, a.dt_softplus) : 0.f;
            c[i] = acc;                                // sum over the thread's later tokens
            acc += d[i] * A_h;
        }
        const float incl = wave_prefix_sum(acc, lane);
        if (lane == 63) wave_tot[w] = incl;
        __syncthreads();
        float after = incl - acc, total = 0.f;        // sum over the tokens after the thread's
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            const float t = wave_tot[k];
            total += t;
            if (k < w) after += t;
        }
#pragma unroll
        for (int i = 0; i < TPT; ++i)
            w_lds[kSsdWindow - 1 - (TPT * tid + i)] = expf(after + c[i]) * d[i];
        const float e_tot = expf(total);
        run *= e_tot;
        __syncthreads();
        // ---- h^T <- e^{S_last} h^T + B^T (w X) over the window, IT tokens per
        // group, pairs of groups (tokens past the window end weigh 0), the next
        // group's loads issued before this group's products; scheduling barriers
        // keep them there (left alone the compiler sinks loads to their use)
        __builtin_amdgcn_s_setprio(0);
        if (tile_ok[0]) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < E; ++e) hacc[t][e] *= e_tot;
            const int n_pairs = (m + 2 * IT - 1) / (2 * IT);
            for (int q = 0; q < 2 * n_pairs; q += 2) {
                load_group(1, (q + 1) * IT);
                __builtin_amdgcn_sched_barrier(0);
                mma_group(0, q * IT);
                load_group(0, (q + 2) * IT);
                __builtin_amdgcn_sched_barrier(0);
                mma_group(1, (q + 1) * IT);
            }
        }
    }
    if (rbw == 0 && part == 0 && tid == 0) a.ws_dtot[(int64_t(s) * a.n_segs + seg) * H + hd] = run;
    float *dst = a.ws_state + (int64_t(s) * a.n_segs + seg) * hpn + head_off + n_base;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!tile_ok[t]) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (n_base + E * (4 * kq + v) >= Nr) continue;
            fE h;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if constexpr (E == 1) h = hacc[t][e][v]; else h[e] = hacc[t][e][v];
            }
            *reinterpret_cast<fE *>(dst + int64_t(p0 + 16 * t + tl) * Nr + E * (4 * kq + v)) = h;
        }
    }
}

// The scan pass.  A workgroup owns a window of 64 TW consecutive rows of the
// flattened (head, row) space inside one B/C group (rows of consecutive heads
// sit next to each other in x, y, the state and the workspace), cut at the
// group's end; wave w owns rows 16 TW w .. 16 TW w + 16 TW - 1, TW tiles of one
// head.  With TW = 2 a wave reads B and C out of LDS once per chunk for 32
// rows, and G^T is formed once for every head of the window; wave 0 forms the
// per-token scalars of up to four heads, one 16-lane DPP row per head.  Grid:
// n_seqs x n_segs x G x (windows per group, a.n_row_blocks) workgroups,
// XCD-contiguous order.  Requires the vector path, N = 16 NT and P % (16 TW)
// == 0.  Segment k > 0 starts from workspace entry k - 1, which the combine
// pass left holding the state carried into it.
template <int NT, int TW>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
ssd_scan_kernel(ScanArgs a) {
    using S = SsdScanShape<NT, TW>;
    constexpr int N = S::N, CT = S::CT, LDN = S::LDN, LDC = S::LDC;
    extern __shared__ float4 lds_raw[];
    float *const lds = reinterpret_cast<float *>(lds_raw);

    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    const int L = (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int wpg = a.n_row_blocks;                  // windows per group
    const int wb = L % wpg;
    const int g = (L / wpg) % a.G;
    const int seg = (L / (wpg * a.G)) % a.n_segs;
    const int s = L / (wpg * a.G * a.n_segs);

    const int H = a.H, P = a.P, G = a.G;
    const int Nr = a.N;                              // state columns in memory (N rounds it up)
    const SegRange sr = segment_range(a, s, seg);
    const int last = sr.n_real - 1;
    if (seg > last) return;                          // past the sequence's segments
    const int t_begin = sr.t_begin, t_end = sr.t_end;
    const int n_tok = t_end - t_begin;
    const bool from_slot = seg == 0 && a.fresh[s] == 0;
    const bool from_carry = seg > 0;
    if (from_slot && n_tok <= 0) return;             // empty resume: slot unchanged

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: row offsets in SGPRs
    const int tl = lane & 15, kq = lane >> 4;        // lane % 16, lane / 16
    const int group_end = (g + 1) * a.heads_per_group * P;   // one past the group's last row
    const int fr_wg = g * a.heads_per_group * P + wb * S::RBW;  // first row h P + p of the window
    const int rows_wg = min(S::RBW, group_end - fr_wg);       // rows of the window (a multiple of 16 TW)
    const int h_wg = fr_wg / P;                      // its first head
    const int n_heads_wg = (fr_wg + rows_wg - 1) / P - h_wg + 1;   // heads it touches (<= MH)
    const int fr0 = fr_wg + 16 * TW * w;             // first row of this wave
    const bool wave_ok = fr0 < fr_wg + rows_wg;      // whole waves: P % (16 TW) == 0
    const int hw = wave_ok ? fr0 / P - h_wg : 0;     // this wave's head, relative to h_wg
    const int64_t HPN = int64_t(H) * P * Nr;
    float *const st_w = a.state + int64_t(a.slot[s]) * HPN + int64_t(fr0) * Nr;
    float *const ws_w = a.ws_state + int64_t(s) * a.n_segs * HPN + int64_t(fr0) * Nr;
    // wave 0, DPP row j = lane / 16: the scalars of head h_wg + j
    const bool hrow_ok = kq < n_heads_wg;
    const float A_j = (tid < 64 && hrow_ok) ? a.A[h_wg + kq] : 0.f;
    const float bias_j = (tid < 64 && hrow_ok && a.dt_bias) ? a.dt_bias[h_wg + kq] : 0.f;

    // ---- state h^T in accumulators: hacc[i][nt] register v of lane l holds
    // h[row fr0 + 16 i + l%16][16 nt + 4 (l/16) + v]; columns at Nr and past
    // (padding to whole tiles, Nr % 4 == 0) stay zero and are never stored
    f4m hacc[TW][NT];
    // Loaded through a buffer descriptor that is empty for a fresh segment 0
    // (zeros, no memory touched) and covers the wave's rows otherwise: the
    // same loads on every path.  Issued right after the first chunk's loads,
    // so the two latencies overlap.
    auto load_state = [&]() {
        const float *src = from_slot ? st_w : ws_w + int64_t(seg > 0 ? seg - 1 : 0) * HPN;
        const int bytes = (from_slot || from_carry) && wave_ok ? 16 * TW * Nr * int(sizeof(float)) : 0;
        const __amdgpu_buffer_rsrc_t rs = buffer_of(src, bytes);
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int n0 = 16 * nt + 4 * kq;
                const int vo = n0 < Nr ? ((16 * i + tl) * Nr + n0) * int(sizeof(float)) : 0x7ffffff0;
                const f4 v = buffer_load4_nt(rs, vo);
                hacc[i][nt] = f4m{v.x, v.y, v.z, v.w};
            }
    };

    // ---- chunk staging: buffer loads -> registers -> LDS (double-buffered).
    // Each thread's byte offsets into a chunk are fixed; a chunk's descriptors
    // cover its tokens only, so the units past the segment end read zeros, and
    // so do the padding columns of B and C (Nr and past).
    // Loads run PF chunks ahead (chunk k lands in register set k % PF: two with
    // one tile per wave; with two tiles, two waves per SIMD leave room for one)
    // and chunk k is committed to LDS buffer k & 1.
    constexpr int kNone = 0x7ffffff0;
    const int x_tok = H * P * int(sizeof(float));
    int vo_bc[S::U_BC], lo_bc[S::U_BC], lo_c[S::U_BC], vo_x[S::U_X], lo_x[S::U_X];
#pragma unroll
    for (int u = 0; u < S::U_BC; ++u) {
        const int q = u * kThreads + tid;            // unit = (token, 4-group)
        const int tt = q / (N / 4), n0 = 4 * (q - tt * (N / 4));
        vo_bc[u] = q < CT * N / 4 && n0 < Nr ? ((tt * G + g) * Nr + n0) * int(sizeof(float)) : kNone;
        lo_bc[u] = q < CT * N / 4 ? tt * LDN + n0 : -1;       // B at stride LDN
        lo_c[u] = tt * LDC + n0;                              // C and B's copy at LDC
    }
#pragma unroll
    for (int u = 0; u < S::U_X; ++u) {
        const int q = u * kThreads + tid;            // unit = (token, 4 rows)
        const int tt = q / (S::RBW / 4), pi = 4 * (q - tt * (S::RBW / 4));
        vo_x[u] = pi < rows_wg ? (tt * H * P + fr_wg + pi) * int(sizeof(float)) : kNone;
        lo_x[u] = tt * S::XR + pi;
    }
    // dt: lane 16 j + t of wave 0 takes token t of head h_wg + j
    const int vo_dt = (tid < 64 && hrow_ok) ? (tl * H + h_wg + kq) * int(sizeof(float)) : kNone;
    struct Stage {
        f4 pb[S::U_BC], pc[S::U_BC], px[S::U_X];
        float pdt;
    };
    Stage stg[S::PF];
    auto issue_loads = [&](Stage &sg, int t0, int nt_) {
        const __amdgpu_buffer_rsrc_t rb = buffer_of(a.B + int64_t(t0) * G * Nr, nt_ * G * Nr * int(sizeof(float)));
        const __amdgpu_buffer_rsrc_t rc = buffer_of(a.C + int64_t(t0) * G * Nr, nt_ * G * Nr * int(sizeof(float)));
        const __amdgpu_buffer_rsrc_t rx = buffer_of(a.x + int64_t(t0) * H * P, nt_ * x_tok);
        const __amdgpu_buffer_rsrc_t rd = buffer_of(a.dt + int64_t(t0) * H, nt_ * H * int(sizeof(float)));
#pragma unroll
        for (int u = 0; u < S::U_BC; ++u) {
            sg.pb[u] = buffer_load<4>(rb, vo_bc[u], 0);
            sg.pc[u] = buffer_load<4>(rc, vo_bc[u], 0);
        }
#pragma unroll
        for (int u = 0; u < S::U_X; ++u) sg.px[u] = buffer_load<4>(rx, vo_x[u], 0);
        sg.pdt = buffer_load<1>(rd, vo_dt, 0);      // raw dt: transformed at the commit
    };
    // Deferred decay: the accumulators hold h / sigma.  A chunk whose decay
    // stays within e^{-kSsdFastDecay} runs in "deferred" form: the state is not
    // rescaled, the update's weights are e^{-S_s} dt_s / sigma and sigma takes
    // the chunk's decay; once sigma would fall below kSsdFloor the state first
    // takes sigma (renormalised, sigma = 1).  A chunk that decays further runs
    // the exact form (the state renormalised first, then scaled by e^{S_15}).
    // In the deferred form the masked intra-chunk term factorises,
    //     e^{S_t - S_s} dt_s = e^{S_t} sigma * (e^{-S_s} dt_s / sigma),
    // so one weighted x serves both products and y takes e^{S_t} sigma per row.
    // Per head: wave 0's lanes of DPP row j hold head j's sigma.
    float sigma = 1.f;
    auto commit = [&](auto bufc, int nt_) {
        constexpr int buf = decltype(bufc)::value;
        float *base = lds + buf * S::BUF;
        const Stage &sg = stg[buf % S::PF];
#pragma unroll
        for (int u = 0; u < S::U_BC; ++u) {
            if (lo_bc[u] >= 0) {
                *reinterpret_cast<f4 *>(base + S::OFF_B + lo_bc[u]) = sg.pb[u];
                *reinterpret_cast<f4 *>(base + S::OFF_BR + lo_c[u]) = sg.pb[u];
                *reinterpret_cast<f4 *>(base + S::OFF_C + lo_c[u]) = sg.pc[u];
            }
        }
#pragma unroll
        for (int u = 0; u < S::U_X; ++u) *reinterpret_cast<f4 *>(base + S::OFF_X + lo_x[u]) = sg.px[u];
        if (tid < 64) {                                  // wave 0: row j = head h_wg + j, lane t = token t
            const float dtv = (tl < nt_ && hrow_ok) ? dt_transform(sg.pdt, bias_j, a.dt_softplus) : 0.f;
            const float Sv = row_prefix_sum(dtv * A_j);
            float S15 = 0.f;
#pragma unroll
            for (int r = 0; r < S::MH; ++r) {
                const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Sv), 16 * r + 15));
                if (kq == r) S15 = v;
            }
            const float e15 = expf(S15);
            const bool fast = S15 >= -kSsdFastDecay;
            float pre = 1.f;
            if (!fast || sigma * e15 < kSsdFloor) {      // renormalise before the chunk
                pre = sigma;
                sigma = 1.f;
            }
            const int o = kq * CT + tl;
            if (fast) {
                base[S::OFF_W + o] = __expf(-Sv) * dtv / sigma;
                base[S::OFF_ES + o] = __expf(Sv) * sigma;
            } else {
                base[S::OFF_S + o] = Sv;
                base[S::OFF_DT + o] = dtv;
                base[S::OFF_ES + o] = expf(Sv);
                base[S::OFF_W + o] = expf(S15 - Sv) * dtv;
            }
            if (tl == 0) {
                base[S::OFF_E15 + kq] = fast ? 1.f : e15;
                base[S::OFF_PRE + kq] = pre;
                base[S::OFF_MODE + kq] = fast ? 1.f : 0.f;
            }
            sigma = fast ? sigma * e15 : 1.f;
        }
    };

    // y of a chunk is finished during the next one: the G^T parts (written to
    // LDS slot c & 1) are summed after the barrier that ends chunk c, scaled by
    // the coefficients kept here and multiplied into the operand kept here,
    // then added to the carried-in term:  y = (ysave + G' X) * yscale.
    f4m ysave[TW];
    float gopnd[TW][4], gcoef[4], yscale[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        gcoef[v] = 0.f;
        yscale[v] = 0.f;
#pragma unroll
        for (int i = 0; i < TW; ++i) gopnd[i][v] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < TW; ++i) ysave[i] = f4m{0.f, 0.f, 0.f, 0.f};
    const int vo_y = ((4 * kq) * H * P + fr0 + tl) * int(sizeof(float));
    auto finish_y = [&](int par, int c) {
        const f4m *gx = reinterpret_cast<const f4m *>(lds + S::OFF_GX + par * S::GX);
        f4m gacc = gx[lane];
#pragma unroll
        for (int k = 1; k < kWaves; ++k) gacc += gx[k * 64 + lane];
        float ga[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) ga[v] = gacc[v] * gcoef[v];
        const int t0 = t_begin + c * CT;
        const __amdgpu_buffer_rsrc_t ry = buffer_of(a.y + int64_t(t0) * H * P, min(CT, t_end - t0) * x_tok);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            f4m y = ysave[i];
#pragma unroll
            for (int v = 0; v < 4; ++v) y = mfma16(ga[v], gopnd[i][v], y);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[v] * yscale[v]), ry,
                                                      vo_y + 16 * i * int(sizeof(float)), v * x_tok, 0);
        }
    };
    auto compute = [&](auto bufc, int c) {
        constexpr int buf = decltype(bufc)::value;   // chunk c's LDS buffer and G^T slot: c & 1
        const float *base = lds + buf * S::BUF;
        // this wave's quarter of G^T = B C^T (steps f = 4 tile + j, n = 16 tile + 4 (l/16) + j)
        f4m gpart = {0.f, 0.f, 0.f, 0.f};
        // wave w takes state tiles w, w + 4, ...: one float4 of B and of C per
        // tile (steps f = 4 tile + j, n = 16 tile + 4 (l/16) + j)
        constexpr int GT = (NT + kWaves - 1) / kWaves;
        float gb[4 * GT], gc[4 * GT];
#pragma unroll
        for (int k = 0; k < GT; ++k) {
            const int nt = w + kWaves * k;
            const int off = 16 * nt + 4 * kq;
            f4 bq = {0.f, 0.f, 0.f, 0.f}, cq = {0.f, 0.f, 0.f, 0.f};
            if (NT % kWaves == 0 || nt < NT) {
                bq = *reinterpret_cast<const f4 *>(base + S::OFF_BR + tl * LDC + off);
                cq = *reinterpret_cast<const f4 *>(base + S::OFF_C + tl * LDC + off);
            }
            gb[4 * k + 0] = bq.x; gb[4 * k + 1] = bq.y; gb[4 * k + 2] = bq.z; gb[4 * k + 3] = bq.w;
            gc[4 * k + 0] = cq.x; gc[4 * k + 1] = cq.y; gc[4 * k + 2] = cq.z; gc[4 * k + 3] = cq.w;
        }
        float xr[TW][4];
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) xr[i][v] = base[S::OFF_X + (4 * kq + v) * S::XR + 16 * TW * w + 16 * i + tl];
        float bup[4][NT];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                bup[q][nt] = base[S::OFF_B + (4 * kq + q) * LDN + 16 * nt + tl];
        f4 creg[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            creg[nt] = *reinterpret_cast<const f4 *>(base + S::OFF_C + tl * LDC + 16 * nt + 4 * kq);
        const float pre = base[S::OFF_PRE + hw];
        const bool fast = base[S::OFF_MODE + hw] != 0.f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4 * GT; ++i) gpart = mfma16(gb[i], gc[i], gpart);
        reinterpret_cast<f4m *>(lds + S::OFF_GX + buf * S::GX)[w * 64 + lane] = gpart;
        __builtin_amdgcn_sched_barrier(0);
        if (!wave_ok) return;                        // past the group: staging and G^T only
        if (c > 0) finish_y(buf ^ 1, c - 1);         // the previous chunk's parts are all in
        if (pre != 1.f) {                            // renormalise the deferred state
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) hacc[i][nt] *= pre;
        }
        f4m yacc[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) yacc[i] = f4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                yacc[i] = mfma16(creg[nt].x, hacc[i][nt][0], yacc[i]);
                yacc[i] = mfma16(creg[nt].y, hacc[i][nt][1], yacc[i]);
                yacc[i] = mfma16(creg[nt].z, hacc[i][nt][2], yacc[i]);
                yacc[i] = mfma16(creg[nt].w, hacc[i][nt][3], yacc[i]);
            }
        const float *sc = base + hw * CT;            // this wave's head's per-token scalars
        float wx[TW][4];
        if (fast) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float wv = sc[S::OFF_W + 4 * kq + v];
                gcoef[v] = (4 * kq + v <= tl) ? 1.f : 0.f;
                yscale[v] = sc[S::OFF_ES + 4 * kq + v];
#pragma unroll
                for (int i = 0; i < TW; ++i) {
                    wx[i][v] = wv * xr[i][v];
                    gopnd[i][v] = wx[i][v];
                }
            }
#pragma unroll
            for (int i = 0; i < TW; ++i) ysave[i] = yacc[i];
        } else {
            const float S_t = sc[S::OFF_S + tl];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int sv = 4 * kq + v;
                gcoef[v] = (sv <= tl) ? __expf(S_t - sc[S::OFF_S + sv]) * sc[S::OFF_DT + sv] : 0.f;
                yscale[v] = 1.f;
                const float es = sc[S::OFF_ES + sv], wv = sc[S::OFF_W + sv];
#pragma unroll
                for (int i = 0; i < TW; ++i) {
                    gopnd[i][v] = xr[i][v];
                    ysave[i][v] = yacc[i][v] * es;
                    wx[i][v] = wv * xr[i][v];
                }
            }
        }
        const float mid = base[S::OFF_E15 + hw];
        if (mid != 1.f) {
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) hacc[i][nt] *= mid;
        }
        // h^T += B^T (w X) for both tiles
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) hacc[i][nt] = mfma16(bup[q][nt], wx[i][q], hacc[i][nt]);
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    const int n_chunks = (n_tok + CT - 1) / CT;
    auto issue_chunk = [&](Stage &sg, int k) {
        const int t0 = t_begin + min(k, n_chunks - 1) * CT;
        issue_loads(sg, t0, min(CT, t_end - t0));
    };
    if (n_chunks > 0) {
#pragma unroll
        for (int k = 0; k < S::PF; ++k) issue_chunk(stg[k], k);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_state();
    __builtin_amdgcn_sched_barrier(0);
    if (n_chunks > 0) commit(B0{}, min(CT, n_tok));
    __syncthreads();
    // the state is in registers before the chunk loop (whose waits then count
    // only the chunk loads)
    __builtin_amdgcn_s_waitcnt(0);
    auto step = [&](int c, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const int t1 = t_begin + (c + 1) * CT;
        issue_chunk(stg[(buf + S::PF) % S::PF], c + S::PF);   // into the set chunk c just left
        __builtin_amdgcn_sched_barrier(0);
        compute(bufc, c);
        // the commit and the barrier at high wave priority: every wave of the
        // workgroup waits at the barrier for the slowest commit, while the
        // other workgroup's wave on the SIMD would take the issue slots
        // (-1.5% cycles at 1 x 4096)
        __builtin_amdgcn_s_setprio(3);
        if (c + 1 < n_chunks) commit(std::integral_constant<int, buf ^ 1>{}, min(CT, t_end - t1));
        __syncthreads();
        __builtin_amdgcn_s_setprio(0);
    };
    // (a pair cut short leaves the loop at once, so the loop head's wait counts
    // only the loads of a whole pair)
    for (int c = 0; c < n_chunks; c += 2) {
        step(c, B0{});
        if (c + 1 >= n_chunks) break;
        step(c + 1, B1{});
    }
    if (n_chunks > 0 && wave_ok) finish_y((n_chunks - 1) & 1, n_chunks - 1);

    // ---- the sequence's end state after its last segment: h = sigma * accumulators
    if (seg == last) {
        float *const sig_lds = lds + S::OFF_SIG;
        if (tid < 64 && tl == 0) sig_lds[kq] = sigma;
        __syncthreads();
        const float sg = sig_lds[hw];
        if (wave_ok)
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                if (16 * nt + 4 * kq < Nr)
                __builtin_nontemporal_store(
                    f4{hacc[i][nt][0] * sg, hacc[i][nt][1] * sg, hacc[i][nt][2] * sg, hacc[i][nt][3] * sg},
                    reinterpret_cast<f4 *>(st_w + int64_t(16 * i + tl) * Nr + 16 * nt + 4 * kq));
    }
}

}  // namespace ssm
