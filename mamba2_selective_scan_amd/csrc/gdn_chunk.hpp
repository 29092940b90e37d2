// gdn_chunk.hpp -- the gated delta-rule prefill in chunked matrix form, on the
// matrix cores.
//
// "ssm_gated_delta.cu" runs the recurrence one token at a time.  Over a chunk
// of 32 tokens (G_t the inclusive running log decay from the chunk start,
// gamma_t = e^{G_t}, S0 the state carried in, rows j, key columns i) the
// recurrence unrolls to
//     S_t      = gamma_t S0 + sum_{s<=t} (gamma_t/gamma_s) delta_s k_s^T
//     delta_t  = beta_t (v_t - gamma_t S0 k_t - sum_{s<t} (gamma_t/gamma_s)(k_s.k_t) delta_s)
// so, with A[t][s] = beta_t (gamma_t/gamma_s)(k_t.k_s) for s < t and
// T = (I + A)^-1 (unit lower triangular),
//     Delta = T diag(beta) (V - diag(gamma) K S0^T)
//     Y     = scale (diag(gamma) Q S0^T + M Delta),  M[t][s] = (gamma_t/gamma_s)(q_t.k_s), s <= t
//     S'    = gamma_31 S0 + Delta^T diag(gamma_31/gamma) K
// the recurrence regrouped: the same numbers in real arithmetic.  Every
// product is a dense fp32 contraction on v_mfma_f32_16x16x4f32 (the lane
// rules of ssd_kernel.hpp), over two 16-token tiles: the lower-triangular T,
// M, K K^T and Q K^T are held as their blocks 00, 10 and 11 (tile of t, tile
// of s).  T00 and T11 come from 16-step forward substitutions, T10 from
// T10 = -T11 A10 T00 (the blockwise inverse of a lower-triangular matrix).
//
// Two kernels.  The prep kernel, one wavefront per (sequence, chunk, key
// head), forms the K K^T and Q K^T blocks once for the value heads that share
// the key head, then per value head the decayed, masked A and M blocks and T,
// and leaves T, M and the per-token weights in a workspace unit.  The scan
// kernel, one workgroup per (sequence, value head, 16 value rows), walks the
// chunks: its four wavefronts own a quarter of the key columns each, form
// their parts of K S0^T for both token tiles, sum them through LDS (two
// barriers per chunk), and each then forms Delta and its columns of the new
// state; Y is formed from per-wave partials one chunk behind, off that chain.
// Chunks of 32 tokens halve the chunk-to-chunk steps of the dependent walk
// against chunks of 16.
// Operands come through buffer loads whose descriptors cover the chunk's
// tokens (zeros past the sequence end), so a partial last chunk needs no
// masking.
#pragma once

#include "gdn_kernel.hpp"
#include "ssd_kernel.hpp"

namespace ssm {

// One workspace unit per (sequence, chunk, value head), in floats.  T and M
// blocks are [16][16] row-major (row: token t of the block's t tile, column:
// token s of its s tile); per-token fields have 32 entries.  The output scale
// is folded in here: M holds scale M and GS holds scale gamma_t.
struct GdnUnit {
    static constexpr int CT = 32;        // tokens per chunk
    static constexpr int T00 = 0, T10 = 256, T11 = 512;
    static constexpr int M00 = 768, M10 = 1024, M11 = 1280;
    static constexpr int GS = 1536;      // scale gamma_t
    static constexpr int BETA = 1568;    // beta_t (0 past the sequence end)
    static constexpr int BG = 1600;      // beta_t gamma_t
    static constexpr int WL = 1632;      // gamma_31 / gamma_t
    static constexpr int GLAST = 1664;   // gamma_31
    static constexpr int FLOATS = 1680;  // 16-float multiple: every field is 16-byte aligned
};

struct GdnChunkArgs {
    GdnArgs a;
    float *ws;                 // [n_seqs][max_chunks][Hv][GdnUnit::FLOATS]
    int32_t max_chunks;        // chunks of 32 tokens per sequence in the workspace
};

__device__ __forceinline__ int n_chunks_of(int len) { return (len + GdnUnit::CT - 1) / GdnUnit::CT; }

__device__ __forceinline__ int64_t gdn_unit(const GdnChunkArgs &c, int s, int chunk, int vh) {
    return ((int64_t(s) * c.max_chunks + chunk) * c.a.Hv + vh) * GdnUnit::FLOATS;
}

// ---- prep: one wavefront per (sequence, chunk, key head); grid ceil(units / 4).
template <int NKT>                       // Dk = 16 NKT
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
gdn_chunk_prep_kernel(GdnChunkArgs c) {
    constexpr int Dk = 16 * NKT;
    constexpr int LA = 17;                           // A block row stride
    __shared__ float a_lds[kWaves][3][16 * LA];      // A00, A11, A10
    __shared__ float t_lds[kWaves][2][16 * 16];      // T00, T11
    __shared__ float g_lds[kWaves][64];              // G_t [32], beta_t [32]
    const GdnArgs &a = c.a;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int tl = lane & 15, kq = lane >> 4;
    const int64_t unit = int64_t(blockIdx.x) * kWaves + w;   // (s, chunk, kh), kh fastest
    const int64_t n_units = int64_t(a.n_blocks);
    const int kh = int(unit % a.Hk);
    const int chunk = int((unit / a.Hk) % c.max_chunks);
    const int s = int(unit / (int64_t(a.Hk) * c.max_chunks));
    bool live = unit < n_units;
    int t0 = 0, n = 0;
    if (live) {
        const int c0 = a.cu_seqlens[s], c1 = a.cu_seqlens[s + 1];
        t0 = c0 + GdnUnit::CT * chunk;
        n = min(GdnUnit::CT, c1 - t0);
        live = n > 0;
    }
    // the K K^T and Q K^T blocks; register v of lane l: row 4 (l/16) + v of the
    // t tile, column l%16 of the s tile
    f4m kk00 = {0.f, 0.f, 0.f, 0.f}, kk10 = kk00, kk11 = kk00;
    f4m qk00 = kk00, qk10 = kk00, qk11 = kk00;
    // g and beta of the first two value heads of this key head, loaded with K
    // and Q so that every load of the wavefront is in flight at once
    float gpre0 = 0.f, gpre1 = 0.f, bpre0 = 0.f, bpre1 = 0.f;
    if (live) {
        const int row_bytes = a.Hk * Dk * int(sizeof(float));
        const __amdgpu_buffer_rsrc_t rk = buffer_of(a.k + int64_t(t0) * a.Hk * Dk, n * row_bytes);
        const __amdgpu_buffer_rsrc_t rq = buffer_of(a.q + int64_t(t0) * a.Hk * Dk, n * row_bytes);
        const int vo = (tl * a.Hk * Dk + kh * Dk + 4 * kq) * int(sizeof(float));
        // lane (l%16, l/16): row l%16 of each tile at columns 16 m + 4 (l/16) .. + 3
        f4 kr[NKT][2], qr[NKT][2];
#pragma unroll
        for (int m = 0; m < NKT; ++m) {
            kr[m][0] = buffer_load<4>(rk, vo + 64 * m, 0);
            kr[m][1] = buffer_load<4>(rk, vo + 64 * m, 16 * row_bytes);
            qr[m][0] = buffer_load<4>(rq, vo + 64 * m, 0);
            qr[m][1] = buffer_load<4>(rq, vo + 64 * m, 16 * row_bytes);
        }
        if (lane < n) {
            gpre0 = a.g[int64_t(t0 + lane) * a.Hv + kh];
            bpre0 = a.beta[int64_t(t0 + lane) * a.Hv + kh];
            if (a.heads_per_key > 1) {
                gpre1 = a.g[int64_t(t0 + lane) * a.Hv + kh + a.Hk];
                bpre1 = a.beta[int64_t(t0 + lane) * a.Hv + kh + a.Hk];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NKT; ++m) {
            const f4 k0 = kr[m][0], k1 = kr[m][1], q0 = qr[m][0], q1 = qr[m][1];
            kk00 = mfma16(k0.x, k0.x, kk00); kk10 = mfma16(k1.x, k0.x, kk10); kk11 = mfma16(k1.x, k1.x, kk11);
            qk00 = mfma16(q0.x, k0.x, qk00); qk10 = mfma16(q1.x, k0.x, qk10); qk11 = mfma16(q1.x, k1.x, qk11);
            kk00 = mfma16(k0.y, k0.y, kk00); kk10 = mfma16(k1.y, k0.y, kk10); kk11 = mfma16(k1.y, k1.y, kk11);
            qk00 = mfma16(q0.y, k0.y, qk00); qk10 = mfma16(q1.y, k0.y, qk10); qk11 = mfma16(q1.y, k1.y, qk11);
            kk00 = mfma16(k0.z, k0.z, kk00); kk10 = mfma16(k1.z, k0.z, kk10); kk11 = mfma16(k1.z, k1.z, kk11);
            qk00 = mfma16(q0.z, k0.z, qk00); qk10 = mfma16(q1.z, k0.z, qk10); qk11 = mfma16(q1.z, k1.z, qk11);
            kk00 = mfma16(k0.w, k0.w, kk00); kk10 = mfma16(k1.w, k0.w, kk10); kk11 = mfma16(k1.w, k1.w, kk11);
            qk00 = mfma16(q0.w, k0.w, qk00); qk10 = mfma16(q1.w, k0.w, qk10); qk11 = mfma16(q1.w, k1.w, qk11);
        }
    }
    for (int r = 0; r < a.heads_per_key; ++r) {
        const int vh = kh + r * a.Hk;                  // value heads reading this key head
        float *const u = c.ws + (live ? gdn_unit(c, s, chunk, vh) : 0);
        // per-token G_t (running log decay over the chunk) and beta_t in lanes 0..31
        const bool tok = live && lane < n;
        const float gv = r == 0 ? gpre0 : r == 1 ? gpre1 : tok ? a.g[int64_t(t0 + lane) * a.Hv + vh] : 0.f;
        const float bv = r == 0 ? bpre0 : r == 1 ? bpre1 : tok ? a.beta[int64_t(t0 + lane) * a.Hv + vh] : 0.f;
        float Gv = row_prefix_sum(gv);
        const float G15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gv), 15));
        if (kq == 1) Gv += G15;
        const float G31 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gv), 31));
        if (lane < 32) {
            g_lds[w][lane] = Gv;
            g_lds[w][32 + lane] = bv;
        }
        __syncthreads();
        if (live) {
            const float Gs0 = g_lds[w][tl], Gs1 = g_lds[w][16 + tl];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 4 * kq + v;
                const float Gt0 = g_lds[w][t], Gt1 = g_lds[w][16 + t];
                const float bt0 = g_lds[w][32 + t], bt1 = g_lds[w][48 + t];
                const float r00 = tl <= t ? expf(Gt0 - Gs0) : 0.f;
                const float r11 = tl <= t ? expf(Gt1 - Gs1) : 0.f;
                const float r10 = expf(Gt1 - Gs0);     // every token of tile 1 follows tile 0
                a_lds[w][0][t * LA + tl] = tl < t ? bt0 * r00 * kk00[v] : 0.f;
                a_lds[w][1][t * LA + tl] = tl < t ? bt1 * r11 * kk11[v] : 0.f;
                a_lds[w][2][t * LA + tl] = bt1 * r10 * kk10[v];
                u[GdnUnit::M00 + t * 16 + tl] = a.scale * r00 * qk00[v];
                u[GdnUnit::M11 + t * 16 + tl] = a.scale * r11 * qk11[v];
                u[GdnUnit::M10 + t * 16 + tl] = a.scale * r10 * qk10[v];
            }
            if (lane < 32) {
                const float gam = expf(Gv);
                u[GdnUnit::GS + lane] = a.scale * gam;
                u[GdnUnit::BETA + lane] = bv;
                u[GdnUnit::BG + lane] = bv * gam;
                u[GdnUnit::WL + lane] = expf(G31 - Gv);
                if (lane == 0) u[GdnUnit::GLAST] = expf(G31);
            }
        }
        __syncthreads();
        // T00 = (I + A00)^-1 in lanes 0..15 and T11 = (I + A11)^-1 in lanes
        // 16..31, side by side by forward substitution, a lane per column l:
        // T[t][l] = [t == l] - sum_{s<t} A[t][s] T[s][l]
        if (live && lane < 32) {
            const int blk = kq, col = tl;
            const float *ab = a_lds[w][blk];
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = t == col ? 1.f : 0.f;
#pragma unroll
                for (int q = 0; q < t; ++q) acc = fmaf(-ab[t * LA + q], x[q], acc);
                x[t] = acc;
            }
            float *const tu = u + (blk ? GdnUnit::T11 : GdnUnit::T00);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                t_lds[w][blk][t * 16 + col] = x[t];
                tu[t * 16 + col] = x[t];
            }
        }
        __syncthreads();
        // T10 = -T11 (A10 T00), on the matrix cores: P = A10 T00, then T11 P
        if (live) {
            f4m p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 4; ++v)
                p = mfma16(a_lds[w][2][tl * LA + 4 * kq + v], t_lds[w][0][(4 * kq + v) * 16 + tl], p);
            f4m t10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 4; ++v) t10 = mfma16(t_lds[w][1][tl * 16 + 4 * kq + v], p[v], t10);
#pragma unroll
            for (int v = 0; v < 4; ++v) u[GdnUnit::T10 + (4 * kq + v) * 16 + tl] = -t10[v];
        }
        __syncthreads();                               // the LDS blocks are reused for the next head
    }
}

// ---- scan: one workgroup per (sequence, value head, 16 value rows); its four
// wavefronts own Dk / 4 key columns each.  Grid n_seqs x Hv x Dv/16, XCD-contiguous.
//
// Per chunk, the dependent chain is K S0^T, then R = beta (V - gamma K S0^T),
// then Delta, then the new state.  Each wave forms its part of K S0^T over its
// key columns and leaves it in LDS; after the chunk's first barrier each wave
// sums the four parts of a quarter of R and leaves that quarter in LDS; after
// the second every wave reads all of R.  The output is kept off that chain:
// each wave forms its part of Q S0^T between the two barriers (covering the
// exchange of R), scales it by scale gamma_t, adds its share of scale M Delta
// (wave 0 the M00 Delta_0 block, wave 1 M10 Delta_0, wave 2 M11 Delta_1) and
// leaves that partial y in LDS; after the next chunk's first barrier each wave
// sums the four partials of a quarter of the chunk's y and stores it (the last
// chunk's after the loop).
//
// What the four waves share -- the chunk's workspace unit (T, M, per-token
// weights) and its V rows -- is loaded once per workgroup, each wave a part,
// two chunks ahead, and staged through LDS in three buffers, so a chunk reads
// it before its first barrier, under its K S0^T products; each wave loads
// only its own K and Q columns, also two chunks ahead, between its state
// products, so the texture path works beside the matrix cores instead of
// stalling a burst of issues.  gfx950 issues a wave's VALU work in series with
// its matrix products, so the VALU work per chunk is kept small: the scale,
// gamma_t and beta_t gamma_t come from the prep kernel, R is formed a quarter
// per wave, and gamma_31 / gamma_t scales Delta (8 values per lane) rather
// than K (16).
// Two wavefronts per SIMD at most (176 VGPRs, 66 KB of LDS at Dk 128): a
// batch of two or more sequences runs two workgroups per CU, one wave's VALU
// and LDS work under the other's products (2 x 4096: 22% fewer cycles than
// one workgroup per CU; one sequence, 256 workgroups, is unchanged).
template <int NKT>                       // Dk = 16 NKT, NKT in {4, 8}
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gdn_chunk_scan_kernel(GdnChunkArgs c) {
    constexpr int Dk = 16 * NKT;
    constexpr int CW = NKT / 4;                      // 16-column tiles per wave
    constexpr int CT = GdnUnit::CT;
    static_assert(NKT % 4 == 0, "Dk must be a multiple of 64");
    // staged chunk data, floats: the workspace unit as laid out there, then V
    // rows [32][VS] (16 value rows, padded so a wave's four row groups use
    // distinct banks)
    constexpr int VS = 20;
    constexpr int UNIT_ROUNDS = 7;                   // 64-float4 rounds covering the unit
    static_assert(GdnUnit::FLOATS <= 256 * UNIT_ROUNDS, "the unit fits its staging rounds");
    constexpr int SV = 256 * UNIT_ROUNDS;            // V rows (past the unit and its padding)
    constexpr int SG = SV + CT * VS;
    __shared__ __attribute__((aligned(16))) float stg[3][SG];
    // token tile, wave, lane: each wave's part of K S0^T (xk) and of y (xy).
    // One copy each: a chunk reads the K S0^T parts between its two barriers
    // and the previous chunk's y parts there too, and writes its own y parts
    // after the second barrier and the next chunk's K S0^T parts after that,
    // so no wave writes either while another may still read it.
    __shared__ f4m xk[2][kWaves][64];
    __shared__ f4m xy[2][kWaves][64];
    // R = beta (V - gamma K S0^T), token tile, lane (register layout of K S0^T)
    __shared__ f4m rx[2][64];
    // each wave's K of the chunk (32 tokens x its 16 CW key columns, rows padded
    // to 16 CW + 4), written and read back transposed by the same wave
    constexpr int LDK = 16 * CW + 4;
    __shared__ __attribute__((aligned(16))) float k_lds[kWaves][CT * LDK];
    const GdnArgs &a = c.a;

    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    const int L = (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int rt = L % a.n_row_blocks;               // 16-row tile
    const int vh = (L / a.n_row_blocks) % a.Hv;
    const int s = L / (a.n_row_blocks * a.Hv);
    const int kh = vh % a.Hk;
    const int c0 = a.cu_seqlens[s], c1 = a.cu_seqlens[s + 1];
    const int len = min(c1 - c0, CT * c.max_chunks);  // chunks past the workspace are not run
    const bool fresh = a.fresh[s] != 0;
    if (!fresh && len <= 0) return;                  // empty resume: slot unchanged

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int tl = lane & 15, kq = lane >> 4;
    const int j0 = 16 * rt;                          // first value row
    const int i0 = w * (Dk / 4);                     // first key column of this wave
    const int Hv = a.Hv, Hk = a.Hk, Dv = a.Dv;
    float *const st = a.state + ((int64_t(a.slot[s]) * Hv + vh) * Dv + j0) * Dk;

    // hacc[cc] register v of lane l: S[j0 + l%16][i0 + 16 cc + 4 (l/16) + v]
    f4m hacc[CW];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) hacc[cc] = f4m{0.f, 0.f, 0.f, 0.f};
    if (!fresh) {
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) {
            const f4 v = *reinterpret_cast<const f4 *>(st + int64_t(tl) * Dk + i0 + 16 * cc + 4 * kq);
            hacc[cc] = f4m{v.x, v.y, v.z, v.w};
        }
    }
    // the state is in registers before any chunk load is issued: left to
    // itself the compiler sinks these loads below them, and the loop then
    // waits on every load in flight each chunk
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) asm volatile("" : "+v"(hacc[cc]));

    const int kq_bytes = Hk * Dk * int(sizeof(float)), v_bytes = Hv * Dv * int(sizeof(float));
    const int vo_kq = (tl * Hk * Dk + kh * Dk + i0 + 4 * kq) * int(sizeof(float));
    // a chunk's own K and Q columns of this wave, token tile b in [0, 2):
    // row 16 b + l%16 at columns i0 + 16 cc + 4 (l/16) + v
    struct KQ {
        f4 kr[2][CW], qr[2][CW];
    };
    auto load_kq = [&](KQ &o, int ch) {
        const int t0 = c0 + CT * ch;
        const int nv = min(CT, len - CT * ch);
        const __amdgpu_buffer_rsrc_t rk = buffer_of(a.k + int64_t(t0) * Hk * Dk, nv * kq_bytes);
        const __amdgpu_buffer_rsrc_t rq = buffer_of(a.q + int64_t(t0) * Hk * Dk, nv * kq_bytes);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int cc = 0; cc < CW; ++cc) {
                o.kr[b][cc] = buffer_load<4>(rk, vo_kq + 64 * cc, 16 * b * kq_bytes);
                o.qr[b][cc] = buffer_load<4>(rq, vo_kq + 64 * cc, 16 * b * kq_bytes);
            }
    };
    // this wave's part of the shared chunk data: rounds 3 w .. 3 w + 2 of nine
    // 64-float4 rounds, the unit in rounds 0..6 (float4 e at e; past the unit
    // the descriptor reads zeros into padding) and V in rounds 7 and 8 (token
    // e/4 of the round's 16, value rows j0 + 4 (e%4) .. + 3); waves 2 and 3
    // issue their remaining loads against an empty descriptor.  Every wave
    // issues the same three loads, so the memory counters need no path-dependent waits.
    struct Stage {
        f4 x[3];
    };
    const int vo_sv = (vh * Dv + j0 + 4 * (lane & 3)) * int(sizeof(float)) + (lane >> 2) * v_bytes;
    auto load_stage = [&](Stage &g, int ch) {
        const int t0 = c0 + CT * ch;
        const int nv = min(CT, len - CT * ch);
        const __amdgpu_buffer_rsrc_t ru = buffer_of(c.ws + gdn_unit(c, s, ch, vh), GdnUnit::FLOATS * 4);
        const __amdgpu_buffer_rsrc_t rv = buffer_of(a.v + int64_t(t0) * Hv * Dv, nv * v_bytes);
        const __amdgpu_buffer_rsrc_t rz = buffer_of(a.v, 0);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int rd = 3 * w + r;                // uniform
            const bool unit = rd < UNIT_ROUNDS, vrow = !unit && rd < UNIT_ROUNDS + 2;
            const __amdgpu_buffer_rsrc_t rs = unit ? ru : vrow ? rv : rz;
            const int vo = unit ? 16 * (64 * rd + lane) : vo_sv;
            const int so = vrow ? 16 * (rd - UNIT_ROUNDS) * v_bytes : 0;
            g.x[r] = buffer_load<4>(rs, vo, so);
        }
    };
    auto put_stage = [&](const Stage &g, int par) {
        float *const d = stg[par];
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int rd = 3 * w + r;
            if (rd < UNIT_ROUNDS)
                *reinterpret_cast<f4 *>(d + 4 * (64 * rd + lane)) = g.x[r];
            else if (rd < UNIT_ROUNDS + 2)
                *reinterpret_cast<f4 *>(d + SV + (16 * (rd - UNIT_ROUNDS) + (lane >> 2)) * VS + 4 * (lane & 3)) = g.x[r];
        }
    };
    auto comp = [](const f4 &x, int v) { return v == 0 ? x.x : v == 1 ? x.y : v == 2 ? x.z : x.w; };
    auto ld4 = [](const float *p) { return *reinterpret_cast<const f4 *>(p); };
    // y of chunk ch from the partials in xy (none for ch = -1, whose partials
    // are never written): wave w sums token tile w/2,
    // registers 2 (w%2) and 2 (w%2) + 1 (tokens 16 (w/2) + 4 (l/16) + 2 (w%2) + e)
    const int yb = w >> 1, yh = w & 1;
    const int vo_y = (4 * kq * Hv * Dv + vh * Dv + j0 + tl) * int(sizeof(float));
    auto put_y = [&](int ch) {
        const float *p = reinterpret_cast<const float *>(&xy[yb][0][lane]) + 2 * yh;
        float2 yv = *reinterpret_cast<const float2 *>(p);
#pragma unroll
        for (int k = 1; k < kWaves; ++k) {
            const float2 t = *reinterpret_cast<const float2 *>(p + 4 * 64 * k);
            yv.x += t.x;
            yv.y += t.y;
        }
        const int t0 = c0 + CT * max(ch, 0);        // ch = -1: nothing is stored
        const int ny = ch >= 0 ? min(CT, len - CT * ch) : 0;
        const __amdgpu_buffer_rsrc_t ry = buffer_of(a.y + int64_t(t0) * Hv * Dv, ny * v_bytes);
        const int so = (16 * yb + 2 * yh) * v_bytes;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv.x), ry, vo_y, so, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv.y), ry, vo_y, so + v_bytes, 0);
    };
    const int row = tl * 16 + 4 * kq;
    const int m_off = w == 0 ? GdnUnit::M00 : w == 1 ? GdnUnit::M10 : GdnUnit::M11;
    // one chunk: o holds its K and Q, its shared data is in stg[sp] (sp = ch
    // mod 3, written at the end of the chunk before last, visible since the
    // last barrier); the K and Q of the chunk after next are loaded into on,
    // its shared data into g and, at the end, into stg[(sp + 2) mod 3]
    auto chunk_step = [&](const KQ &o, KQ &on, Stage &g, int ch, int sp) {
        const int last = n_chunks_of(len) - 1;
        // K to LDS, read back transposed for the state update:
        // kt[b][cc][v] = K[16 b + 4 (l/16) + v][i0 + 16 cc + l%16]
        float *const kw = k_lds[w];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int cc = 0; cc < CW; ++cc)
                *reinterpret_cast<f4 *>(kw + (16 * b + tl) * LDK + 16 * cc + 4 * kq) = o.kr[b][cc];
        // this wave's part of K S0^T over its key columns, both tiles; the
        // reads of the chunk's shared data and of K transposed follow it
        f4m ks[2], qs[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) ks[b] = qs[b] = f4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < CW; ++cc)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int b = 0; b < 2; ++b) ks[b] = mfma16(comp(o.kr[b][cc], v), hacc[cc][v], ks[b]);
#pragma unroll
        for (int b = 0; b < 2; ++b) xk[b][w][lane] = ks[b];
        const float *gp = stg[sp];
        const f4 t00 = ld4(gp + GdnUnit::T00 + row), t10 = ld4(gp + GdnUnit::T10 + row),
                 t11 = ld4(gp + GdnUnit::T11 + row), mb = ld4(gp + m_off + row);
        f4 gs[2], wl[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            gs[b] = ld4(gp + GdnUnit::GS + 16 * b + 4 * kq);
            wl[b] = ld4(gp + GdnUnit::WL + 16 * b + 4 * kq);
        }
        // this wave's quarter of R: token tile yb, registers 2 yh and 2 yh + 1
        // (tokens tq and tq + 1), value row j0 + l%16
        const int tq = 16 * yb + 4 * kq + 2 * yh;
        const float2 beq = *reinterpret_cast<const float2 *>(gp + GdnUnit::BETA + tq);
        const float2 bgq = *reinterpret_cast<const float2 *>(gp + GdnUnit::BG + tq);
        const float vq0 = gp[SV + tq * VS + tl], vq1 = gp[SV + (tq + 1) * VS + tl];
        const float glast = gp[GdnUnit::GLAST];
        float kt[2][CW][4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int cc = 0; cc < CW; ++cc)
#pragma unroll
                for (int v = 0; v < 4; ++v) kt[b][cc][v] = kw[(16 * b + 4 * kq + v) * LDK + 16 * cc + tl];
        __syncthreads();
        // this wave's quarter of R from the four parts of K S0^T
        {
            const float *pk = reinterpret_cast<const float *>(&xk[yb][0][lane]) + 2 * yh;
            float2 ksq = *reinterpret_cast<const float2 *>(pk);
#pragma unroll
            for (int k = 1; k < kWaves; ++k) {
                const float2 t = *reinterpret_cast<const float2 *>(pk + 4 * 64 * k);
                ksq.x += t.x;
                ksq.y += t.y;
            }
            float2 rq;
            rq.x = fmaf(-bgq.x, ksq.x, beq.x * vq0);
            rq.y = fmaf(-bgq.y, ksq.y, beq.y * vq1);
            *reinterpret_cast<float2 *>(reinterpret_cast<float *>(&rx[yb][lane]) + 2 * yh) = rq;
        }
        // the shared data of the chunk after next
        __builtin_amdgcn_sched_barrier(0);
        load_stage(g, min(ch + 2, last));
        __builtin_amdgcn_sched_barrier(0);
        // the previous chunk's y: its partials were left before this chunk's first barrier
        put_y(ch - 1);
        // this wave's part of Q S0^T, covering the exchange of R
#pragma unroll
        for (int cc = 0; cc < CW; ++cc)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int b = 0; b < 2; ++b) qs[b] = mfma16(comp(o.qr[b][cc], v), hacc[cc][v], qs[b]);
        __syncthreads();
        // R, register v of lane l: token 16 b + 4 (l/16) + v, value row j0 + l%16
        float rv[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const f4m r = rx[b][lane];
#pragma unroll
            for (int v = 0; v < 4; ++v) rv[b][v] = r[v];
        }
        // Delta_0 = T00 R_0, Delta_1 = T10 R_0 + T11 R_1
        f4m dl0 = {0.f, 0.f, 0.f, 0.f}, dl1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            dl0 = mfma16(comp(t00, v), rv[0][v], dl0);
            dl1 = mfma16(comp(t10, v), rv[0][v], dl1);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) dl1 = mfma16(comp(t11, v), rv[1][v], dl1);
        // this wave's partial y: scale gamma_t (Q S0^T over its columns) plus its M block's share
        f4m yw[2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) yw[b][v] = comp(gs[b], v) * qs[b][v];
        if (w == 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) yw[0] = mfma16(comp(mb, v), dl0[v], yw[0]);
        } else if (w == 1) {
#pragma unroll
            for (int v = 0; v < 4; ++v) yw[1] = mfma16(comp(mb, v), dl0[v], yw[1]);
        } else if (w == 2) {
#pragma unroll
            for (int v = 0; v < 4; ++v) yw[1] = mfma16(comp(mb, v), dl1[v], yw[1]);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) xy[b][w][lane] = yw[b];
        // S' = gamma_31 S0 + (diag(gamma_31/gamma) Delta)^T K, this wave's columns:
        // A operand K[s][i0 + 16 cc + l%16] with s = 16 b + 4 (l/16) + v, B operand the scaled Delta
        f4m dw0, dw1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            dw0[v] = comp(wl[0], v) * dl0[v];
            dw1[v] = comp(wl[1], v) * dl1[v];
        }
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) hacc[cc] *= glast;
        // the state products with the loads of the chunk after next between
        // them, one load per two products
        __builtin_amdgcn_sched_barrier(0);
        load_kq(on, min(ch + 2, last));
#pragma unroll
        for (int cc = 0; cc < CW; ++cc)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                hacc[cc] = mfma16(kt[0][cc][v], dw0[v], hacc[cc]);
                hacc[cc] = mfma16(kt[1][cc][v], dw1[v], hacc[cc]);
            }
#pragma unroll
        for (int i = 0; i < 4 * CW; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one VMEM read
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMA
        }
        __builtin_amdgcn_sched_barrier(0);
        // the shared data of the chunk after next, for the reads of that chunk
        put_stage(g, sp == 0 ? 2 : sp - 1);
    };

    const int n_chunks = n_chunks_of(len);
    // chunk ch's K and Q are in o(ch mod 3) and its shared data in stg[ch mod 3],
    // both loaded two chunks ahead
    KQ o0, o1, o2;
    Stage g;
    if (n_chunks > 0) {
        load_kq(o0, 0);
        load_kq(o1, min(1, n_chunks - 1));
        load_stage(g, 0);
        put_stage(g, 0);
        load_stage(g, min(1, n_chunks - 1));
        put_stage(g, 1);
    }
    __syncthreads();
    // whole rounds of three chunks, then the rest, with no branch between a
    // round's chunks (a branch there makes the compiler's load waits conservative)
    int ch = 0;
    for (; ch + 3 <= n_chunks; ch += 3) {
        chunk_step(o0, o2, g, ch, 0);
        chunk_step(o1, o0, g, ch + 1, 1);
        chunk_step(o2, o1, g, ch + 2, 2);
    }
    if (ch < n_chunks) chunk_step(o0, o2, g, ch, 0);
    if (ch + 1 < n_chunks) chunk_step(o1, o0, g, ch + 1, 1);
    if (n_chunks > 0) {                              // the last chunk's y
        __syncthreads();
        put_y(n_chunks - 1);
    }
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
        *reinterpret_cast<f4 *>(st + int64_t(tl) * Dk + i0 + 16 * cc + 4 * kq) =
            f4{hacc[cc][0], hacc[cc][1], hacc[cc][2], hacc[cc][3]};
}

}  // namespace ssm
