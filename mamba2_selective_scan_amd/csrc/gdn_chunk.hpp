// gdn_chunk.hpp -- the gated delta-rule prefill in chunked matrix form, on the
// matrix cores.
//
// "ssm_gated_delta.cu" runs the recurrence one token at a time.  Over a chunk
// of 16 tokens (G_t the inclusive running log decay from the chunk start,
// gamma_t = e^{G_t}, S0 the state carried in, rows j, key columns i) the
// recurrence unrolls to
//     S_t      = gamma_t S0 + sum_{s<=t} (gamma_t/gamma_s) delta_s k_s^T
//     delta_t  = beta_t (v_t - gamma_t S0 k_t - sum_{s<t} (gamma_t/gamma_s)(k_s.k_t) delta_s)
// so, with A[t][s] = beta_t (gamma_t/gamma_s)(k_t.k_s) for s < t and
// T = (I + A)^-1 (unit lower triangular),
//     Delta = T diag(beta) (V - diag(gamma) K S0^T)
//     Y     = scale (diag(gamma) Q S0^T + M Delta),  M[t][s] = (gamma_t/gamma_s)(q_t.k_s), s <= t
//     S'    = gamma_15 S0 + Delta^T diag(gamma_15/gamma) K
// the recurrence regrouped: the same numbers in real arithmetic.  Every
// product is a dense fp32 contraction on v_mfma_f32_16x16x4f32 (the lane
// rules of ssd_kernel.hpp); T comes from a 16-step forward substitution.
//
// Two kernels.  The prep kernel, one wavefront per (sequence, chunk, key
// head), forms K K^T and Q K^T once for the value heads that share the key
// head, then per value head the decayed, masked A and M and T, and leaves T,
// M and the per-token weights in a workspace unit.  The scan kernel, one
// workgroup per (sequence, value head, 16 value rows), walks the chunks: its
// four wavefronts own a quarter of the key columns each, form their parts of
// K S0^T and Q S0^T, sum them through LDS (one barrier per chunk), and each
// then forms Delta, Y and its columns of the new state.  Operands come through
// buffer loads whose descriptors cover the chunk's tokens (zeros past the
// sequence end), so a partial last chunk needs no masking.
#pragma once

#include "gdn_kernel.hpp"
#include "ssd_kernel.hpp"

namespace ssm {

// One workspace unit per (sequence, chunk, value head), in floats.
struct GdnUnit {
    static constexpr int T = 0;          // T[16][16] row-major
    static constexpr int M = 256;        // M[16][16] row-major
    static constexpr int GAM = 512;      // gamma_t
    static constexpr int BETA = 528;     // beta_t (0 past the sequence end)
    static constexpr int BGAM = 544;     // beta_t gamma_t
    static constexpr int WL = 560;       // gamma_15 / gamma_t
    static constexpr int GLAST = 576;    // gamma_15
    static constexpr int FLOATS = 592;   // 16-float multiple: every field is 16-byte aligned
};

struct GdnChunkArgs {
    GdnArgs a;
    float *ws;                 // [n_seqs][max_chunks][Hv][GdnUnit::FLOATS]
    int32_t max_chunks;        // chunks of 16 tokens per sequence in the workspace
};

__device__ __forceinline__ int64_t gdn_unit(const GdnChunkArgs &c, int s, int chunk, int vh) {
    return ((int64_t(s) * c.max_chunks + chunk) * c.a.Hv + vh) * GdnUnit::FLOATS;
}

// ---- prep: one wavefront per (sequence, chunk, key head); grid ceil(units / 4).
template <int NKT>                       // Dk = 16 NKT
__global__ void __launch_bounds__(kThreads) gdn_chunk_prep_kernel(GdnChunkArgs c) {
    constexpr int Dk = 16 * NKT;
    __shared__ float a_lds[kWaves][16 * 17];         // A (row stride 17), then per-token scalars
    __shared__ float g_lds[kWaves][32];              // G_t, beta_t
    const GdnArgs &a = c.a;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
        t0 = c0 + 16 * chunk;
        n = min(16, c1 - t0);
        live = n > 0;
    }
    // K K^T and Q K^T: lane (l%16, l/16) holds row l%16 at columns 16 m + 4 (l/16) + j
    f4m kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
    if (live) {
        const int row_bytes = a.Hk * Dk * int(sizeof(float));
        const __amdgpu_buffer_rsrc_t rk = buffer_of(a.k + int64_t(t0) * a.Hk * Dk, n * row_bytes);
        const __amdgpu_buffer_rsrc_t rq = buffer_of(a.q + int64_t(t0) * a.Hk * Dk, n * row_bytes);
        const int vo = (tl * a.Hk * Dk + kh * Dk + 4 * kq) * int(sizeof(float));
        f4 kr[NKT], qr[NKT];
#pragma unroll
        for (int m = 0; m < NKT; ++m) {
            kr[m] = buffer_load<4>(rk, vo + 64 * m, 0);
            qr[m] = buffer_load<4>(rq, vo + 64 * m, 0);
        }
#pragma unroll
        for (int m = 0; m < NKT; ++m) {
            kk = mfma16(kr[m].x, kr[m].x, kk);
            qk = mfma16(qr[m].x, kr[m].x, qk);
            kk = mfma16(kr[m].y, kr[m].y, kk);
            qk = mfma16(qr[m].y, kr[m].y, qk);
            kk = mfma16(kr[m].z, kr[m].z, kk);
            qk = mfma16(qr[m].z, kr[m].z, qk);
            kk = mfma16(kr[m].w, kr[m].w, kk);
            qk = mfma16(qr[m].w, kr[m].w, qk);
        }
    }
    // kk / qk register v of lane l: row t = 4 (l/16) + v, column s = l%16
    for (int r = 0; r < a.heads_per_key; ++r) {
        const int vh = kh + r * a.Hk;                  // value heads reading this key head
        float *const u = c.ws + (live ? gdn_unit(c, s, chunk, vh) : 0);
        // per-token G_t (running log decay) and beta_t; every 16-lane row holds them
        const bool tok = live && tl < n;
        const float gv = tok ? a.g[int64_t(t0 + tl) * a.Hv + vh] : 0.f;
        const float bv = tok ? a.beta[int64_t(t0 + tl) * a.Hv + vh] : 0.f;
        const float Gv = row_prefix_sum(gv);
        const float G15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gv), 15));
        if (lane < 16) {
            g_lds[w][lane] = Gv;
            g_lds[w][16 + lane] = bv;
        }
        __syncthreads();
        if (live) {
            const float Gs = g_lds[w][tl];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 4 * kq + v;
                const float Gt = g_lds[w][t], bt = g_lds[w][16 + t];
                const float ratio = tl <= t ? expf(Gt - Gs) : 0.f;
                a_lds[w][t * 17 + tl] = tl < t ? bt * ratio * kk[v] : 0.f;
                u[GdnUnit::M + t * 16 + tl] = ratio * qk[v];
            }
            if (lane < 16) {
                const float gam = expf(Gv);
                u[GdnUnit::GAM + lane] = gam;
                u[GdnUnit::BETA + lane] = bv;
                u[GdnUnit::BGAM + lane] = bv * gam;
                u[GdnUnit::WL + lane] = expf(G15 - Gv);
                if (lane == 0) u[GdnUnit::GLAST] = expf(G15);
            }
        }
        __syncthreads();
        // T = (I + A)^-1 by forward substitution, lane l < 16 owning column l:
        // T[t][l] = [t == l] - sum_{s<t} A[t][s] T[s][l]
        if (live && lane < 16) {
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = t == lane ? 1.f : 0.f;
#pragma unroll
                for (int q = 0; q < t; ++q) acc = fmaf(-a_lds[w][t * 17 + q], x[q], acc);
                x[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) u[GdnUnit::T + t * 16 + lane] = x[t];
        }
        __syncthreads();                               // a_lds / g_lds reused for the next head
    }
}

// ---- scan: one workgroup per (sequence, value head, 16 value rows); its four
// wavefronts own Dk / 4 key columns each.  Grid n_seqs x Hv x Dv/16, XCD-contiguous.
template <int NKT>                       // Dk = 16 NKT, NKT in {4, 8}
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
gdn_chunk_scan_kernel(GdnChunkArgs c) {
    constexpr int Dk = 16 * NKT;
    constexpr int CW = NKT / 4;                      // 16-column tiles per wave
    static_assert(NKT % 4 == 0, "Dk must be a multiple of 64");
    __shared__ f4m xch[2][2][kWaves][64];            // parity, (K S0^T, Q S0^T), wave, lane
    // each wave's K tile of the chunk (16 tokens x its 16 CW key columns, rows
    // padded to 16 CW + 4), written and read back transposed by the same wave
    constexpr int LDK = 16 * CW + 4;
    __shared__ __attribute__((aligned(16))) float k_lds[kWaves][16 * LDK];
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
    const int len = min(c1 - c0, 16 * c.max_chunks);  // chunks past the workspace are not run
    const bool fresh = a.fresh[s] != 0;
    if (!fresh && len <= 0) return;                  // empty resume: slot unchanged

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

    // one chunk's operands, loaded a chunk ahead
    struct Ops {
        f4 kr[CW], qr[CW];        // K, Q row l%16 at columns i0 + 16 cc + 4 (l/16) + v
        float vv[4];              // V[4 (l/16) + v][j0 + l%16]
        f4 trow, mrow;            // T, M row l%16 at columns 4 (l/16) + v
        f4 gam, beta, bgam, wl;   // token 4 (l/16) + v
        float glast;
    };
    const int kq_bytes = Hk * Dk * int(sizeof(float)), v_bytes = Hv * Dv * int(sizeof(float));
    const int vo_kq = (tl * Hk * Dk + kh * Dk + i0 + 4 * kq) * int(sizeof(float));
    const int vo_v = (4 * kq * Hv * Dv + vh * Dv + j0 + tl) * int(sizeof(float));
    auto load = [&](Ops &o, int ch) {
        const int t0 = c0 + 16 * ch;
        const int nv = min(16, len - 16 * ch);
        const __amdgpu_buffer_rsrc_t rk = buffer_of(a.k + int64_t(t0) * Hk * Dk, nv * kq_bytes);
        const __amdgpu_buffer_rsrc_t rq = buffer_of(a.q + int64_t(t0) * Hk * Dk, nv * kq_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_of(a.v + int64_t(t0) * Hv * Dv, nv * v_bytes);
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) {
            o.kr[cc] = buffer_load<4>(rk, vo_kq + 64 * cc, 0);
            o.qr[cc] = buffer_load<4>(rq, vo_kq + 64 * cc, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) o.vv[v] = buffer_load<1>(rv, vo_v, v * v_bytes);
        const float *u = c.ws + gdn_unit(c, s, ch, vh);
        o.trow = *reinterpret_cast<const f4 *>(u + GdnUnit::T + tl * 16 + 4 * kq);
        o.mrow = *reinterpret_cast<const f4 *>(u + GdnUnit::M + tl * 16 + 4 * kq);
        o.gam = *reinterpret_cast<const f4 *>(u + GdnUnit::GAM + 4 * kq);
        o.beta = *reinterpret_cast<const f4 *>(u + GdnUnit::BETA + 4 * kq);
        o.bgam = *reinterpret_cast<const f4 *>(u + GdnUnit::BGAM + 4 * kq);
        o.wl = *reinterpret_cast<const f4 *>(u + GdnUnit::WL + 4 * kq);
        o.glast = u[GdnUnit::GLAST];
    };
    const int vo_y = (4 * kq * Hv * Dv + vh * Dv + j0 + tl) * int(sizeof(float));
    auto chunk_step = [&](const Ops &o, int ch, int par) {
        // K transposed for the state update, through this wave's LDS tile:
        // kt[cc][v] = K[4 (l/16) + v][i0 + 16 cc + l%16]
        float *const kw = k_lds[w];
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) *reinterpret_cast<f4 *>(kw + tl * LDK + 16 * cc + 4 * kq) = o.kr[cc];
        float kt[CW][4];
#pragma unroll
        for (int cc = 0; cc < CW; ++cc)
#pragma unroll
            for (int v = 0; v < 4; ++v) kt[cc][v] = kw[(4 * kq + v) * LDK + 16 * cc + tl];
        // this wave's parts of K S0^T and Q S0^T over its key columns
        f4m ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) {
            ks = mfma16(o.kr[cc].x, hacc[cc][0], ks);
            qs = mfma16(o.qr[cc].x, hacc[cc][0], qs);
            ks = mfma16(o.kr[cc].y, hacc[cc][1], ks);
            qs = mfma16(o.qr[cc].y, hacc[cc][1], qs);
            ks = mfma16(o.kr[cc].z, hacc[cc][2], ks);
            qs = mfma16(o.qr[cc].z, hacc[cc][2], qs);
            ks = mfma16(o.kr[cc].w, hacc[cc][3], ks);
            qs = mfma16(o.qr[cc].w, hacc[cc][3], qs);
        }
        xch[par][0][w][lane] = ks;
        xch[par][1][w][lane] = qs;
        __syncthreads();
        // every wave needs all of K S0^T (for Delta); Q S0^T only the wave that writes y
        ks = xch[par][0][0][lane];
#pragma unroll
        for (int k = 1; k < kWaves; ++k) ks += xch[par][0][k][lane];
        if (w == 0) {
            qs = xch[par][1][0][lane];
#pragma unroll
            for (int k = 1; k < kWaves; ++k) qs += xch[par][1][k][lane];
        }
        // register v of lane l: token t = 4 (l/16) + v, value row j0 + l%16
        const float gam[4] = {o.gam.x, o.gam.y, o.gam.z, o.gam.w};
        const float bet[4] = {o.beta.x, o.beta.y, o.beta.z, o.beta.w};
        const float bgm[4] = {o.bgam.x, o.bgam.y, o.bgam.z, o.bgam.w};
        const float wl[4] = {o.wl.x, o.wl.y, o.wl.z, o.wl.w};
        const float tr[4] = {o.trow.x, o.trow.y, o.trow.z, o.trow.w};
        const float mr[4] = {o.mrow.x, o.mrow.y, o.mrow.z, o.mrow.w};
        float rv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) rv[v] = bet[v] * o.vv[v] - bgm[v] * ks[v];
        f4m dl = {0.f, 0.f, 0.f, 0.f};                // Delta = T R
#pragma unroll
        for (int v = 0; v < 4; ++v) dl = mfma16(tr[v], rv[v], dl);
        if (w == 0) {
            f4m ym = {0.f, 0.f, 0.f, 0.f};            // M Delta
#pragma unroll
            for (int v = 0; v < 4; ++v) ym = mfma16(mr[v], dl[v], ym);
            const int t0 = c0 + 16 * ch;
            const __amdgpu_buffer_rsrc_t ry = buffer_of(a.y + int64_t(t0) * Hv * Dv, min(16, len - 16 * ch) * v_bytes);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.scale * (gam[v] * qs[v] + ym[v])),
                                                      ry, vo_y, v * v_bytes, 0);
        }
        // S' = gamma_15 S0 + Delta^T diag(gamma_15/gamma) K, this wave's columns:
        // A operand wl_s K[s][i0 + 16 cc + l%16] with s = 4 (l/16) + v, B operand Delta
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) {
            hacc[cc] *= o.glast;
#pragma unroll
            for (int v = 0; v < 4; ++v) hacc[cc] = mfma16(wl[v] * kt[cc][v], dl[v], hacc[cc]);
        }
    };

    const int n_chunks = (len + 15) / 16;
    // The next chunk's loads are issued before this chunk's products, always
    // (the last chunk's again past the end), so the same number of loads is
    // in flight on every path and a chunk waits only for its own; scheduling
    // barriers keep them there (left alone the compiler sinks loads to their use).
    Ops o0, o1;
    const int last = n_chunks - 1;
    if (n_chunks > 0) load(o0, 0);
    for (int ch = 0; ch < n_chunks; ch += 2) {
        load(o1, min(ch + 1, last));
        __builtin_amdgcn_sched_barrier(0);
        chunk_step(o0, ch, 0);
        load(o0, min(ch + 2, last));
        __builtin_amdgcn_sched_barrier(0);
        if (ch + 1 < n_chunks) chunk_step(o1, ch + 1, 1);
    }
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
        *reinterpret_cast<f4 *>(st + int64_t(tl) * Dk + i0 + 16 * cc + 4 * kq) =
            f4{hacc[cc][0], hacc[cc][1], hacc[cc][2], hacc[cc][3]};
}

}  // namespace ssm
