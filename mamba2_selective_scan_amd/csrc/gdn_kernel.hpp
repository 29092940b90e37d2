// gdn_kernel.hpp -- the gated delta-rule recurrence on gfx950, on the same
// register-resident design as the Mamba2 scan (scan_kernel.hpp).
//
// The recurrence ("ssm_gated_delta.cu", fc_ssm_recurrence and its _seq and
// _slots forms): per value head, the state is Dv rows of Dk values, row j
// contiguous over the key coordinate i.  Per token, for every row,
//     row *= exp(g);  pred = row . k;  delta = (v[j] - pred) * beta;
//     row += k * delta;  y[j] = scale * (row . q)
// The rows play the part of the scan's head-dim rows, the key coordinate the
// part of its state index, k, q and v the part of B, C and x.  So the layout
// is the scan's: a row's Dk values are split over R adjacent lanes of a
// 64-wide wavefront, lane r holding the float4 groups r, r+R, ...; a token's
// k, q, v, decay and beta for a chunk of CT tokens are staged in LDS,
// double-buffered, with one barrier per chunk; y leaves through an LDS tile.
//
// Where it departs from Foundry's kernels: they give each row a block of S
// threads and two shared-memory trees with a barrier per level (their warp
// rewrite, a warp per row with a shuffle butterfly).  Here the two dot
// products of a token are DPP butterflies inside the row's R lanes, with no
// barrier, and they run side by side: y uses the identity
//     row_new . q = row_dec . q + delta * (k . q)
// (the page's two-pass factorisation), so y needs the decayed row's dot with
// q, computed with the dot with k, plus k . q, which depends only on the token
// and is computed once per token per workgroup at staging time.  Only float
// association differs from the direct form.
#pragma once

#include "scan_kernel.hpp"

namespace ssm {

struct GdnArgs {
    const int32_t *cu_seqlens;   // [n_seqs+1]; unused by decode
    const int32_t *slot;         // [n_seqs]
    const uint8_t *fresh;        // [n_seqs]
    const float *q;              // [T][Hk][Dk]
    const float *k;              // [T][Hk][Dk]
    const float *v;              // [T][Hv][Dv]
    const float *g;              // [T][Hv] log decay
    const float *beta;           // [T][Hv]
    float *state;                // [n_slots][Hv][Dv][Dk]
    float *y;                    // [T][Hv][Dv]
    float *snapshots;            // [T][Hv][Dv][Dk] or null
    float scale;
    int32_t Hv, Hk, Dk, Dv;
    int32_t heads_per_key;       // Hv / Hk
    int32_t n_row_blocks;        // ceil(Dv / RB)
    int32_t n_blocks;            // n_seqs * Hv * n_row_blocks
};

template <int R_, int J_, int CT_>
struct GdnShape {
    static constexpr int R = R_;                    // lanes per row
    static constexpr int J = J_;                    // float4 groups per lane
    static constexpr int E = 4 * J;                 // state values per lane
    static constexpr int CT = CT_;                  // tokens per staged chunk
    static constexpr int NP = 4 * R * J;            // staged (zero-padded) key width
    static constexpr int ROWS_PER_WAVE = 64 / R;
    static constexpr int RB = kWaves * ROWS_PER_WAVE;   // rows per workgroup
    // One staging buffer, in floats: k[CT][NP] q[CT][NP] v[CT][RB] y[CT][YR]
    // decay[CT] beta[CT] qk[CT]
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + CT * NP;
    static constexpr int OFF_V = OFF_Q + CT * NP;
    // y tile rows padded as in the scan's Shape: lane r of a row stores token
    // r's y, so a row stride of RB would put lanes r and r + 64/RB in one bank
    static constexpr int YR = R == 4 ? 80 : R == 8 ? 40 : R == 16 ? 20 : 12;
    static constexpr int OFF_Y = OFF_V + CT * RB;
    static constexpr int OFF_DECAY = OFF_Y + CT * YR;
    static constexpr int OFF_BETA = OFF_DECAY + CT;
    static constexpr int OFF_QK = OFF_BETA + CT;
    static constexpr int BUF = ((OFF_QK + CT) + 3) / 4 * 4;
    static constexpr int U_KQ = (CT * NP / 4 + kThreads - 1) / kThreads;   // float4 of k (and of q)
    static constexpr int U_V = (CT * RB / 4 + kThreads - 1) / kThreads;    // float4 of v
    static constexpr int TPT = kThreads / CT;       // lanes per token in the k . q pass
    static_assert(R == 4 || R == 8 || R == 16 || R == 32 || R == 64, "R must be a power of two in [4, 64]");
    static_assert(TPT >= 4 && TPT <= 64 && TPT * CT == kThreads, "CT must be a power of two in [4, 64]");
    static_assert(RB % 4 == 0, "rows per block must be a multiple of 4");

    static constexpr int lds_floats(bool decode) { return decode ? 0 : 2 * BUF; }
};

// One token of the delta rule on a lane's E = 4J state values, given its J
// groups of k and q: decay, the row's dots with k and q (DPP over the row's R
// lanes), the rank-1 write; returns y, identical in every lane of the row.
// The per-token prefill and both decode kernels go through here.
template <int R, int J>
__device__ __forceinline__ float gdn_token(float (&h)[4 * J], const f4 (&kv)[J], const f4 (&qv)[J],
                                           float decay, float beta, float qk, float vr, float scale) {
    float pk0 = 0.f, pk1 = 0.f, pq0 = 0.f, pq1 = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float *hj = h + 4 * j;
        hj[0] *= decay; hj[1] *= decay; hj[2] *= decay; hj[3] *= decay;
        pk0 = __builtin_fmaf(hj[0], kv[j].x, pk0);
        pk1 = __builtin_fmaf(hj[1], kv[j].y, pk1);
        pk0 = __builtin_fmaf(hj[2], kv[j].z, pk0);
        pk1 = __builtin_fmaf(hj[3], kv[j].w, pk1);
        pq0 = __builtin_fmaf(hj[0], qv[j].x, pq0);
        pq1 = __builtin_fmaf(hj[1], qv[j].y, pq1);
        pq0 = __builtin_fmaf(hj[2], qv[j].z, pq0);
        pq1 = __builtin_fmaf(hj[3], qv[j].w, pq1);
    }
    const float pred = row_allreduce<R>(pk0 + pk1);
    const float oq = row_allreduce<R>(pq0 + pq1);
    const float delta = (vr - pred) * beta;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float *hj = h + 4 * j;
        hj[0] = __builtin_fmaf(kv[j].x, delta, hj[0]);
        hj[1] = __builtin_fmaf(kv[j].y, delta, hj[1]);
        hj[2] = __builtin_fmaf(kv[j].z, delta, hj[2]);
        hj[3] = __builtin_fmaf(kv[j].w, delta, hj[3]);
    }
    return scale * __builtin_fmaf(qk, delta, oq);
}

template <class S, bool VEC, bool DECODE, bool SNAP>
__global__ void __launch_bounds__(kThreads) gdn_kernel(GdnArgs a) {
    extern __shared__ float4 lds_raw[];
    float *const lds = reinterpret_cast<float *>(lds_raw);
    constexpr int R = S::R, J = S::J, E = S::E, CT = S::CT, NP = S::NP, RB = S::RB;

    // ---- workgroup -> (sequence, key head, its value heads, row block), with
    // the XCD-contiguous order of the scan: the value heads that share a key
    // head's q and k sit next to each other, on one XCD's L2.
    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    const int L = (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int rb = L % a.n_row_blocks;
    const int m = (L / a.n_row_blocks) % a.Hv;
    const int s = L / (a.n_row_blocks * a.Hv);
    const int kh = m / a.heads_per_key;
    const int vh = (m % a.heads_per_key) * a.Hk + kh;        // key head of vh is vh % Hk

    const int Hv = a.Hv, Hk = a.Hk, Dk = a.Dk, Dv = a.Dv;
    int t_begin, t_end;
    if constexpr (DECODE) {
        t_begin = s;
        t_end = s + 1;
    } else {
        t_begin = a.cu_seqlens[s];
        t_end = a.cu_seqlens[s + 1];
    }
    const int n_tok = t_end - t_begin;
    const bool fresh = a.fresh[s] != 0;
    if (!fresh && n_tok <= 0) return;                // empty resume: slot unchanged

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = (tid >> 6) * S::ROWS_PER_WAVE + lane / R;   // row within the block
    const int r = lane % R;                                    // lane within the row
    const int p0 = rb * RB;
    const int rows_valid = min(RB, Dv - p0);
    const bool row_ok = i < rows_valid;
    // this lane's row of the slot (dereferenced only when row_ok)
    float *const st_row = a.state + ((int64_t(a.slot[s]) * Hv + vh) * Dv + p0 + i) * int64_t(Dk);

    float h[E];
#pragma unroll
    for (int e = 0; e < E; ++e) h[e] = 0.f;

    auto store_row = [&](float *dst, bool nontemporal) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            const int nv = row_ok ? clamp4(Dk - n0) : 0;
            if constexpr (VEC) {
                if (nv > 0) {
                    const f4 v = {h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
                    if (nontemporal)
                        __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(dst + n0));
                    else
                        *reinterpret_cast<f4 *>(dst + n0) = v;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (c < nv) dst[n0 + c] = h[4 * j + c];
            }
        }
    };
    auto snapshot = [&](int t) {
        store_row(a.snapshots + ((int64_t(t) * Hv + vh) * Dv + p0 + i) * int64_t(Dk), false);
    };

    // ---- state -> registers
    if (!fresh) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            const int nv = row_ok ? clamp4(Dk - n0) : 0;
            if constexpr (VEC) {
                if (nv > 0) {
                    const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(st_row + n0));
                    h[4 * j + 0] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (c < nv) h[4 * j + c] = st_row[n0 + c];
            }
        }
    }

    // One token on the lane's E values (gdn_token): y, identical in every
    // lane of the row.  Decode and prefill share it.
    auto token = [&](const f4 (&kv)[J], const f4 (&qv)[J], float decay, float beta, float qk,
                     float vr) -> float {
        return gdn_token<R, J>(h, kv, qv, decay, beta, qk, vr, a.scale);
    };

    if constexpr (DECODE) {
        // One token: the lane's groups of k and q, its row's v and the head's
        // decay and beta straight into registers; k . q from the row's lanes.
        const int64_t kq = (int64_t(s) * Hk + kh) * Dk;
        f4 kv[J], qv[J];
        float kq0 = 0.f, kq1 = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            const int nv = clamp4(Dk - n0);
            kv[j] = load4<VEC>(a.k + kq + n0, nv);
            qv[j] = load4<VEC>(a.q + kq + n0, nv);
            kq0 = __builtin_fmaf(kv[j].x, qv[j].x, kq0);
            kq1 = __builtin_fmaf(kv[j].y, qv[j].y, kq1);
            kq0 = __builtin_fmaf(kv[j].z, qv[j].z, kq0);
            kq1 = __builtin_fmaf(kv[j].w, qv[j].w, kq1);
        }
        const float qk = row_allreduce<R>(kq0 + kq1);
        const float decay = expf(a.g[int64_t(s) * Hv + vh]);
        const float beta = a.beta[int64_t(s) * Hv + vh];
        const float vr = row_ok ? a.v[(int64_t(s) * Hv + vh) * Dv + p0 + i] : 0.f;
        const float yv = token(kv, qv, decay, beta, qk, vr);
        if (r == 0 && row_ok) a.y[(int64_t(s) * Hv + vh) * Dv + p0 + i] = yv;
        if constexpr (SNAP) snapshot(s);
    } else {
        __builtin_amdgcn_s_waitcnt(0);               // state loads done before the pipeline

        f4 pk[S::U_KQ], pq[S::U_KQ], pv[S::U_V];
        float pg = 0.f, pb = 0.f;
        auto issue_loads = [&](int t0, int nt) {
#pragma unroll
            for (int u = 0; u < S::U_KQ; ++u) {
                const int q = u * kThreads + tid;                 // unit = (token, 4-group)
                const int tt = q / (NP / 4);
                const int n0 = 4 * (q - tt * (NP / 4));
                const bool ok = (q < CT * NP / 4) && (tt < nt);
                const int64_t off = (int64_t(t0 + tt) * Hk + kh) * Dk + n0;
                const int nv = ok ? clamp4(Dk - n0) : 0;
                pk[u] = load4<VEC>(a.k + off, nv);
                pq[u] = load4<VEC>(a.q + off, nv);
            }
#pragma unroll
            for (int u = 0; u < S::U_V; ++u) {
                const int q = u * kThreads + tid;                 // unit = (token, 4 rows)
                const int tt = q / (RB / 4);
                const int pi = 4 * (q - tt * (RB / 4));
                const bool ok = (q < CT * RB / 4) && (tt < nt);
                const int nv = ok ? clamp4(rows_valid - pi) : 0;
                pv[u] = load4<VEC>(a.v + (int64_t(t0 + tt) * Hv + vh) * Dv + p0 + pi, nv);
            }
            pg = (tid < nt) ? a.g[int64_t(t0 + tid) * Hv + vh] : 0.f;
            pb = (tid < nt) ? a.beta[int64_t(t0 + tid) * Hv + vh] : 0.f;
        };
        auto commit = [&](int buf) {
            float *base = lds + buf * S::BUF;
            f4 *Ks4 = reinterpret_cast<f4 *>(base + S::OFF_K);
            f4 *Qs4 = reinterpret_cast<f4 *>(base + S::OFF_Q);
            f4 *Vs4 = reinterpret_cast<f4 *>(base + S::OFF_V);
#pragma unroll
            for (int u = 0; u < S::U_KQ; ++u) {
                const int q = u * kThreads + tid;
                if (q < CT * NP / 4) {
                    Ks4[q] = pk[u];
                    Qs4[q] = pq[u];
                }
            }
#pragma unroll
            for (int u = 0; u < S::U_V; ++u) {
                const int q = u * kThreads + tid;
                if (q < CT * RB / 4) Vs4[q] = pv[u];
            }
            if (tid < CT) {
                base[S::OFF_DECAY + tid] = expf(pg);
                base[S::OFF_BETA + tid] = pb;
            }
        };
        // k . q of each staged token: TPT adjacent lanes per token, a DPP sum.
        auto qk_pass = [&](int buf) {
            float *base = lds + buf * S::BUF;
            const f4 *Ks4 = reinterpret_cast<const f4 *>(base + S::OFF_K);
            const f4 *Qs4 = reinterpret_cast<const f4 *>(base + S::OFF_Q);
            const int tt = tid / S::TPT, lt = tid % S::TPT;
            float acc = 0.f;
            for (int gq = lt; gq < NP / 4; gq += S::TPT) {
                const f4 kk = Ks4[tt * (NP / 4) + gq];
                const f4 qq = Qs4[tt * (NP / 4) + gq];
                acc = __builtin_fmaf(kk.x, qq.x, acc);
                acc = __builtin_fmaf(kk.y, qq.y, acc);
                acc = __builtin_fmaf(kk.z, qq.z, acc);
                acc = __builtin_fmaf(kk.w, qq.w, acc);
            }
            acc = row_allreduce<S::TPT>(acc);
            if (lt == 0) base[S::OFF_QK + tt] = acc;
        };

        constexpr int KY = R < 16 ? R : 16;
        const int rk = r % KY;
        int chunk_t0 = 0;
        auto token_y = [&](const float *base, int tt) -> float {
            f4 kv[J], qv[J];
            lds_groups<R, J>(kv, base + S::OFF_K + 4 * r + tt * NP);
            lds_groups<R, J>(qv, base + S::OFF_Q + 4 * r + tt * NP);
            const float yv = token(kv, qv, base[S::OFF_DECAY + tt], base[S::OFF_BETA + tt],
                                   base[S::OFF_QK + tt], base[S::OFF_V + tt * RB + i]);
            if constexpr (SNAP) snapshot(chunk_t0 + tt);
            return yv;
        };
        auto compute = [&](int buf, int nt) {
            const float *base = lds + buf * S::BUF;
            float *Ys = lds + buf * S::BUF + S::OFF_Y + i;
            float y_keep = 0.f;
            int t0 = 0;
            // KY tokens at a time from pointers formed once per group (the
            // tokens' offsets fold into the LDS instructions), each token's
            // operands read one token ahead of its arithmetic
            struct Tok {
                f4 kv[J], qv[J];
                float decay, beta, qk, v;
            };
            for (; t0 + KY <= nt; t0 += KY) {
                const float *gk = base + S::OFF_K + 4 * r + t0 * NP;
                const float *gv = base + S::OFF_V + t0 * RB + i;
                const float *gs = base + t0;
                auto load = [&](int kk) __attribute__((always_inline)) {
                    Tok o;
                    lds_groups<R, J>(o.kv, gk + kk * NP);
                    lds_groups<R, J>(o.qv, gk + (S::OFF_Q - S::OFF_K) + kk * NP);
                    o.decay = gs[S::OFF_DECAY + kk];
                    o.beta = gs[S::OFF_BETA + kk];
                    o.qk = gs[S::OFF_QK + kk];
                    o.v = gv[kk * RB];
                    return o;
                };
                Tok in[2];
                in[0] = load(0);
#pragma unroll
                for (int kk = 0; kk < KY; ++kk) {
                    if (kk + 1 < KY) in[(kk + 1) & 1] = load(kk + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    const Tok &o = in[kk & 1];
                    const float yv = token(o.kv, o.qv, o.decay, o.beta, o.qk, o.v);
                    if constexpr (SNAP) snapshot(chunk_t0 + t0 + kk);
                    y_keep = (rk == kk) ? yv : y_keep;
                }
                Ys[(t0 + rk) * S::YR] = y_keep;
            }
            if (t0 < nt) {
                for (int tt = t0; tt < nt; ++tt) {
                    const float yv = token_y(base, tt);
                    y_keep = (rk == tt - t0) ? yv : y_keep;
                }
                if (rk < nt - t0) Ys[(t0 + rk) * S::YR] = y_keep;
            }
        };
        auto flush_y = [&](int buf, int t0, int nt) {
            const float *Ys = lds + buf * S::BUF + S::OFF_Y;
            if constexpr (VEC) {
                for (int q = tid; q < nt * (RB / 4); q += kThreads) {
                    const int tt = q / (RB / 4);
                    const int pi = 4 * (q - tt * (RB / 4));
                    if (pi < rows_valid)
                        *reinterpret_cast<f4 *>(a.y + (int64_t(t0 + tt) * Hv + vh) * Dv + p0 + pi) =
                            *reinterpret_cast<const f4 *>(Ys + tt * S::YR + pi);
                }
            } else {
                for (int q = tid; q < nt * RB; q += kThreads) {
                    const int tt = q / RB;
                    const int pi = q - tt * RB;
                    if (pi < rows_valid) a.y[(int64_t(t0 + tt) * Hv + vh) * Dv + p0 + pi] = Ys[tt * S::YR + pi];
                }
            }
        };

        // ---- chunks, double-buffered: prefetch chunk c+1 into registers,
        // write out chunk c-1's y, compute chunk c, stage chunk c+1.
        const int n_chunks = (n_tok + CT - 1) / CT;
        if (n_chunks > 0) {
            issue_loads(t_begin, min(CT, n_tok));
            commit(0);
        }
        __syncthreads();
        for (int c = 0; c < n_chunks; ++c) {
            const int buf = c & 1;
            const int t0 = t_begin + c * CT;
            const int nt = min(CT, t_end - t0);
            const bool has_next = c + 1 < n_chunks;
            qk_pass(buf);
            if (has_next) issue_loads(t0 + CT, min(CT, t_end - t0 - CT));
            if (c > 0) flush_y(buf ^ 1, t0 - CT, CT);    // previous chunk, always full
            __syncthreads();                             // k . q of this chunk is staged
            chunk_t0 = t0;
            compute(buf, nt);
            if (has_next) commit(buf ^ 1);
            __syncthreads();
        }
        if (n_chunks > 0) {
            const int c = n_chunks - 1;
            flush_y(c & 1, t_begin + c * CT, n_tok - c * CT);
        }
    }

    // ---- registers -> state slot
    store_row(st_row, true);
}

}  // namespace ssm
