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
// One workgroup per (sequence, time segment, head, block of 64 rows): its four
// wavefronts own 16 rows each.  B, C and x of a chunk are staged in LDS,
// double-buffered (rows padded so the strided state-update reads are
// conflict-free), the per-token scalars are formed once in wave 0.  The kernel
// leaves exactly what the register segment scan leaves: y of the segment, the
// segment's end state (workspace entry, or the slot when the sequence was not
// cut), the running decay product per token and the segment total.
#pragma once

#include "scan_kernel.hpp"

namespace ssm {

using f4m = float __attribute__((ext_vector_type(4)));

template <int NT>                       // N = 16 * NT state elements
struct SsdShape {
    static constexpr int N = 16 * NT;
    static constexpr int CT = 16;                   // tokens per chunk
    static constexpr int RBW = 64;                  // rows per workgroup (4 waves x 16)
    static constexpr int LDN = N + 4;               // padded LDS row of B / C
    static constexpr int OFF_C = 0;
    static constexpr int OFF_B = OFF_C + CT * LDN;
    static constexpr int OFF_X = OFF_B + CT * LDN;  // x[CT][64]
    static constexpr int OFF_S = OFF_X + CT * RBW;  // S_t
    static constexpr int OFF_DT = OFF_S + CT;       // dt_t (0 past the segment)
    static constexpr int OFF_ES = OFF_DT + CT;      // e^{S_t}
    static constexpr int OFF_W = OFF_ES + CT;       // e^{S_15 - S_t} dt_t
    static constexpr int OFF_E15 = OFF_W + CT;      // e^{S_15}
    static constexpr int BUF = ((OFF_E15 + 1) + 3) / 4 * 4;
    static constexpr int U_BC = (CT * N / 4 + kThreads - 1) / kThreads;    // float4 units of B (and of C)
    static constexpr int U_X = (CT * RBW / 4 + kThreads - 1) / kThreads;   // float4 units of x
    static constexpr int lds_floats() { return 2 * BUF; }
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

// Grid: n_seqs x n_segs x H x ceil(P / 64) workgroups (a.n_row_blocks = ceil(P/64),
// a.n_blocks their product), XCD-contiguous order as the register kernel's.
// Requires the vector path (16-byte aligned arrays), N = 16 * NT, P % 16 == 0.
template <int NT>
__global__ void __launch_bounds__(kThreads) ssd_segscan_kernel(ScanArgs a) {
    using S = SsdShape<NT>;
    constexpr int N = S::N, CT = S::CT, LDN = S::LDN;
    extern __shared__ float4 lds_raw[];
    float *const lds = reinterpret_cast<float *>(lds_raw);

    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    const int L = (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int rbw = L % a.n_row_blocks;
    const int hd = (L / a.n_row_blocks) % a.H;
    const int seg = (L / (a.n_row_blocks * a.H)) % a.n_segs;
    const int s = L / (a.n_row_blocks * a.H * a.n_segs);

    const int H = a.H, P = a.P, G = a.G;
    const int g = hd / a.heads_per_group;
    const SegRange sr = segment_range(a, s, seg);
    if (seg >= sr.n_real) return;                    // the sequence is shorter
    const int t_begin = sr.t_begin, t_end = sr.t_end;
    const int n_tok = t_end - t_begin;
    const bool split = sr.n_real > 1;
    const bool fresh = seg > 0 || a.fresh[s] != 0;   // later segments start from zero
    if (!split && !fresh && n_tok <= 0) return;      // empty resume: slot unchanged

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int tl = lane & 15, kq = lane >> 4;        // lane % 16, lane / 16
    const int prow0 = rbw * S::RBW;                  // first row of the workgroup
    const int p0 = prow0 + 16 * w;                   // first row of this wave
    const bool wave_ok = p0 < P;                     // P % 16 == 0: whole wave tiles
    const int64_t hpn = int64_t(H) * P * N;
    float *const st_head = a.state + (int64_t(a.slot[s]) * H + hd) * int64_t(P) * N;
    float *const ws_head = a.ws_state + (int64_t(s) * a.n_segs + seg) * hpn + int64_t(hd) * P * N;
    const float A_h = a.A[hd];
    const float bias_h = a.dt_bias ? a.dt_bias[hd] : 0.f;

    // ---- state h^T in accumulators: hacc[nt] register v of lane l holds
    // h[p0 + l%16][16 nt + 4 (l/16) + v]
    f4m hacc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) hacc[nt] = f4m{0.f, 0.f, 0.f, 0.f};
    if (!fresh && wave_ok) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(
                st_head + int64_t(p0 + tl) * N + 16 * nt + 4 * kq));
            hacc[nt] = f4m{v.x, v.y, v.z, v.w};
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    // ---- chunk staging: global -> registers -> LDS (double-buffered)
    f4 pb[S::U_BC], pc[S::U_BC], px[S::U_X];
    float pdt = 0.f;
    auto issue_loads = [&](int t0, int nt_) {
#pragma unroll
        for (int u = 0; u < S::U_BC; ++u) {
            const int q = u * kThreads + tid;                 // unit = (token, 4-group)
            const int tt = q / (N / 4);
            const int n0 = 4 * (q - tt * (N / 4));
            const bool ok = (q < CT * N / 4) && (tt < nt_);
            const int64_t off = (int64_t(t0 + tt) * G + g) * N + n0;
            pb[u] = load4<true>(a.B + off, ok ? 4 : 0);
            pc[u] = load4<true>(a.C + off, ok ? 4 : 0);
        }
#pragma unroll
        for (int u = 0; u < S::U_X; ++u) {
            const int q = u * kThreads + tid;                 // unit = (token, 4 rows)
            const int tt = q / (S::RBW / 4);
            const int pi = 4 * (q - tt * (S::RBW / 4));
            const bool ok = (q < CT * S::RBW / 4) && (tt < nt_) && (prow0 + pi < P);
            px[u] = load4<true>(a.x + (int64_t(t0 + tt) * H + hd) * P + prow0 + pi, ok ? 4 : 0);
        }
        pdt = (tid < nt_) ? dt_transform(a.dt[int64_t(t0 + tid) * H + hd], bias_h, a.dt_softplus)
                          : 0.f;
    };
    float run = 1.f;                                     // wave 0: decay product so far
    auto commit = [&](int buf, int t0, int nt_) {
        float *base = lds + buf * S::BUF;
#pragma unroll
        for (int u = 0; u < S::U_BC; ++u) {
            const int q = u * kThreads + tid;
            if (q < CT * N / 4) {
                const int tt = q / (N / 4);
                const int n0 = 4 * (q - tt * (N / 4));
                *reinterpret_cast<f4 *>(base + S::OFF_B + tt * LDN + n0) = pb[u];
                *reinterpret_cast<f4 *>(base + S::OFF_C + tt * LDN + n0) = pc[u];
            }
        }
#pragma unroll
        for (int u = 0; u < S::U_X; ++u) {
            const int q = u * kThreads + tid;
            if (q < CT * S::RBW / 4) reinterpret_cast<f4 *>(base + S::OFF_X)[q] = px[u];
        }
        if (tid < 64) {                                  // wave 0, all lanes active
            // lanes 0..15 hold the chunk's tokens (0 past the segment end)
            const float dtv = (tid < nt_) ? pdt : 0.f;
            const float Sv = row_prefix_sum(dtv * A_h);
            const float S15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Sv), 15));
            const float eS = expf(Sv);
            const float e15 = expf(S15);
            if (tid < CT) {
                base[S::OFF_S + tid] = Sv;
                base[S::OFF_DT + tid] = dtv;
                base[S::OFF_ES + tid] = eS;
                base[S::OFF_W + tid] = expf(S15 - Sv) * dtv;
            }
            if (tid == 0) base[S::OFF_E15] = e15;
            // a split sequence's segment also leaves the running product for
            // the correction pass (one row block per head)
            if (split && rbw == 0 && tid < nt_) a.ws_dcum[int64_t(t0 + tid) * H + hd] = run * eS;
            run *= e15;
        }
    };

    auto compute = [&](int buf, int t0, int nt_) {
        if (!wave_ok) return;
        const float *base = lds + buf * S::BUF;
        // per-lane scalars: own token t = l%16; rows s = 4(l/16) + v
        const float S_t = base[S::OFF_S + tl];
        float Ss[4], dts[4], eSr[4], wq[4], xr[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int sv = 4 * kq + v;
            Ss[v] = base[S::OFF_S + sv];
            dts[v] = base[S::OFF_DT + sv];
            eSr[v] = base[S::OFF_ES + sv];
            wq[v] = base[S::OFF_W + sv];
            xr[v] = base[S::OFF_X + sv * S::RBW + 16 * w + tl];
        }
        const float e15 = base[S::OFF_E15];
        // operands: C and B rows of token l%16, n = 16 nt + 4 (l/16) + v
        f4 creg[NT], breg[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            creg[nt] = *reinterpret_cast<const f4 *>(base + S::OFF_C + tl * LDN + 16 * nt + 4 * kq);
            breg[nt] = *reinterpret_cast<const f4 *>(base + S::OFF_B + tl * LDN + 16 * nt + 4 * kq);
        }
        // G^T = B C^T and Y = C h^T, interleaved (independent chains)
        f4m gacc = {0.f, 0.f, 0.f, 0.f}, yacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            gacc = mfma16(breg[nt].x, creg[nt].x, gacc);
            yacc = mfma16(creg[nt].x, hacc[nt][0], yacc);
            gacc = mfma16(breg[nt].y, creg[nt].y, gacc);
            yacc = mfma16(creg[nt].y, hacc[nt][1], yacc);
            gacc = mfma16(breg[nt].z, creg[nt].z, gacc);
            yacc = mfma16(creg[nt].z, hacc[nt][2], yacc);
            gacc = mfma16(breg[nt].w, creg[nt].w, gacc);
            yacc = mfma16(creg[nt].w, hacc[nt][3], yacc);
        }
        // G'^T[s][t] = G^T[s][t] e^{S_t - S_s} dt_s for s <= t, else 0
        // (lane l, register v: s = 4(l/16) + v, t = l%16); Y rows t = 4(l/16) + v
        // take the carried-in state's decay e^{S_t}
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int sv = 4 * kq + v;
            gacc[v] = (sv <= tl) ? gacc[v] * expf(S_t - Ss[v]) * dts[v] : 0.f;
            yacc[v] *= eSr[v];
        }
        // Y += G' X
#pragma unroll
        for (int v = 0; v < 4; ++v) yacc = mfma16(gacc[v], xr[v], yacc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 4 * kq + v;
            if (tt < nt_) a.y[(int64_t(t0 + tt) * H + hd) * P + p0 + tl] = yacc[v];
        }
        // h^T = e^{S_15} h^T + B^T (w X): tile nt, step q, lane l: A = B[4(l/16)+q][16 nt + l%16],
        // B operand = w_s x[s][p] with s = 4(l/16) + q
        float wx[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) wx[q] = wq[q] * xr[q];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) hacc[nt] *= e15;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                hacc[nt] = mfma16(base[S::OFF_B + (4 * kq + q) * LDN + 16 * nt + tl], wx[q], hacc[nt]);
        }
    };

    const int n_chunks = (n_tok + CT - 1) / CT;
    if (n_chunks > 0) {
        issue_loads(t_begin, min(CT, n_tok));
        commit(0, t_begin, min(CT, n_tok));
    }
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        const int t0 = t_begin + c * CT;
        const int nt_ = min(CT, t_end - t0);
        const bool has_next = c + 1 < n_chunks;
        if (has_next) issue_loads(t0 + CT, min(CT, t_end - t0 - CT));
        compute(buf, t0, nt_);
        if (has_next) commit(buf ^ 1, t0 + CT, min(CT, t_end - t0 - CT));
        __syncthreads();
    }
    // a split sequence's segment records its total decay once per head
    if (split && rbw == 0 && tid == 0) a.ws_dtot[(int64_t(s) * a.n_segs + seg) * H + hd] = run;

    // ---- h^T -> the segment's workspace entry (or the slot if not split)
    if (wave_ok) {
        float *dst = split ? ws_head : st_head;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            __builtin_nontemporal_store(f4{hacc[nt][0], hacc[nt][1], hacc[nt][2], hacc[nt][3]},
                                        reinterpret_cast<f4 *>(dst + int64_t(p0 + tl) * N + 16 * nt + 4 * kq));
    }
}

}  // namespace ssm
