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
    int32_t n_blocks;            // n_seqs * H * n_row_blocks
};

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
    // One staging buffer, in floats: B[CT][NP] C[CT][NP] x[CT][RB] y[CT][RB] dt[CT] dA[CT]
    static constexpr int OFF_B = 0;
    static constexpr int OFF_C = OFF_B + CT * NP;
    static constexpr int OFF_X = OFF_C + CT * NP;
    static constexpr int OFF_Y = OFF_X + CT * RB;
    static constexpr int OFF_DT = OFF_Y + CT * RB;
    static constexpr int OFF_DA = OFF_DT + CT;
    static constexpr int BUF = ((OFF_DA + CT) + 3) / 4 * 4;
    static constexpr int TILE = RB * NPT;           // state tile (scalar path), floats
    // register prefetch units per thread
    static constexpr int U_BC = (CT * NP / 4 + kThreads - 1) / kThreads;    // float4 of B (and of C)
    static constexpr int U_X = (CT * RB / 4 + kThreads - 1) / kThreads;     // float4 of x
    static_assert(R == 4 || R == 8 || R == 16 || R == 32 || R == 64, "R must be a power of two in [4, 64]");
    static_assert(CT <= kThreads, "one thread stages each token's dt");
    static_assert(RB % 4 == 0, "rows per block must be a multiple of 4");

    static constexpr int lds_floats(bool decode, bool vec) {
        const int staging = decode ? 0 : 2 * BUF;   // decode reads its one token from global
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
        hj[0] = hj[0] * dA + b[j].x * x_dt;
        hj[1] = hj[1] * dA + b[j].y * x_dt;
        hj[2] = hj[2] * dA + b[j].z * x_dt;
        hj[3] = hj[3] * dA + b[j].w * x_dt;
        acc0 += hj[0] * c[j].x;
        acc1 += hj[1] * c[j].y;
        acc0 += hj[2] * c[j].z;
        acc1 += hj[3] * c[j].w;
    }
    return acc0 + acc1;
}

// The lane's J 4-groups of one token's B (or C) row in LDS; p points at the
// lane's first group, groups are 4*R floats apart.
template <int R, int J>
__device__ __forceinline__ void lds_groups(f4 (&v)[J], const float *p) {
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = *reinterpret_cast<const f4 *>(p + 4 * R * j);
}

template <class S, bool VEC, bool DECODE>
__global__ void __launch_bounds__(kThreads) scan_kernel(ScanArgs a) {
    extern __shared__ float4 lds_raw[];
    float *const lds = reinterpret_cast<float *>(lds_raw);

    constexpr int R = S::R, J = S::J, E = S::E, CT = S::CT, NP = S::NP, RB = S::RB;

    // ---- workgroup -> (sequence, head, row block); XCD-contiguous order
    const int bid = blockIdx.x;
    const int nb = a.n_blocks;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, k = bid / kXcds;
    const int L = (xcd < rem) ? xcd * (per + 1) + k : rem * (per + 1) + (xcd - rem) * per + k;
    const int rb = L % a.n_row_blocks;
    const int hd = (L / a.n_row_blocks) % a.H;
    const int s = L / (a.n_row_blocks * a.H);

    const int H = a.H, P = a.P, N = a.N, G = a.G;
    const int g = hd / a.heads_per_group;
    const int t_begin = DECODE ? s : a.cu_seqlens[s];
    const int t_end = DECODE ? s + 1 : a.cu_seqlens[s + 1];
    const int n_tok = t_end - t_begin;
    const bool fresh = a.fresh[s] != 0;
    if (!fresh && n_tok <= 0) return;               // resume with no tokens: slot unchanged

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = (tid >> 6) * S::ROWS_PER_WAVE + lane / R;   // row within the block
    const int r = lane % R;                                    // lane within the row
    const int p0 = rb * RB;
    const int rows_valid = min(RB, P - p0);
    const bool row_ok = i < rows_valid;
    float *const st_block = a.state + ((int64_t(a.slot[s]) * H + hd) * P + p0) * int64_t(N);
    const float A_h = a.A[hd];

    // ---- state -> registers
    float h[E];
#pragma unroll
    for (int e = 0; e < E; ++e) h[e] = 0.f;
    if (!fresh) {
        if constexpr (VEC) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int n0 = 4 * (j * R + r);
                if (row_ok && n0 < N) {
                    const f4 v = __builtin_nontemporal_load(
                        reinterpret_cast<const f4 *>(st_block + int64_t(i) * N + n0));
                    h[4 * j + 0] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
                }
            }
        } else {
            // coalesced LDS tile: one linear sweep over the block's contiguous rows
            const int total = rows_valid * N;
            for (int q = tid; q < total; q += kThreads) {
                const int row = q / N;
                lds[row * S::NPT + (q - row * N)] = st_block[q];
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
        const float dt = a.dt[int64_t(s) * H + hd];
        const float x = row_ok ? a.x[(int64_t(s) * H + hd) * P + p0 + i] : 0.f;
        const float dA = expf(dt * A_h);
        const float yv = row_allreduce<R>(update_token<J>(h, bl, cl, dA, x * dt));
        if (r == 0 && row_ok) a.y[(int64_t(s) * H + hd) * P + p0 + i] = yv;
    } else {
        // All state loads are complete before the chunk pipeline starts, so the
        // token loop never waits on the next chunk's prefetch.
        __builtin_amdgcn_s_waitcnt(0);

        // ---- chunk staging: global -> registers -> LDS
        f4 pb[S::U_BC], pc[S::U_BC], px[S::U_X];
        float pdt = 0.f;

        auto issue_loads = [&](int t0, int nt) {
#pragma unroll
            for (int u = 0; u < S::U_BC; ++u) {
                const int q = u * kThreads + tid;                 // unit = (token, 4-group)
                const int tt = q / (NP / 4);
                const int n0 = 4 * (q - tt * (NP / 4));
                const bool ok = (q < CT * NP / 4) && (tt < nt);
                const int64_t off = (int64_t(t0 + tt) * G + g) * N + n0;
                const int nv = ok ? clamp4(N - n0) : 0;
                pb[u] = load4<VEC>(a.B + off, nv);
                pc[u] = load4<VEC>(a.C + off, nv);
            }
#pragma unroll
            for (int u = 0; u < S::U_X; ++u) {
                const int q = u * kThreads + tid;                 // unit = (token, 4 rows)
                const int tt = q / (RB / 4);
                const int pi = 4 * (q - tt * (RB / 4));
                const bool ok = (q < CT * RB / 4) && (tt < nt);
                const int nv = ok ? clamp4(rows_valid - pi) : 0;
                px[u] = load4<VEC>(a.x + (int64_t(t0 + tt) * H + hd) * P + p0 + pi, nv);
            }
            pdt = (tid < nt) ? a.dt[int64_t(t0 + tid) * H + hd] : 0.f;
        };

        auto commit = [&](int buf) {
            float *base = lds + buf * S::BUF;
            f4 *Bs4 = reinterpret_cast<f4 *>(base + S::OFF_B);
            f4 *Cs4 = reinterpret_cast<f4 *>(base + S::OFF_C);
            f4 *Xs4 = reinterpret_cast<f4 *>(base + S::OFF_X);
#pragma unroll
            for (int u = 0; u < S::U_BC; ++u) {
                const int q = u * kThreads + tid;
                if (q < CT * NP / 4) { Bs4[q] = pb[u]; Cs4[q] = pc[u]; }
            }
#pragma unroll
            for (int u = 0; u < S::U_X; ++u) {
                const int q = u * kThreads + tid;
                if (q < CT * RB / 4) Xs4[q] = px[u];
            }
            if (tid < CT) {
                base[S::OFF_DT + tid] = pdt;
                base[S::OFF_DA + tid] = expf(pdt * A_h);
            }
        };

        // Tokens go in groups of KY.  Every lane of a row ends a token with the
        // row's y; lane r keeps the y of the group's token r % KY and stores it
        // once per group, so the per-token cost is one select.  Inside a group
        // the token index is a compile-time constant: LDS offsets fold into the
        // instructions and the keep-select needs no runtime compare.
        constexpr int KY = R < 16 ? R : 16;
        const int rk = r % KY;
        auto compute = [&](int buf, int nt) {
            const float *base = lds + buf * S::BUF;
            const float *Bl = base + S::OFF_B + 4 * r;
            const float *Cl = base + S::OFF_C + 4 * r;
            const float *Xl = base + S::OFF_X + i;
            const float *Dt = base + S::OFF_DT;
            const float *Da = base + S::OFF_DA;
            float *Ys = lds + buf * S::BUF + S::OFF_Y + i;
            float y_keep = 0.f;
            int t0 = 0;
            for (; t0 + KY <= nt; t0 += KY) {
#pragma unroll
                for (int kk = 0; kk < KY; ++kk) {
                    const int tt = t0 + kk;
                    f4 bv[J], cv[J];
                    lds_groups<R, J>(bv, Bl + tt * NP);
                    lds_groups<R, J>(cv, Cl + tt * NP);
                    const float yv =
                        row_allreduce<R>(update_token<J>(h, bv, cv, Da[tt], Xl[tt * RB] * Dt[tt]));
                    y_keep = (rk == kk) ? yv : y_keep;
                }
                Ys[(t0 + rk) * RB] = y_keep;
            }
            if (t0 < nt) {
                for (int tt = t0; tt < nt; ++tt) {
                    f4 bv[J], cv[J];
                    lds_groups<R, J>(bv, Bl + tt * NP);
                    lds_groups<R, J>(cv, Cl + tt * NP);
                    const float yv =
                        row_allreduce<R>(update_token<J>(h, bv, cv, Da[tt], Xl[tt * RB] * Dt[tt]));
                    y_keep = (rk == tt - t0) ? yv : y_keep;
                }
                if (rk < nt - t0) Ys[(t0 + rk) * RB] = y_keep;
            }
        };

        auto flush_y = [&](int buf, int t0, int nt) {
            const float *Ys = lds + buf * S::BUF + S::OFF_Y;
            if constexpr (VEC) {
                for (int q = tid; q < nt * (RB / 4); q += kThreads) {
                    const int tt = q / (RB / 4);
                    const int pi = 4 * (q - tt * (RB / 4));
                    if (pi < rows_valid)
                        *reinterpret_cast<f4 *>(a.y + (int64_t(t0 + tt) * H + hd) * P + p0 + pi) =
                            *reinterpret_cast<const f4 *>(Ys + tt * RB + pi);
                }
            } else {
                for (int q = tid; q < nt * RB; q += kThreads) {
                    const int tt = q / RB;
                    const int pi = q - tt * RB;
                    if (pi < rows_valid) a.y[(int64_t(t0 + tt) * H + hd) * P + p0 + pi] = Ys[tt * RB + pi];
                }
            }
        };

        // ---- token loop, chunk by chunk, double-buffered.  Chunk c's y tile is
        // written out during chunk c+1, after that chunk's prefetch is issued and
        // before its token loop: the stores then drain under the compute, and
        // the registers that carried them are free again by the time they are
        // reused (vector-memory counters on this chip count stores too).
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
            if (has_next) issue_loads(t0 + CT, min(CT, t_end - t0 - CT));
            if (c > 0) flush_y(buf ^ 1, t0 - CT, CT);    // previous chunk, always full
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
    if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n0 = 4 * (j * R + r);
            if (row_ok && n0 < N) {
                const f4 v = {h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
                __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(st_block + int64_t(i) * N + n0));
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
            st_block[q] = lds[row * S::NPT + (q - row * N)];
        }
    }
}

}  // namespace ssm
