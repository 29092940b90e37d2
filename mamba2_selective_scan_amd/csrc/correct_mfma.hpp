// correct_mfma.hpp -- the correction pass of the time-split prefill on the
// matrix cores.
//
// For a time segment k >= 1 of a split sequence and head h, the segment scan
// started from zero, so the state carried into the segment, carry[p][n], is
// still missing from its y.  Its contribution to token t is
//     y[t][h][p] += dcum(t) * sum_n C[t][g][n] * carry[p][n]
// with dcum(t) the product of dA from the segment start through t (recorded by
// the segment scan).  Over a segment this is a dense
// fp32 contraction [tokens x N] x [N x P], done here with
// v_mfma_f32_32x32x2f32: each wavefront owns a tile of 32 tokens x 32 rows.
//
// Operand layout (checked on gfx950 with an in-bounds probe): A[i][k] is lane
// i + 32k, B[k][j] is lane j + 32k, and accumulator register v of lane l holds
// D[8(v/4) + 4(l/32) + v%4][l%32].  The contraction index n is permuted so that
// MFMA step s, lane half q covers n = q*N/2 + s: every lane then loads one
// contiguous run of N/2 floats of its token's C row (A operand) and of its
// row's carry (B operand) with float4 loads straight from global memory.
#pragma once

#include "scan_kernel.hpp"

namespace ssm {

using f16v = float __attribute__((ext_vector_type(16)));

// KH >= N/2 MFMA steps (N % 8 == 0, vector path).  Grid: n_seqs x n_segs x H x
// n_tblocks workgroups of 4 wavefronts; workgroup b of a segment takes token
// tiles b*4 + w, stepping by n_tblocks*4 tiles until the segment ends.
template <int KH>
__global__ void __launch_bounds__(kThreads) correct_mfma_kernel(ScanArgs a, int n_tblocks) {
    int q = blockIdx.x;
    const int tb = q % n_tblocks;
    q /= n_tblocks;
    const int hd = q % a.H;
    q /= a.H;
    const int seg = q % a.n_segs;
    const int s = q / a.n_segs;
    if (seg == 0) return;                              // segment 0 started from the true state
    const SegRange sr = segment_range(a, s, seg);
    if (seg >= sr.n_real) return;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int li = lane & 31, half = lane >> 5;
    const int H = a.H, P = a.P, N = a.N, G = a.G;
    const int g = hd / a.heads_per_group;
    const int nh = N / 2;
    const int64_t hpn = int64_t(H) * P * N;
    // the state carried into this segment (left in entry seg-1 by the combine pass)
    const float *carry = a.ws_state + (int64_t(s) * a.n_segs + seg - 1) * hpn + int64_t(hd) * P * N;
    const int stride = n_tblocks * 4 * 32;

    for (int t0 = sr.t_begin + (tb * 4 + w) * 32; t0 < sr.t_end; t0 += stride) {
        const int t = t0 + li;
        const bool tok_ok = t < sr.t_end;
        // A operand: this lane's token row of C, n in [half*nh, half*nh + nh)
        float av[KH];
        {
            const float *crow = a.C + (int64_t(t) * G + g) * N + half * nh;
#pragma unroll
            for (int j = 0; j < KH / 4; ++j) {
                const f4 v = (tok_ok && 4 * j < nh) ? *reinterpret_cast<const f4 *>(crow + 4 * j)
                                                    : f4{0.f, 0.f, 0.f, 0.f};
                av[4 * j + 0] = v.x; av[4 * j + 1] = v.y; av[4 * j + 2] = v.z; av[4 * j + 3] = v.w;
            }
        }
        // dcum for the tile's tokens, left by the segment scan
        const float dcum = tok_ok ? a.ws_dcum[int64_t(t) * H + hd] : 0.f;

        for (int p0 = 0; p0 < P; p0 += 32) {
            const int p = p0 + li;
            const bool row_ok = p < P;
            float bv[KH];
            {
                const float *krow = carry + int64_t(p) * N + half * nh;
#pragma unroll
                for (int j = 0; j < KH / 4; ++j) {
                    const f4 v = (row_ok && 4 * j < nh) ? *reinterpret_cast<const f4 *>(krow + 4 * j)
                                                        : f4{0.f, 0.f, 0.f, 0.f};
                    bv[4 * j + 0] = v.x; bv[4 * j + 1] = v.y; bv[4 * j + 2] = v.z; bv[4 * j + 3] = v.w;
                }
            }
            f16v acc = {};
#pragma unroll
            for (int k = 0; k < KH; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[k], bv[k], acc, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = 8 * (v / 4) + 4 * half + (v % 4);     // token within the tile
                const float dc = __shfl(dcum, i, 64);
                if (row_ok && t0 + i < sr.t_end) {
                    float *yp = a.y + (int64_t(t0 + i) * H + hd) * P + p;
                    *yp += dc * acc[v];
                }
            }
        }
    }
}

}  // namespace ssm
