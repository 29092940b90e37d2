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

// KH >= N/2 MFMA steps (N % 8 == 0, vector path), taken in chunks of KC = 16:
// a chunk's C and carry operands are 4 float4 per lane, and the next chunk's
// loads are in flight while the current chunk's 16 MFMAs run, instead of the
// wave holding the whole contraction's operands.  Grid: n_seqs x (n_segs - 1) x
// H x n_tblocks workgroups of 4 wavefronts (segments 1 and up); workgroup b of
// a segment takes token tiles b*4 + w, stepping by n_tblocks*4 tiles until the
// segment ends.
// FULL: N/2 == KH, so no chunk reaches past the row and nothing is masked.
template <int KH, bool FULL>
__global__ void __launch_bounds__(kThreads) correct_mfma_kernel(ScanArgs a, int n_tblocks) {
    constexpr int KC = 16;                              // MFMA steps per chunk
    constexpr int NCH = KH / KC;
    static_assert(KH % KC == 0, "whole chunks");
    // XCD-contiguous order (as the scan's): the hardware deals workgroups to
    // the XCDs round robin, so consecutive logical blocks -- the token tiles of
    // one head, then the neighbouring heads that share its C rows -- are given
    // to one XCD and share its L2.
    const int bid = blockIdx.x;
    const int nb = gridDim.x;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int xcd = bid % kXcds, kx = bid / kXcds;
    int q = (xcd < rem) ? xcd * (per + 1) + kx : rem * (per + 1) + (xcd - rem) * per + kx;
    const int tb = q % n_tblocks;
    q /= n_tblocks;
    const int hd = q % a.H;
    q /= a.H;
    // the grid holds segments 1..n_segs-1 only (segment 0 started from the true state)
    const int seg = q % (a.n_segs - 1) + 1;
    const int s = q / (a.n_segs - 1);
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

    // Chunk c of a row: floats [16c, 16c + 16) of the lane's half.  Rows are
    // clamped to valid ones and loaded unmasked: a C row of a token past the
    // segment only feeds output rows that are never stored, a carry row past
    // P only output columns that are never stored.  Past nh (N/2 < KH) the
    // carry is zeroed so the C values there add nothing; every load is still
    // issued (no branch between loads).
    auto load_chunk = [&](f4 (&v)[4], const float *row, bool zero_pad, int c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = KC * c + 4 * j;
            if constexpr (FULL) {
                v[j] = *reinterpret_cast<const f4 *>(row + k);
            } else {
                const f4 x = *reinterpret_cast<const f4 *>(row + min(k, nh - 4));
                const bool good = !zero_pad || k < nh;
                v[j] = f4{good ? x.x : 0.f, good ? x.y : 0.f, good ? x.z : 0.f, good ? x.w : 0.f};
            }
        }
    };

    for (int t0 = sr.t_begin + (tb * 4 + w) * 32; t0 < sr.t_end; t0 += stride) {
        const int tc = min(t0 + li, sr.t_end - 1);                 // a token of this tile
        // A operand: this lane's token row of C, n in [half*nh, half*nh + nh)
        const float *crow = a.C + (int64_t(tc) * G + g) * N + half * nh;
        // dcum for the tile's tokens, left by the segment scan
        const float dcum = a.ws_dcum[int64_t(tc) * H + hd];

        for (int p0 = 0; p0 < P; p0 += 32) {
            const int p = p0 + li;
            const bool row_ok = p < P;
            const int pc = min(p, P - 1);                    // a row of this tile
            const float *krow = carry + int64_t(pc) * N + half * nh;
            // operands in two ping-pong buffers: the loads of chunk c+1 are
            // issued before chunk c's MFMAs (the scheduling barriers keep the
            // compiler from sinking them below the MFMAs, which would leave
            // every chunk waiting on its own loads)
            f4 a0[4], b0[4], a1[4], b1[4];
            load_chunk(a0, crow, false, 0);
            load_chunk(b0, krow, true, 0);
            // the tile's y, read after chunk 0's operands (the memory counter
            // is in order) and before the contraction, which hides them
            // (addresses clamped into this wave's own tile)
            float yv[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = 8 * (v / 4) + 4 * half + (v % 4);     // token within the tile
                yv[v] = a.y[(int64_t(min(t0 + i, sr.t_end - 1)) * H + hd) * P + pc];
            }
            f16v acc = {};
            auto mfma16 = [&](const f4 (&x)[4], const f4 (&y)[4]) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[j].x, y[j].x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[j].y, y[j].y, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[j].z, y[j].z, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[j].w, y[j].w, acc, 0, 0, 0);
                }
            };
#pragma unroll
            for (int c = 0; c < NCH; c += 2) {
                if (c + 1 < NCH) {
                    load_chunk(a1, crow, false, c + 1);
                    load_chunk(b1, krow, true, c + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma16(a0, b0);
                __builtin_amdgcn_sched_barrier(0);
                if (c + 2 < NCH) {
                    load_chunk(a0, crow, false, c + 2);
                    load_chunk(b0, krow, true, c + 2);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (c + 1 < NCH) mfma16(a1, b1);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = 8 * (v / 4) + 4 * half + (v % 4);
                const float dc = __shfl(dcum, i, 64);
                if (row_ok && t0 + i < sr.t_end)
                    a.y[(int64_t(t0 + i) * H + hd) * P + p] = __builtin_fmaf(dc, acc[v], yv[v]);
            }
        }
    }
}

}  // namespace ssm
