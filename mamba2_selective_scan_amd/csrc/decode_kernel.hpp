// decode_kernel.hpp -- the decode step (one token per sequence) on the vector
// path, with every load in flight before the first wait.
//
// A decode step is almost nothing but state traffic: each (sequence, head,
// row)'s N values are read once and written once ("perf(cuda): keep the Mamba2
// scan state in registers, stage tokens by chunk #90", How the layout was
// chosen).  The step is one dependent chain per wavefront -- fresh flag and
// slot, then the state, then the arithmetic, then the stores -- and with every
// wavefront of the grid resident at once the kernel's time is that chain's
// latency plus the transfer.  So nothing waits that need not:
//  * the token's B and C rows, x and dt do not depend on the slot, so they
//    are requested first, together with the fresh flag (oldest, so waiting
//    for it waits for nothing else); B and C are loaded once per workgroup
//    (a float4 or two per thread) and shared through LDS, behind a barrier
//    that waits under the state loads' latency -- every lane loading its own
//    J groups of both put eight times the state's load instructions through
//    the texture path (13.2-13.5 against 13.1-13.2 us at 16 x 1);
//  * the state is read through a buffer descriptor that is empty for a fresh
//    sequence (those loads return zeros and touch no memory) and covers only
//    the block's valid rows otherwise, and written through one that covers
//    the valid rows: no branch, so no wait at a branch join.
// The arithmetic is the scan kernel's update_token, so the state after a
// decode step is bit for bit the state after a one-token prefill.  Same grid
// and lane layout as the scan kernel's decode shape: one workgroup of four
// wavefronts per (sequence, head, RB rows), R lanes per row, E = 4J state
// values per lane.  Requires N % 4 == 0,
// P % 4 == 0 and 16-byte aligned arrays; no A per state, no snapshots.
#pragma once

#include "buffer_io.hpp"
#include "scan_kernel.hpp"

namespace ssm {

// A wave-uniform float moved to a scalar register (bit for bit).
__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Eight wavefronts per SIMD (at most 64 VGPRs): the decode 16 x 1 grid at
// H 64, P 64 (8192 wavefronts) is then resident in one round.
template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
decode_kernel(ScanArgs a) {
    constexpr int R = S::R, J = S::J, E = S::E, RB = S::RB;
    constexpr int kNone = 0x7ffffff0;               // a byte offset past every descriptor
    // Workgroups in plain order: consecutive ids (dealt round-robin over the
    // XCDs) take consecutive 16 KB runs of the slots.  The prefill kernels'
    // XCD-contiguous order, which keeps a B/C group in one L2, measured 3%
    // slower here (13.7 against 13.3 us at 16 x 1, H 64 P 64 N 128), where
    // B and C are a few KB.
    const int L = blockIdx.x;
    const int rb = L % a.n_row_blocks;
    const int hd = (L / a.n_row_blocks) % a.H;
    const int s = L / (a.n_row_blocks * a.H);       // sequence = its token
    const int H = a.H, P = a.P, N = a.N, G = a.G;
    const int g = hd / a.heads_per_group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = (tid >> 6) * S::ROWS_PER_WAVE + lane / R;   // row within the block
    const int r = lane % R;                                    // lane within the row
    const int p0 = rb * RB;
    const int rows_valid = min(RB, P - p0);

    // 1. the fresh flag, then the token's operands (none depends on the slot)
    const int fresh = buffer_load_u8(a.fresh, s + 1, s);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t bc = (int64_t(s) * G + g) * N;
    const __amdgpu_buffer_rsrc_t rbv = buffer_of(a.B + bc, N * int(sizeof(float)));
    const __amdgpu_buffer_rsrc_t rcv = buffer_of(a.C + bc, N * int(sizeof(float)));
    // B and C rows as NU float4 units, B's R J then C's: unit q of the
    // workgroup is thread q % kThreads's load q / kThreads; groups past N fall
    // past the descriptor (zeros); every thread issues UPT loads
    constexpr int RJ = R * J, NU = 2 * RJ;
    constexpr int UPT = (NU + kThreads - 1) / kThreads;
    __shared__ f4 bc_lds[NU];
    f4 bcv[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const int q = u * kThreads + tid;
        const bool is_c = q >= RJ;
        const int uq = is_c ? q - RJ : q;
        bcv[u] = buffer_load<4>(is_c ? rcv : rbv, q < NU ? uq * int(sizeof(f4)) : kNone, 0);
    }
    // state: rows past the block's valid ones land past the state descriptors;
    // a group past N would land in the next row, so it gets an offset past all
    int vo_s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int n0 = 4 * (j * R + r);
        vo_s[j] = n0 < N ? (i * N + n0) * int(sizeof(float)) : kNone;
    }
    const int64_t row0 = (int64_t(s) * H + hd) * P + p0;       // x and y of the block's first row
    const __amdgpu_buffer_rsrc_t rx = buffer_of(a.x + row0, rows_valid * int(sizeof(float)));
    const float xv = buffer_load<1>(rx, i * int(sizeof(float)), 0);
    // dt and dA are the workgroup's (scalar loads): formed before the state
    // loads and kept in scalar registers, so their arithmetic neither waits
    // on a vector load nor holds vector registers beside the state
    const float dt = uniform(
        dt_transform(a.dt[int64_t(s) * H + hd], a.dt_bias ? a.dt_bias[hd] : 0.f, a.dt_softplus));
    const float dA = uniform(expf(dt * a.A[hd]));

    // 2. the state: an empty descriptor when the sequence is fresh
    float *const st_block = a.state + ((int64_t(a.slot[s]) * H + hd) * P + p0) * int64_t(N);
    const int st_bytes = rows_valid * N * int(sizeof(float));
    const __amdgpu_buffer_rsrc_t rs_in = buffer_of(st_block, __builtin_amdgcn_readfirstlane(fresh) ? 0 : st_bytes);
    float h[E];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const f4 v = buffer_load4_nt(rs_in, vo_s[j]);
        h[4 * j + 0] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
    }

    // B and C meet in LDS while the state is in flight
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const int q = u * kThreads + tid;
        if (q < NU) bc_lds[q] = bcv[u];
    }
    __syncthreads();
    f4 bl[J], cl[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        bl[j] = bc_lds[R * j + r];
        cl[j] = bc_lds[RJ + R * j + r];
    }

    // 3. the token
    const float part = update_token<J>(h, bl, cl, dA, xv * dt);
    const float yv = row_allreduce<R>(part);

    // 4. y from each row's first lane, the state back to the slot
    const __amdgpu_buffer_rsrc_t ry = buffer_of(a.y + row0, rows_valid * int(sizeof(float)));
    if (r == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), ry, i * int(sizeof(float)), 0, 0);
    const __amdgpu_buffer_rsrc_t rs_out = buffer_of(st_block, st_bytes);
#pragma unroll
    for (int j = 0; j < J; ++j)
        buffer_store4_nt(f4{h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]}, rs_out, vo_s[j]);
}

}  // namespace ssm
