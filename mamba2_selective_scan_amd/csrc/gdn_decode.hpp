// gdn_decode.hpp -- the delta rule's decode step (one token per sequence) on
// the vector path, with every load in flight before the first wait.
//
// Like the scan's decode step, a delta-rule decode step is almost nothing but
// the state read and written once per (sequence, value head, row); its time
// is one dependent chain per wavefront (fresh flag and slot, then the state,
// then the arithmetic, then the stores) plus the transfer.  So the token's k,
// q and v are requested together with the fresh flag (the oldest load), the
// decay and beta sit in scalar registers, and the state moves through buffer
// descriptors that are empty for a fresh sequence and clipped to the block's
// valid rows otherwise: no branch, so no wait at a branch join.  The
// arithmetic is gdn_token, the per-token prefill's.  Same lane layout as the
// per-token kernel's decode shape, with workgroups in plain order (as the
// scan's decode step measured faster).  Requires Dk % 4 == 0, Dv % 4 == 0 and
// 16-byte aligned arrays; no snapshots.
#pragma once

#include "buffer_io.hpp"
#include "gdn_kernel.hpp"

namespace ssm {

__device__ __forceinline__ float gdn_uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

template <class S>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
gdn_decode_kernel(GdnArgs a) {
    constexpr int R = S::R, J = S::J, E = S::E, RB = S::RB;
    constexpr int kNone = 0x7ffffff0;                // a byte offset past every descriptor
    const int L = blockIdx.x;
    const int rb = L % a.n_row_blocks;
    const int m = (L / a.n_row_blocks) % a.Hv;
    const int s = L / (a.n_row_blocks * a.Hv);       // sequence = its token
    const int kh = m / a.heads_per_key;
    const int vh = (m % a.heads_per_key) * a.Hk + kh;        // key head of vh is vh % Hk
    const int Hv = a.Hv, Hk = a.Hk, Dk = a.Dk, Dv = a.Dv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = (tid >> 6) * S::ROWS_PER_WAVE + lane / R;   // row within the block
    const int r = lane % R;                                    // lane within the row
    const int p0 = rb * RB;
    const int rows_valid = min(RB, Dv - p0);

    // 1. the fresh flag, then the token's operands (none depends on the slot)
    const int fresh = buffer_load_u8(a.fresh, s + 1, s);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t kq_off = (int64_t(s) * Hk + kh) * Dk;
    const __amdgpu_buffer_rsrc_t rk = buffer_of(a.k + kq_off, Dk * int(sizeof(float)));
    const __amdgpu_buffer_rsrc_t rq = buffer_of(a.q + kq_off, Dk * int(sizeof(float)));
    f4 kv[J], qv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int vo = (4 * r + 4 * R * j) * int(sizeof(float));     // past Dk: zeros
        kv[j] = buffer_load<4>(rk, vo, 0);
        qv[j] = buffer_load<4>(rq, vo, 0);
    }
    const int64_t row0 = (int64_t(s) * Hv + vh) * Dv + p0;   // v and y of the block's first row
    const __amdgpu_buffer_rsrc_t rv = buffer_of(a.v + row0, rows_valid * int(sizeof(float)));
    const float vr = buffer_load<1>(rv, i * int(sizeof(float)), 0);
    const float decay = gdn_uniform(expf(a.g[int64_t(s) * Hv + vh]));
    const float beta = gdn_uniform(a.beta[int64_t(s) * Hv + vh]);
    int vo_s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int n0 = 4 * (j * R + r);
        vo_s[j] = n0 < Dk ? (i * Dk + n0) * int(sizeof(float)) : kNone;
    }

    // 2. the state: an empty descriptor when the sequence is fresh
    float *const st_block = a.state + ((int64_t(a.slot[s]) * Hv + vh) * Dv + p0) * int64_t(Dk);
    const int st_bytes = rows_valid * Dk * int(sizeof(float));
    const __amdgpu_buffer_rsrc_t rs_in = buffer_of(st_block, __builtin_amdgcn_readfirstlane(fresh) ? 0 : st_bytes);
    float h[E];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const f4 v = buffer_load4_nt(rs_in, vo_s[j]);
        h[4 * j + 0] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
    }

    // 3. the token: k . q from the row's lanes, then the update
    float kq0 = 0.f, kq1 = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        kq0 = __builtin_fmaf(kv[j].x, qv[j].x, kq0);
        kq1 = __builtin_fmaf(kv[j].y, qv[j].y, kq1);
        kq0 = __builtin_fmaf(kv[j].z, qv[j].z, kq0);
        kq1 = __builtin_fmaf(kv[j].w, qv[j].w, kq1);
    }
    const float qk = row_allreduce<R>(kq0 + kq1);
    const float yv = gdn_token<R, J>(h, kv, qv, decay, beta, qk, vr, a.scale);

    // 4. y from each row's first lane, the state back to the slot
    const __amdgpu_buffer_rsrc_t ry = buffer_of(a.y + row0, rows_valid * int(sizeof(float)));
    if (r == 0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), ry, i * int(sizeof(float)), 0, 0);
    const __amdgpu_buffer_rsrc_t rs_out = buffer_of(st_block, st_bytes);
#pragma unroll
    for (int j = 0; j < J; ++j)
        buffer_store4_nt(f4{h[4 * j + 0], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]}, rs_out, vo_s[j]);
}

}  // namespace ssm
