// conv_norm.hip -- gfx950 kernels and C ABI (include/ssm_conv_norm.h) for the
// two steps beside the scan in a Mamba2-style layer: causal depthwise conv1d +
// SiLU with a rolling history, and gated RMSNorm.  Both are streaming,
// HBM-bound operations, so the design is about moving each byte once, in whole
// cache lines, with enough loads in flight; neither needs LDS staging.
//
// Causal conv1d + SiLU ("ssm_gated_delta.cu": fc_ssm_conv1d_silu,
// fc_ssm_conv1d_silu_seq and fc_ssm_conv1d_silu_slots).  Foundry runs one
// thread per channel through all positions of one sequence, with the history
// in registers.  At a 4096-token prefill that is only D threads walking 4096
// dependent steps; here the positions of each sequence are cut into chunks of
// kConvChunk tokens and every (chunk, run of channels) is its own workgroup.
// A chunk other than a sequence's first rebuilds its history from the K-1 raw
// inputs just before it (they are inputs, not results, so chunks are
// independent); only the first chunk reads the slot and it alone writes the
// final history back, after its own reads, so no two workgroups touch a slot.
// Each lane owns four adjacent channels (float4 loads and stores across a
// token row: a wavefront moves 1 KB contiguous per instruction) and walks its
// chunk's tokens in order, with four tokens' loads issued ahead of the math.
// (Measured on MI355X at 1 x 4096 tokens, D = 6144: 16-token chunks with
// 4-token batches ran at 34.6 us against 39.8 us for 32 / 4, 43.8 us for
// 32 / 8 and 43.1 us for 64 / 4; nontemporal stores made no difference.)
//
// Workgroups of the packed batch are numbered without any host-side table:
// sequence s owns the workgroups F(s) .. F(s) + chunks(s) - 1 with
// F(s) = s + cu_seqlens[s] / kConvChunk.  F grows by at least chunks(s) from
// one sequence to the next (a zero-length sequence still owns one workgroup,
// which zeroes a fresh slot), so the grid needs n_seqs + n_tokens / kConvChunk
// workgroups and a workgroup finds its sequence by searching F over
// cu_seqlens: all 256 lanes test one candidate each and a ballot count narrows
// the range 256-fold per round (one round for up to 256 sequences).
//
// Gated RMSNorm ("ssm_gated_delta.cu": fc_ssm_gated_norm).  Foundry gives a
// head a 256-thread block and a shared-memory tree with a barrier per level.
// Here a row is 16 adjacent lanes (one DPP row of the wavefront), each lane
// holding float4 pieces of the row in registers; the sum of squares is a
// 4-step DPP butterfly inside those 16 lanes, so there is no LDS and no
// barrier, and a 256-lane workgroup normalises 16 rows at once.
#include "ssm_conv_norm.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "scan_kernel.hpp"
#include "status.hpp"

namespace ssm {
namespace {

constexpr int kConvChunk = 16;     // tokens per conv workgroup
constexpr int kConvBatch = 4;      // token loads issued ahead of the math
constexpr int kNormLanes = 16;     // lanes per normalised row (one DPP row)
constexpr int kNormRows = kThreads / kNormLanes;

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// NF consecutive floats at p: float4 loads when VEC (p 16-byte aligned, NF % 4 == 0).
template <int NF, bool VEC>
__device__ __forceinline__ void load_run(float (&d)[NF], const float *p) {
    if constexpr (VEC) {
        static_assert(NF % 4 == 0, "float4 runs");
#pragma unroll
        for (int i = 0; i < NF / 4; ++i) {
            const f4 v = *reinterpret_cast<const f4 *>(p + 4 * i);
            d[4 * i + 0] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NF; ++i) d[i] = p[i];
    }
}

template <int NF, bool VEC>
__device__ __forceinline__ void store_run(float *p, const float (&d)[NF]) {
    if constexpr (VEC) {
        static_assert(NF % 4 == 0, "float4 runs");
#pragma unroll
        for (int i = 0; i < NF / 4; ++i)
            *reinterpret_cast<f4 *>(p + 4 * i) = f4{d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < NF; ++i) p[i] = d[i];
    }
}

struct ConvArgs {
    const int32_t *cu_seqlens;   // [n_seqs+1]; unused by decode
    const int32_t *slot;         // [n_seqs]
    const uint8_t *fresh;        // [n_seqs]
    const float *x;              // [T][D]
    const float *w;              // [D][K]
    float *state;                // [n_slots][D][K-1]
    float *out;                  // [T][D]
    float *snaps;                // [T][D][K-1] or null
    int D;
    int n_seqs;
};

// Largest s in [0, n_seqs) with s + cu[s] / kConvChunk <= j.  Block-uniform;
// every lane of the workgroup must call it.
__device__ int find_sequence(const int32_t *cu, int n_seqs, int j, int *counts) {
    int lo = 0, hi = n_seqs - 1;                       // F(lo) <= j holds throughout
    while (hi > lo) {
        const int stride = (hi - lo + kThreads) / kThreads;
        const int s = lo + int(threadIdx.x) * stride;
        const bool ok = s <= hi && s + cu[s] / kConvChunk <= j;
        const uint64_t b = __ballot(ok);
        if ((threadIdx.x & 63) == 0) counts[threadIdx.x >> 6] = __popcll(b);
        __syncthreads();
        int k = 0;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) k += counts[wv];
        __syncthreads();
        // F is strictly increasing, so the lanes that passed are a prefix.
        lo += (k - 1) * stride;
        hi = min(hi, lo + stride - 1);
    }
    return lo;
}

// V channels per lane (4: float4 path), KM1 = K-1 history values per channel.
template <int V, int KM1, bool DECODE, bool SNAP>
__global__ void __launch_bounds__(kThreads) conv1d_silu_kernel(ConvArgs a) {
    constexpr int K = KM1 + 1;
    constexpr bool VEC = V == 4;
    constexpr int NH = KM1 > 0 ? V * KM1 : 1;          // history registers (>= 1 for C++)
    __shared__ int counts[kWaves];

    // Plain numbering: consecutive chunks go to different XCDs, so all XCDs
    // stream neighbouring token rows at once.  (Giving each XCD a contiguous
    // run of chunks, so the K-1 inputs a chunk re-reads from its neighbour sit
    // in the same L2, measured slower on MI355X: 37.3 us against 34.5 us at
    // 1 x 4096 tokens, D = 6144.)
    const int unit = int(blockIdx.x);

    int s, c, seq0, len, t0, t1;
    if constexpr (DECODE) {
        s = unit; c = 0; seq0 = s; len = 1; t0 = s; t1 = s + 1;
    } else {
        s = find_sequence(a.cu_seqlens, a.n_seqs, unit, counts);
        seq0 = a.cu_seqlens[s];
        len = a.cu_seqlens[s + 1] - seq0;
        c = unit - (s + seq0 / kConvChunk);
        const int n_chunks = len > 0 ? (len + kConvChunk - 1) / kConvChunk : 1;
        if (c >= n_chunks) return;                      // past this sequence's chunks
        t0 = seq0 + c * kConvChunk;
        t1 = min(t0 + kConvChunk, seq0 + len);
    }
    const int ch = (int(blockIdx.y) * kThreads + int(threadIdx.x)) * V;
    if (ch >= a.D) return;
    const int64_t D = a.D;

    float w[V * K];                                     // w[v*K + k]
    load_run<V * K, VEC>(w, a.w + int64_t(ch) * K);
    // The first batch of inputs is loaded before the history, whose address
    // waits on the slot index (for one-token decode that hides one round trip).
    float xb[kConvBatch][V];
    auto load_batch = [&](int tb) {
#pragma unroll
        for (int u = 0; u < kConvBatch; ++u)
            if (tb + u < t1) load_run<V, VEC>(xb[u], a.x + int64_t(tb + u) * D + ch);
    };
    load_batch(t0);

    float h[NH] = {};                                   // h[v*KM1 + i], oldest first
    const bool owner = c == 0;                          // the slot belongs to chunk 0
    bool fresh = false;
    int slot = 0;
    if (owner) {
        slot = a.slot[s];
        fresh = a.fresh[s] != 0;
        if constexpr (KM1 > 0) {
            if (!fresh) load_run<NH, VEC>(h, a.state + (int64_t(slot) * D + ch) * KM1);
        }
    } else if constexpr (KM1 > 0) {
        // The history at a later chunk's start: the raw inputs just before it.
#pragma unroll
        for (int i = 0; i < KM1; ++i) {
            float xv[V];
            load_run<V, VEC>(xv, a.x + int64_t(t0 - KM1 + i) * D + ch);
#pragma unroll
            for (int v = 0; v < V; ++v) h[v * KM1 + i] = xv[v];
        }
    }

    for (int tb = t0; tb < t1; tb += kConvBatch) {
        if (tb != t0) load_batch(tb);
#pragma unroll
        for (int u = 0; u < kConvBatch; ++u) {
            if (tb + u >= t1) break;
            float o[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                // the token's own tap first, then the history oldest to newest
                float acc = xb[u][v] * w[v * K + KM1];
#pragma unroll
                for (int i = 0; i < KM1; ++i) acc = fmaf(h[v * KM1 + i], w[v * K + i], acc);
                o[v] = silu(acc);
            }
            store_run<V, VEC>(a.out + int64_t(tb + u) * D + ch, o);
            if constexpr (KM1 > 0) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
#pragma unroll
                    for (int i = 0; i + 1 < KM1; ++i) h[v * KM1 + i] = h[v * KM1 + i + 1];
                    h[v * KM1 + KM1 - 1] = xb[u][v];
                }
                if constexpr (SNAP) store_run<NH, VEC>(a.snaps + (int64_t(tb + u) * D + ch) * KM1, h);
            }
        }
    }

    if constexpr (KM1 > 0) {
        if (owner && (len > 0 || fresh)) {
            if (len > kConvChunk) {
                // Chunk 0 stopped early: the final history is the sequence's
                // last K-1 raw inputs (len > kConvChunk >= K-1).
#pragma unroll
                for (int i = 0; i < KM1; ++i) {
                    float xv[V];
                    load_run<V, VEC>(xv, a.x + int64_t(seq0 + len - KM1 + i) * D + ch);
#pragma unroll
                    for (int v = 0; v < V; ++v) h[v * KM1 + i] = xv[v];
                }
            }
            store_run<NH, VEC>(a.state + (int64_t(slot) * D + ch) * KM1, h);
        }
    }
}

struct NormArgs {
    const float *y, *z, *w;
    float *out;
    int64_t n_rows;
    int L;
    float eps;
};

// V floats per access (4: float4 path); E accesses per lane hold the row in
// registers (E = 0: any length, y read twice).
template <int V, int E>
__global__ void __launch_bounds__(kThreads) gated_rmsnorm_kernel(NormArgs a) {
    constexpr bool VEC = V == 4;
    constexpr int STEP = kNormLanes * V;
    const int64_t row = int64_t(blockIdx.x) * kNormRows + threadIdx.x / kNormLanes;
    if (row >= a.n_rows) return;                        // all 16 lanes of the row together
    const int r = int(threadIdx.x) % kNormLanes;
    const int L = a.L;
    const float *yr = a.y + row * L;
    const float *zr = a.z + row * L;
    float *orow = a.out + row * L;

    float ss = 0.f;
    if constexpr (E > 0) {
        float yv[E][V];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int d = e * STEP + r * V;
            if (d < L) {
                load_run<V, VEC>(yv[e], yr + d);
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) yv[e][v] = 0.f;
            }
#pragma unroll
            for (int v = 0; v < V; ++v) ss = fmaf(yv[e][v], yv[e][v], ss);
        }
        ss = row_allreduce<kNormLanes>(ss);
        const float inv_rms = 1.0f / sqrtf(ss / float(L) + a.eps);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int d = e * STEP + r * V;
            if (d < L) {
                float zv[V], wv[V], o[V];
                load_run<V, VEC>(zv, zr + d);
                load_run<V, VEC>(wv, a.w + d);
#pragma unroll
                for (int v = 0; v < V; ++v) o[v] = yv[e][v] * inv_rms * wv[v] * silu(zv[v]);
                store_run<V, VEC>(orow + d, o);
            }
        }
    } else {
        for (int d = r * V; d < L; d += STEP) {
            float yv[V];
            load_run<V, VEC>(yv, yr + d);
#pragma unroll
            for (int v = 0; v < V; ++v) ss = fmaf(yv[v], yv[v], ss);
        }
        ss = row_allreduce<kNormLanes>(ss);
        const float inv_rms = 1.0f / sqrtf(ss / float(L) + a.eps);
        for (int d = r * V; d < L; d += STEP) {
            float yv[V], zv[V], wv[V], o[V];
            load_run<V, VEC>(yv, yr + d);
            load_run<V, VEC>(zv, zr + d);
            load_run<V, VEC>(wv, a.w + d);
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = yv[v] * inv_rms * wv[v] * silu(zv[v]);
            store_run<V, VEC>(orow + d, o);
        }
    }
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int launch(const void *kern, void *arg, dim3 grid, hipStream_t stream) {
    void *params[] = {arg};
    const hipError_t err = hipLaunchKernel(kern, grid, dim3(kThreads), params, 0, stream);
    return err == hipSuccess ? SSM_OK : hip_fail(err, SSM_ERR_LAUNCH);
}

template <int V, bool DECODE, bool SNAP>
const void *conv_kernel_for(int km1) {
    switch (km1) {
    case 0: return reinterpret_cast<const void *>(&conv1d_silu_kernel<V, 0, DECODE, false>);
    case 1: return reinterpret_cast<const void *>(&conv1d_silu_kernel<V, 1, DECODE, SNAP>);
    case 2: return reinterpret_cast<const void *>(&conv1d_silu_kernel<V, 2, DECODE, SNAP>);
    default: return reinterpret_cast<const void *>(&conv1d_silu_kernel<V, 3, DECODE, SNAP>);
    }
}

int conv_common(const ssm_conv_dims *d, int32_t n_seqs, int32_t n_tokens, const int32_t *cu,
                const int32_t *slot, const uint8_t *fresh, const float *x, const float *weight,
                float *conv_state, int32_t n_slots, float *out, float *snapshots, bool decode,
                void *stream) {
    if (!d) return SSM_ERR_NULL;
    if (d->channels < 1 || d->kernel < 1 || n_seqs < 0 || n_tokens < 0) return SSM_ERR_DIMS;
    if (d->kernel > SSM_CONV_MAX_KERNEL) return SSM_ERR_UNSUPPORTED;
    if (n_seqs == 0) return SSM_OK;
    if (n_slots < 1) return SSM_ERR_DIMS;
    const int km1 = d->kernel - 1;
    if (!slot || !fresh || !weight || (!decode && !cu) || (km1 > 0 && !conv_state))
        return SSM_ERR_NULL;
    if (n_tokens > 0 && (!x || !out)) return SSM_ERR_NULL;
    bool vec = d->channels % 4 == 0;
    const void *floats[] = {x, weight, km1 > 0 ? conv_state : nullptr, out,
                            km1 > 0 ? snapshots : nullptr};
    for (const void *p : floats) {
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
        if (p && !aligned(p, 16)) vec = false;
    }
    if (!aligned(slot, 4) || (cu && !aligned(cu, 4))) return SSM_ERR_ALIGN;

    const int per_block = kThreads * (vec ? 4 : 1);
    const int64_t ch_blocks = (int64_t(d->channels) + per_block - 1) / per_block;
    const int64_t units = decode ? int64_t(n_seqs) : int64_t(n_seqs) + n_tokens / kConvChunk;
    if (ch_blocks > 65535 || units > INT32_MAX) return SSM_ERR_UNSUPPORTED;

    ConvArgs args{decode ? nullptr : cu, slot, fresh, x, weight, km1 > 0 ? conv_state : nullptr,
                  out, km1 > 0 ? snapshots : nullptr, d->channels, n_seqs};
    const bool snap = args.snaps != nullptr;
    const void *kern;
    if (decode)
        kern = vec ? conv_kernel_for<4, true, false>(km1) : conv_kernel_for<1, true, false>(km1);
    else if (snap)
        kern = vec ? conv_kernel_for<4, false, true>(km1) : conv_kernel_for<1, false, true>(km1);
    else
        kern = vec ? conv_kernel_for<4, false, false>(km1) : conv_kernel_for<1, false, false>(km1);
    return launch(kern, &args, dim3(unsigned(units), unsigned(ch_blocks)),
                  static_cast<hipStream_t>(stream));
}

template <int V>
const void *norm_kernel_for(int L) {
    constexpr int STEP = kNormLanes * V;
    if (L <= STEP) return reinterpret_cast<const void *>(&gated_rmsnorm_kernel<V, 1>);
    if (L <= 2 * STEP) return reinterpret_cast<const void *>(&gated_rmsnorm_kernel<V, 2>);
    if (L <= 4 * STEP) return reinterpret_cast<const void *>(&gated_rmsnorm_kernel<V, 4>);
    if (L <= 8 * STEP) return reinterpret_cast<const void *>(&gated_rmsnorm_kernel<V, 8>);
    if (L <= 16 * STEP) return reinterpret_cast<const void *>(&gated_rmsnorm_kernel<V, 16>);
    return reinterpret_cast<const void *>(&gated_rmsnorm_kernel<V, 0>);
}

}  // namespace
}  // namespace ssm

extern "C" {

int ssm_conv1d_silu_prefill(const ssm_conv_dims *dims, int32_t n_seqs, int32_t n_tokens,
                            const int32_t *cu_seqlens, const int32_t *slot,
                            const uint8_t *fresh, const float *x, const float *weight,
                            float *conv_state, int32_t n_slots, float *out, float *snapshots,
                            void *stream) {
    return ssm::conv_common(dims, n_seqs, n_tokens, cu_seqlens, slot, fresh, x, weight, conv_state,
                            n_slots, out, snapshots, false, stream);
}

int ssm_conv1d_silu_decode(const ssm_conv_dims *dims, int32_t n_seqs, const int32_t *slot,
                           const uint8_t *fresh, const float *x, const float *weight,
                           float *conv_state, int32_t n_slots, float *out, void *stream) {
    return ssm::conv_common(dims, n_seqs, n_seqs, nullptr, slot, fresh, x, weight, conv_state,
                            n_slots, out, nullptr, true, stream);
}

int ssm_gated_rmsnorm(int64_t n_rows, int32_t row_len, const float *y, const float *z,
                      const float *weight, float eps, float *out, void *stream) {
    if (n_rows < 0 || row_len < 1 || !(eps >= 0.0f) || !std::isfinite(eps)) return SSM_ERR_DIMS;
    if (n_rows == 0) return SSM_OK;
    if (!y || !z || !weight || !out) return SSM_ERR_NULL;
    bool vec = row_len % 4 == 0;
    for (const void *p : {static_cast<const void *>(y), static_cast<const void *>(z),
                          static_cast<const void *>(weight), static_cast<const void *>(out)}) {
        if (!ssm::aligned(p, 4)) return SSM_ERR_ALIGN;
        if (!ssm::aligned(p, 16)) vec = false;
    }
    const int64_t blocks = (n_rows + ssm::kNormRows - 1) / ssm::kNormRows;
    if (blocks > INT32_MAX || n_rows > INT64_MAX / row_len) return SSM_ERR_UNSUPPORTED;
    ssm::NormArgs args{y, z, weight, out, n_rows, row_len, eps};
    const void *kern = vec ? ssm::norm_kernel_for<4>(row_len) : ssm::norm_kernel_for<1>(row_len);
    return ssm::launch(kern, &args, dim3(unsigned(blocks)), static_cast<hipStream_t>(stream));
}

}  // extern "C"
