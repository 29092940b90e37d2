// gdn.hip -- the C ABI (include/ssm_gdn.h) over the gated delta-rule kernels.
//
// Host side only: validate, pick the compiled shape for the key width, enqueue
// the launches on the caller's stream (one per-token kernel, or the chunked
// prep and scan kernels with a caller's workspace).  No allocation, no
// synchronisation.
#include "ssm_gdn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "gdn_chunk.hpp"
#include "gdn_decode.hpp"
#include "gdn_kernel.hpp"
#include "status.hpp"

namespace {

using ssm::GdnArgs;
using ssm::GdnShape;
using ssm::kThreads;

// Key widths up to n_max use R lanes per row, J float4 groups per lane and CT
// tokens per staged chunk for prefill, DR lanes with DJ groups for decode (the
// scan's choices at the same widths: a row of the delta rule has the shape of
// a row of the scan).
struct GdnRow {
    int n_max, R, J, CT, DR, DJ;
};
constexpr GdnRow kGdnShapes[] = {
    {16, 4, 1, 32, 4, 1},
    {32, 8, 1, 32, 8, 1},
    {64, 16, 1, 32, 16, 1},
    {128, 16, 2, 32, 8, 4},
    {256, 16, 4, 16, 16, 4},
};
static_assert(kGdnShapes[sizeof(kGdnShapes) / sizeof(kGdnShapes[0]) - 1].n_max == SSM_GDN_MAX_DK,
              "the table must cover every supported key width");

constexpr int kMaxDevices = 64;

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

template <class S, bool VEC, bool DECODE, bool SNAP>
int launch(GdnArgs a, int64_t n_blocks, hipStream_t stream) {
    const void *kern = reinterpret_cast<const void *>(&ssm::gdn_kernel<S, VEC, DECODE, SNAP>);
    const int lds_bytes = S::lds_floats(DECODE) * int(sizeof(float));
    if (lds_bytes > 64 * 1024) {
        // Opt in to more than 64 KB of dynamic LDS, once per device and kernel.
        static std::atomic<uint8_t> opted[kMaxDevices];
        int dev = 0;
        const hipError_t derr = hipGetDevice(&dev);
        if (derr != hipSuccess) return ssm::hip_fail(derr, SSM_ERR_LAUNCH);
        if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
        if (!opted[dev].load(std::memory_order_acquire)) {
            const hipError_t aerr =
                hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
            if (aerr != hipSuccess) return ssm::hip_fail(aerr, SSM_ERR_LAUNCH);
            opted[dev].store(1, std::memory_order_release);
        }
    }
    a.n_row_blocks = (a.Dv + S::RB - 1) / S::RB;
    const int64_t blocks = n_blocks * a.n_row_blocks;
    if (blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    a.n_blocks = int32_t(blocks);
    void *params[] = {&a};
    const hipError_t err = hipLaunchKernel(kern, dim3(unsigned(blocks)), dim3(kThreads), params,
                                           size_t(lds_bytes), stream);
    return err == hipSuccess ? SSM_OK : ssm::hip_fail(err, SSM_ERR_LAUNCH);
}

// The decode step on the vector path without snapshots (gdn_decode.hpp).
template <class S>
int launch_decode(GdnArgs a, int64_t n_blocks, hipStream_t stream) {
    a.n_row_blocks = (a.Dv + S::RB - 1) / S::RB;
    const int64_t blocks = n_blocks * a.n_row_blocks;
    if (blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    a.n_blocks = int32_t(blocks);
    void *params[] = {&a};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&ssm::gdn_decode_kernel<S>),
                                           dim3(unsigned(blocks)), dim3(kThreads), params, 0, stream);
    return err == hipSuccess ? SSM_OK : ssm::hip_fail(err, SSM_ERR_LAUNCH);
}

template <int R, int J, int CT, bool DECODE>
int launch_vs(const GdnArgs &a, int64_t units, bool vec, hipStream_t stream) {
    using S = GdnShape<R, J, CT>;
    const bool snap = a.snapshots != nullptr;
    if constexpr (DECODE) {
        if (vec && !snap) return launch_decode<S>(a, units, stream);
    }
    if (vec)
        return snap ? launch<S, true, DECODE, true>(a, units, stream)
                    : launch<S, true, DECODE, false>(a, units, stream);
    return snap ? launch<S, false, DECODE, true>(a, units, stream)
                : launch<S, false, DECODE, false>(a, units, stream);
}

int dispatch(const GdnArgs &a, int64_t units, bool vec, bool decode, hipStream_t stream) {
    const int dk = a.Dk;
#define SSM_GDN_ROW(IDX)                                                                        \
    if (dk <= kGdnShapes[IDX].n_max)                                                            \
        return decode ? launch_vs<kGdnShapes[IDX].DR, kGdnShapes[IDX].DJ, kGdnShapes[IDX].CT,    \
                                  true>(a, units, vec, stream)                                   \
                      : launch_vs<kGdnShapes[IDX].R, kGdnShapes[IDX].J, kGdnShapes[IDX].CT,      \
                                  false>(a, units, vec, stream);
    SSM_GDN_ROW(0)
    SSM_GDN_ROW(1)
    SSM_GDN_ROW(2)
    SSM_GDN_ROW(3)
    SSM_GDN_ROW(4)
#undef SSM_GDN_ROW
    return SSM_ERR_UNSUPPORTED;
}

// The chunked matrix-core prefill: key widths 64 and 128, whole 16-row value
// tiles, sequences of at least kGdnChunkMinLen tokens (shorter ones gain
// nothing from chunks), no snapshots, 16-byte aligned arrays.
constexpr int kGdnChunkMinLen = 32;
bool chunk_shape(const ssm_gdn_dims *d) {
    // a chunk's rows of q, k and v must fit 32-bit buffer offsets
    const int64_t chunk_bytes = ssm::GdnUnit::CT * int64_t(sizeof(float));
    return (d->d_k == 64 || d->d_k == 128) && d->d_v % 16 == 0 &&
           int64_t(d->n_k_heads) * d->d_k * chunk_bytes < INT32_MAX &&
           int64_t(d->n_v_heads) * d->d_v * chunk_bytes < INT32_MAX;
}
size_t chunk_ws_bytes(const ssm_gdn_dims *d, int32_t n_seqs, int32_t max_seqlen) {
    const size_t chunks = (size_t(max_seqlen) + ssm::GdnUnit::CT - 1) / ssm::GdnUnit::CT;
    return size_t(n_seqs) * chunks * size_t(d->n_v_heads) * ssm::GdnUnit::FLOATS * sizeof(float);
}

template <int NKT>
int launch_chunked(ssm::GdnChunkArgs ca, int32_t n_seqs, hipStream_t stream) {
    const GdnArgs &a = ca.a;
    const int64_t prep_units = int64_t(n_seqs) * ca.max_chunks * a.Hk;
    const int64_t scan_blocks = int64_t(n_seqs) * a.Hv * (a.Dv / 16);
    if (prep_units > INT32_MAX - 3 || scan_blocks > INT32_MAX) return SSM_ERR_UNSUPPORTED;
    ssm::GdnChunkArgs prep = ca;
    prep.a.n_blocks = int32_t(prep_units);
    void *pp[] = {&prep};
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&ssm::gdn_chunk_prep_kernel<NKT>),
                                     dim3(unsigned((prep_units + ssm::kWaves - 1) / ssm::kWaves)), dim3(kThreads),
                                     pp, 0, stream);
    if (err != hipSuccess) return ssm::hip_fail(err, SSM_ERR_LAUNCH);
    ssm::GdnChunkArgs scan = ca;
    scan.a.n_row_blocks = a.Dv / 16;
    scan.a.n_blocks = int32_t(scan_blocks);
    void *sp[] = {&scan};
    err = hipLaunchKernel(reinterpret_cast<const void *>(&ssm::gdn_chunk_scan_kernel<NKT>),
                          dim3(unsigned(scan_blocks)), dim3(kThreads), sp, 0, stream);
    return err == hipSuccess ? SSM_OK : ssm::hip_fail(err, SSM_ERR_LAUNCH);
}

int gdn_common(const ssm_gdn_dims *d, int32_t n_seqs, int32_t n_tokens, const int32_t *cu,
               const int32_t *slot, const uint8_t *fresh, const float *q, const float *k,
               const float *v, const float *g, const float *beta, float scale, float *state,
               int32_t n_slots, float *y, float *snapshots, bool decode, void *stream,
               int32_t max_seqlen = 0, void *ws = nullptr, size_t ws_bytes = 0) {
    if (!d) return SSM_ERR_NULL;
    if (d->n_v_heads < 1 || d->n_k_heads < 1 || d->d_k < 1 || d->d_v < 1 || n_seqs < 0 ||
        n_tokens < 0 || d->n_v_heads % d->n_k_heads != 0)
        return SSM_ERR_DIMS;
    if (d->d_k > SSM_GDN_MAX_DK) return SSM_ERR_UNSUPPORTED;
    if (n_seqs == 0) return SSM_OK;
    if (n_slots < 1) return SSM_ERR_DIMS;
    if (!slot || !fresh || !state || (!decode && !cu)) return SSM_ERR_NULL;
    if (n_tokens > 0 && (!q || !k || !v || !g || !beta || !y)) return SSM_ERR_NULL;
    bool vec = d->d_k % 4 == 0 && d->d_v % 4 == 0;
    const void *floats[] = {q, k, v, g, beta, state, y, snapshots};
    for (const void *p : floats) {
        if (p && !aligned(p, 4)) return SSM_ERR_ALIGN;
    }
    for (const void *p : {static_cast<const void *>(q), static_cast<const void *>(k),
                          static_cast<const void *>(v), static_cast<const void *>(state),
                          static_cast<const void *>(y), static_cast<const void *>(snapshots)})
        if (p && !aligned(p, 16)) vec = false;
    if (!aligned(slot, 4) || (cu && !aligned(cu, 4))) return SSM_ERR_ALIGN;

    GdnArgs a{};
    a.cu_seqlens = decode ? nullptr : cu;
    a.slot = slot;
    a.fresh = fresh;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.y = y;
    a.snapshots = snapshots;
    a.scale = scale;
    a.Hv = d->n_v_heads;
    a.Hk = d->n_k_heads;
    a.Dk = d->d_k;
    a.Dv = d->d_v;
    a.heads_per_key = d->n_v_heads / d->n_k_heads;
    if (!decode && !snapshots && vec && chunk_shape(d) && max_seqlen >= kGdnChunkMinLen) {
        if (!ws) return SSM_ERR_NULL;
        if (ws_bytes < chunk_ws_bytes(d, n_seqs, max_seqlen)) return SSM_ERR_DIMS;
        if (!aligned(ws, 16)) return SSM_ERR_ALIGN;
        ssm::GdnChunkArgs ca{};
        ca.a = a;
        ca.ws = static_cast<float *>(ws);
        ca.max_chunks = int32_t((int64_t(max_seqlen) + ssm::GdnUnit::CT - 1) / ssm::GdnUnit::CT);
        hipStream_t st = static_cast<hipStream_t>(stream);
        return d->d_k == 64 ? launch_chunked<4>(ca, n_seqs, st) : launch_chunked<8>(ca, n_seqs, st);
    }
    const int64_t units = int64_t(n_seqs) * d->n_v_heads;   // times the row blocks, per shape
    return dispatch(a, units, vec, decode, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int ssm_gdn_prefill(const ssm_gdn_dims *dims, int32_t n_seqs, int32_t n_tokens,
                    const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                    const float *q, const float *k, const float *v, const float *g,
                    const float *beta, float scale, float *state, int32_t n_slots, float *y,
                    float *snapshots, void *stream) {
    return gdn_common(dims, n_seqs, n_tokens, cu_seqlens, slot, fresh, q, k, v, g, beta, scale,
                      state, n_slots, y, snapshots, false, stream);
}

int ssm_gdn_prefill_workspace_size(const ssm_gdn_dims *dims, int32_t n_seqs, int32_t max_seqlen,
                                   size_t *bytes) {
    if (!dims || !bytes) return SSM_ERR_NULL;
    if (dims->n_v_heads < 1 || dims->n_k_heads < 1 || dims->d_k < 1 || dims->d_v < 1 ||
        n_seqs < 0 || max_seqlen < 0 || dims->n_v_heads % dims->n_k_heads != 0)
        return SSM_ERR_DIMS;
    *bytes = chunk_shape(dims) && max_seqlen >= kGdnChunkMinLen
                 ? chunk_ws_bytes(dims, n_seqs, max_seqlen) : 0;
    return SSM_OK;
}

int ssm_gdn_prefill_ws(const ssm_gdn_dims *dims, int32_t n_seqs, int32_t n_tokens,
                       const int32_t *cu_seqlens, const int32_t *slot, const uint8_t *fresh,
                       const float *q, const float *k, const float *v, const float *g,
                       const float *beta, float scale, float *state, int32_t n_slots, float *y,
                       int32_t max_seqlen, void *workspace, size_t workspace_bytes,
                       void *stream) {
    if (max_seqlen < 0) return SSM_ERR_DIMS;
    return gdn_common(dims, n_seqs, n_tokens, cu_seqlens, slot, fresh, q, k, v, g, beta, scale,
                      state, n_slots, y, nullptr, false, stream, max_seqlen, workspace,
                      workspace_bytes);
}

int ssm_gdn_decode(const ssm_gdn_dims *dims, int32_t n_seqs, const int32_t *slot,
                   const uint8_t *fresh, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, float scale, float *state,
                   int32_t n_slots, float *y, float *snapshots, void *stream) {
    return gdn_common(dims, n_seqs, n_seqs, nullptr, slot, fresh, q, k, v, g, beta, scale, state,
                      n_slots, y, snapshots, true, stream);
}

}  // extern "C"
