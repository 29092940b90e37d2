// calib.hip -- the read-modify-write stream of include/ssm_calib.h: the
// achievable HBM rate for a kernel that reads and writes each element once.
#include "ssm_calib.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

using f4 = float __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int PL>
__global__ void __launch_bounds__(kThreads) stream_rw_kernel(f4 *data, float a, float b) {
    f4 *base = data + int64_t(blockIdx.x) * (kThreads * PL) + threadIdx.x;
    f4 v[PL];
#pragma unroll
    for (int k = 0; k < PL; ++k) v[k] = __builtin_nontemporal_load(base + k * kThreads);
#pragma unroll
    for (int k = 0; k < PL; ++k) __builtin_nontemporal_store(v[k] * a + b, base + k * kThreads);
}

template <int PL>
int launch(float *data, int64_t n4, float a, float b, hipStream_t stream) {
    if (n4 % (int64_t(kThreads) * PL) != 0) return -2;
    const int64_t blocks = n4 / (int64_t(kThreads) * PL);
    if (blocks > INT32_MAX) return -2;
    hipLaunchKernelGGL(stream_rw_kernel<PL>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       reinterpret_cast<f4 *>(data), a, b);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace

extern "C" int ssm_calib_stream_rw(float *data, int64_t n_float4, int32_t per_lane, float a,
                                   float b, void *stream_ptr) {
    if (!data) return -2;
    if (reinterpret_cast<uintptr_t>(data) % 16 != 0) return -4;
    if (n_float4 <= 0) return -2;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    switch (per_lane) {
    case 1: return launch<1>(data, n_float4, a, b, stream);
    case 2: return launch<2>(data, n_float4, a, b, stream);
    case 4: return launch<4>(data, n_float4, a, b, stream);
    case 8: return launch<8>(data, n_float4, a, b, stream);
    default: return -2;
    }
}
