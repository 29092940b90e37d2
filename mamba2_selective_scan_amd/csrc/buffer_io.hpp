// buffer_io.hpp -- raw buffer loads and stores for the gfx950 kernels.
//
// A buffer descriptor covers [base, base + bytes).  A load at a byte offset
// past that range returns zeros and a store there is dropped, without
// touching memory, so kernels can read a window's or a row block's operands
// and write its results with no clamping and no branches, and can put the
// per-step advance in the scalar offset (no vector address arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// E consecutive floats as one load: a vector for E > 1, a float for E = 1.
template <int E> struct VecT { using type = float __attribute__((ext_vector_type(E))); };
template <> struct VecT<1> { using type = float; };
template <int E> __device__ __forceinline__ float vget(const typename VecT<E>::type &v, int e) {
    if constexpr (E == 1) return v; else return v[e];
}

constexpr int kBufferFlags = 0x00020000;   // raw (stride 0) 32-bit elements, gfx9 descriptor word 3
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, bytes, kBufferFlags);
}
template <int E>
__device__ __forceinline__ typename VecT<E>::type buffer_load(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
    using T = typename VecT<E>::type;
    if constexpr (E == 1) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voffset, soffset, 0));
    } else if constexpr (E == 2) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, voffset, soffset, 0));
    } else if constexpr (E == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0));
    } else {
        static_assert(E == 8, "1, 2, 4 or 8 floats");
        const auto lo = __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0);
        const auto hi = __builtin_amdgcn_raw_buffer_load_b128(r, voffset + 16, soffset, 0);
        T v;
        v.lo = __builtin_bit_cast(typename VecT<4>::type, lo);
        v.hi = __builtin_bit_cast(typename VecT<4>::type, hi);
        return v;
    }
}

// Cache-policy bit of a non-temporal access (the `nt` modifier on gfx950).
constexpr int kBufferNonTemporal = 2;

// 16 bytes from a descriptor, or to one (dropped past its range).
__device__ __forceinline__ typename VecT<4>::type buffer_load4_nt(__amdgpu_buffer_rsrc_t r, int voffset) {
    return __builtin_bit_cast(typename VecT<4>::type,
                              __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, kBufferNonTemporal));
}
__device__ __forceinline__ void buffer_store4_nt(typename VecT<4>::type v, __amdgpu_buffer_rsrc_t r, int voffset) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voffset, 0, kBufferNonTemporal);
}

// One byte (0 past the descriptor's range).
__device__ __forceinline__ int buffer_load_u8(const uint8_t *base, int bytes, int offset) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, bytes, kBufferFlags);
    return int(__builtin_amdgcn_raw_buffer_load_b8(r, offset, 0, 0));
}

}  // namespace ssm
