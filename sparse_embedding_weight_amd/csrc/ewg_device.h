// Device helpers of libembedding_wgrad.so: element types, rounding, and
// 16-byte vector loads/stores. Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ewg {

// fp32 -> bf16, round to nearest, ties to even. Adding 0x7fff plus the lowest
// kept bit to the dropped half carries into the kept half exactly when the
// dropped half is above one half ulp, or equal to it with an odd kept half; a
// carry out of the mantissa moves into the exponent (largest values -> inf).
// NaN keeps its sign and becomes quiet.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// Element type tags: storage type, widening to fp32, rounding from fp32.
struct BF16 {
    using T = uint16_t;
    static __device__ __forceinline__ float widen(T v) { return bf16_to_f32(v); }
    static __device__ __forceinline__ T narrow(float x) { return f32_to_bf16_rne(x); }
    // the fp32 value of narrow(x)
    static __device__ __forceinline__ float round(float x) { return bf16_to_f32(f32_to_bf16_rne(x)); }
};

struct F32 {
    using T = float;
    static __device__ __forceinline__ float widen(T v) { return v; }
    static __device__ __forceinline__ T narrow(float x) { return x; }
    static __device__ __forceinline__ float round(float x) { return x; }
};

// Load / store N consecutive elements. The address must be aligned to
// min(16, N * sizeof(T)) bytes; wider groups are moved as 16-byte pieces.
template <typename T, int N>
__device__ __forceinline__ void load_vec(const T *__restrict__ p, T (&out)[N]) {
    constexpr int bytes = N * (int)sizeof(T);
    if constexpr (bytes >= 16) {
        static_assert(bytes % 16 == 0, "vector group must be a multiple of 16 bytes");
#pragma unroll
        for (int k = 0; k < bytes / 16; ++k) {
            uint4 w = reinterpret_cast<const uint4 *>(p)[k];
            __builtin_memcpy(reinterpret_cast<char *>(out) + 16 * k, &w, 16);
        }
    } else if constexpr (bytes == 8) {
        uint2 w = *reinterpret_cast<const uint2 *>(p);
        __builtin_memcpy(out, &w, 8);
    } else if constexpr (bytes == 4) {
        uint32_t w = *reinterpret_cast<const uint32_t *>(p);
        __builtin_memcpy(out, &w, 4);
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = p[k];
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_vec(T *__restrict__ p, const T (&v)[N]) {
    constexpr int bytes = N * (int)sizeof(T);
    if constexpr (bytes >= 16) {
        static_assert(bytes % 16 == 0, "vector group must be a multiple of 16 bytes");
#pragma unroll
        for (int k = 0; k < bytes / 16; ++k) {
            uint4 w;
            __builtin_memcpy(&w, reinterpret_cast<const char *>(v) + 16 * k, 16);
            reinterpret_cast<uint4 *>(p)[k] = w;
        }
    } else if constexpr (bytes == 8) {
        uint2 w;
        __builtin_memcpy(&w, v, 8);
        *reinterpret_cast<uint2 *>(p) = w;
    } else if constexpr (bytes == 4) {
        uint32_t w;
        __builtin_memcpy(&w, v, 4);
        *reinterpret_cast<uint32_t *>(p) = w;
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) p[k] = v[k];
    }
}

// Pointer forms of load_vec / store_vec for a group of N elements inside a
// larger register array.
template <typename T, int N>
__device__ __forceinline__ void load_piece(const T *__restrict__ p, T *out) {
    load_vec<T, N>(p, *reinterpret_cast<T(*)[N]>(out));
}

template <typename T, int N>
__device__ __forceinline__ void store_piece(T *__restrict__ p, const T *v) {
    store_vec<T, N>(p, *reinterpret_cast<const T(*)[N]>(v));
}

// Lane layout of a column tile of 64 lanes x VEC columns: VEC / P pieces of P
// columns, piece s of lane l at columns s * 64 * P + l * P + [0, P) of the tile.
// P is the largest group of at most 16 bytes in both element types, so every
// load or store of a piece is contiguous across the wave (for bf16 grad and
// fp32 main_grad: 8-byte grad and 16-byte main_grad pieces of 4 columns).
template <typename G, typename M, int VEC>
constexpr int piece_cols() {
    constexpr int widest = sizeof(typename G::T) > sizeof(typename M::T) ? (int)sizeof(typename G::T)
                                                                           : (int)sizeof(typename M::T);
    return VEC < 16 / widest ? VEC : 16 / widest;
}

// ---- device-coherent moves -------------------------------------------------
// Data that one workgroup writes and another reads in the same launch (the
// partial sums of long runs, the chunk and run records) bypasses the
// non-coherent part of the cache hierarchy: 32-bit loads and stores go through
// relaxed device-scope atomics; wider ones use raw buffer instructions with the
// same device-scope cache policy. A buffer instruction also checks its offset
// against the byte range of its resource: an access past the range reads 0
// and writes nothing.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;   // untyped 32-bit elements, no swizzle
constexpr int kDeviceScope = 16;              // cache-policy bits of device scope

// `base` and `bytes` must be the same in every lane of the wave (a buffer
// resource lives in scalar registers); they are read from the first lane, so
// the compiler need not guard every access with a loop over distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes),
                                             kRawBufferWord3);
}

template <int CP = kDeviceScope>
__device__ __forceinline__ u32x4 load_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, CP);
}

__device__ __forceinline__ void store_coherent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                                 u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, kDeviceScope);
}

// P consecutive floats (P = 1, 2 or a multiple of 4), aligned to
// min(16, 4 * P) bytes; CP = 0 for data read only by a later kernel.
template <int P, int CP = kDeviceScope>
__device__ __forceinline__ void store_coherent_floats(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                                      const float *v) {
    if constexpr (P % 4 == 0) {
#pragma unroll
        for (int k = 0; k < P / 4; ++k) {
            const u32x4 w = {__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                             __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)(byte_off + 16u * k), 0, CP);
        }
    } else if constexpr (P == 2) {
        const u32x2 w = {__float_as_uint(v[0]), __float_as_uint(v[1])};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)byte_off, 0, CP);
    } else {
        static_assert(P == 1, "pieces of 1, 2 or 4k floats");
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, (int)byte_off, 0, CP);
    }
}

__device__ __forceinline__ uint32_t load_coherent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t fetch_add_coherent(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-side bounds checks, compiled in with -DEWG_DEVICE_CHECKS=1 (off by
// default): an index at or past its bound is counted in the workspace
// header's check_failures word and replaced by the last valid index, so that
// a checked build never accesses memory out of bounds.
#ifndef EWG_DEVICE_CHECKS
#define EWG_DEVICE_CHECKS 0
#endif
template <typename I>
__device__ __forceinline__ I checked_index(I i, I bound, int32_t *failures) {
    if constexpr (EWG_DEVICE_CHECKS != 0) {
        if (!(i < bound)) {
            __hip_atomic_fetch_add(failures, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return bound - 1;
        }
    }
    (void)bound;
    (void)failures;
    return i;
}

// Finish one element of a run: total = the ordered sum of its chunk sums.
// Round once to grad's dtype, add to main_grad in fp32, round to its dtype.
template <typename G, typename M>
__device__ __forceinline__ typename M::T finish(float total, typename M::T old) {
    float g = G::round(total);
    return M::narrow(M::widen(old) + g);
}

}  // namespace ewg
