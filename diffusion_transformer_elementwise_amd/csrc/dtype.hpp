// Storage types of the kernels: bf16, IEEE binary16 and binary32. The
// arithmetic is binary32 for all of them; loads widen exactly and stores
// narrow once with round-to-nearest-even (v_cvt_pk_bf16_f32 for bf16, the
// binary16 convert for f16, nothing for f32).
//
// Pack<DT> holds 8 consecutive elements: one 16-byte access for the 2-byte
// types, two for binary32. Pack index i covers elements 8i .. 8i+7, so the
// kernels' indexing does not depend on the type.
#pragma once

#include "bf16x8.hpp"

namespace rga {

enum : int { kBF16 = 0, kF16 = 1, kF32 = 2 };
enum : int { kModRow = 0, kModToken = 1 };

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Pack;

template <>
struct Pack<kBF16> {
    u32x4 v;
    __device__ __forceinline__ float get(int e) const
    {
        return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
    }
    __device__ __forceinline__ static Pack make(const float* f)
    {
        Pack p;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p.v[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
        return p;
    }
    __device__ __forceinline__ static Pack zero()
    {
        Pack p;
        p.v = u32x4{0, 0, 0, 0};
        return p;
    }
    __device__ __forceinline__ static Pack load(const void* b, int64_t i)
    {
        Pack p;
        p.v = load16(static_cast<const u32x4*>(b) + i);
        return p;
    }
    __device__ __forceinline__ static Pack load_stream(const void* b, int64_t i)
    {
        Pack p;
        p.v = load16_stream(static_cast<const u32x4*>(b) + i);
        return p;
    }
    __device__ __forceinline__ void store_stream(void* b, int64_t i) const
    {
        store16_stream(static_cast<u32x4*>(b) + i, v);
    }
};

template <>
struct Pack<kF16> {
    u32x4 v;
    __device__ __forceinline__ float get(int e) const
    {
        // copy the word out first: clang's __builtin_bit_cast applied to a
        // vector element expression reads from the start of the vector
        const uint32_t w = v[e >> 1];
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        return (float)h[e & 1];
    }
    __device__ __forceinline__ static Pack make(const float* f)
    {
        Pack p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2 w = {f[2 * i], f[2 * i + 1]};
            p.v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));
        }
        return p;
    }
    __device__ __forceinline__ static Pack zero()
    {
        Pack p;
        p.v = u32x4{0, 0, 0, 0};
        return p;
    }
    __device__ __forceinline__ static Pack load(const void* b, int64_t i)
    {
        Pack p;
        p.v = load16(static_cast<const u32x4*>(b) + i);
        return p;
    }
    __device__ __forceinline__ static Pack load_stream(const void* b, int64_t i)
    {
        Pack p;
        p.v = load16_stream(static_cast<const u32x4*>(b) + i);
        return p;
    }
    __device__ __forceinline__ void store_stream(void* b, int64_t i) const
    {
        store16_stream(static_cast<u32x4*>(b) + i, v);
    }
};

template <>
struct Pack<kF32> {
    u32x4 a, b;
    __device__ __forceinline__ float get(int e) const
    {
        return __uint_as_float(e < 4 ? a[e] : b[e - 4]);
    }
    __device__ __forceinline__ static Pack make(const float* f)
    {
        Pack p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p.a[i] = __float_as_uint(f[i]);
            p.b[i] = __float_as_uint(f[4 + i]);
        }
        return p;
    }
    __device__ __forceinline__ static Pack zero()
    {
        Pack p;
        p.a = u32x4{0, 0, 0, 0};
        p.b = u32x4{0, 0, 0, 0};
        return p;
    }
    __device__ __forceinline__ static Pack load(const void* base, int64_t i)
    {
        const u32x4* q = static_cast<const u32x4*>(base) + 2 * i;
        Pack p;
        p.a = load16(q);
        p.b = load16(q + 1);
        return p;
    }
    __device__ __forceinline__ static Pack load_stream(const void* base, int64_t i)
    {
        const u32x4* q = static_cast<const u32x4*>(base) + 2 * i;
        Pack p;
        p.a = load16_stream(q);
        p.b = load16_stream(q + 1);
        return p;
    }
    __device__ __forceinline__ void store_stream(void* base, int64_t i) const
    {
        u32x4* q = static_cast<u32x4*>(base) + 2 * i;
        store16_stream(q, a);
        store16_stream(q + 1, b);
    }
};

// Single elements, for the generic kernels (any D, element-aligned pointers).
template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i)
{
    if constexpr (DT == kF32) {
        return static_cast<const float*>(base)[i];
    } else if constexpr (DT == kF16) {
        return (float)static_cast<const _Float16*>(base)[i];
    } else {
        return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
    }
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v)
{
    if constexpr (DT == kF32) {
        static_cast<float*>(base)[i] = v;
    } else if constexpr (DT == kF16) {
        static_cast<_Float16*>(base)[i] = (_Float16)v;
    } else {
        static_cast<uint16_t*>(base)[i] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
    }
}

}  // namespace rga
