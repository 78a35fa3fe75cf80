// Device-side helpers for 128-bit bf16 vectors on gfx950.
//
// One 16-byte access carries 8 consecutive bf16 values as four 32-bit words;
// element 2i is the low half of word i and element 2i+1 its high half
// (little-endian). Widening is exact (a bf16 pattern is the upper half of a
// binary32 pattern); narrowing uses the CDNA4 packed convert
// v_cvt_pk_bf16_f32, which rounds to nearest even under the default mode
// register and keeps subnormals (the kernels are built with f32 denormals
// preserved).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rga {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w)
{
    return __uint_as_float(w << 16);
}

__device__ __forceinline__ float bf16_hi(uint32_t w)
{
    return __uint_as_float(w & 0xFFFF0000u);
}

// Two binary32 values -> one word of two bf16 (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The calling wave's index in its workgroup, held by the whole wave in a
// scalar register: the compiler takes threadIdx.x / 64 for a per-lane
// value, and with it every row index, address, offset and branch derived
// from it (vector arithmetic for each, lane masks for each branch).
__device__ __forceinline__ int wave_in_group()
{
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Plain 128-bit global load / store (global_load_dwordx4 / store).
__device__ __forceinline__ u32x4 load16(const u32x4* p)
{
    return *p;
}

__device__ __forceinline__ void store16(u32x4* p, u32x4 v)
{
    *p = v;
}

// Streaming variants (global_load/store_dwordx4 ... nt): the nontemporal
// hint marks lines as read or written once. On MI355X this is what lets a
// chain of streaming kernels run near the HBM limit: plain stores leave
// dirty lines in the L2 and memory-side caches whose write-back is then
// paid by the next kernel, and plain loads allocate lines nobody reuses.
__device__ __forceinline__ u32x4 load16_stream(const u32x4* p)
{
    return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store16_stream(u32x4* p, u32x4 v)
{
    __builtin_nontemporal_store(v, p);
}

}  // namespace rga
