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

// Lane-interleaved packs, for kernels where a lane may hold any 8 elements of
// a chunk (no summation order to keep). A chunk is h <= 64 consecutive packs
// starting at pack c0, handled by lanes t < h. For the 2-byte types lane t
// takes pack c0 + t as above. For binary32 lane t takes the 16-byte words
// 2*c0 + t and 2*c0 + h + t, so that each load or store instruction of the
// wave covers one contiguous run of memory; two adjacent words per lane
// leave every instruction half a cache line per lane and measured about 15 %
// slower on MI355X.
template <int DT>
struct Interleaved {
    __device__ __forceinline__ static Pack<DT> load(const void* b, int64_t c0, int t, int h)
    {
        (void)h;
        return Pack<DT>::load(b, c0 + t);
    }
    __device__ __forceinline__ static Pack<DT> load_stream(const void* b, int64_t c0, int t, int h)
    {
        (void)h;
        return Pack<DT>::load_stream(b, c0 + t);
    }
    __device__ __forceinline__ static void store_stream(const Pack<DT>& p, void* b, int64_t c0,
                                                        int t, int h)
    {
        (void)h;
        p.store_stream(b, c0 + t);
    }
};

template <>
struct Interleaved<kF32> {
    __device__ __forceinline__ static Pack<kF32> load(const void* base, int64_t c0, int t, int h)
    {
        const u32x4* q = static_cast<const u32x4*>(base) + 2 * c0 + t;
        Pack<kF32> p;
        p.a = load16(q);
        p.b = load16(q + h);
        return p;
    }
    __device__ __forceinline__ static Pack<kF32> load_stream(const void* base, int64_t c0, int t,
                                                             int h)
    {
        const u32x4* q = static_cast<const u32x4*>(base) + 2 * c0 + t;
        Pack<kF32> p;
        p.a = load16_stream(q);
        p.b = load16_stream(q + h);
        return p;
    }
    __device__ __forceinline__ static void store_stream(const Pack<kF32>& p, void* base,
                                                        int64_t c0, int t, int h)
    {
        u32x4* q = static_cast<u32x4*>(base) + 2 * c0 + t;
        store16_stream(q, p.a);
        store16_stream(q + h, p.b);
    }
};

// Grouped packs, for kernels where lane t must hold pack c0 + t of a chunk
// of h <= 64 packs (a summation order fixes which elements a lane adds).
// Packs past the chunk (t >= h, or h <= 0) load as zeros and are not
// stored. For the 2-byte types a pack is one 16-byte word per lane. For
// binary32 a pack is two words; lane t moves words wa(t) and 64 + wa(t) of
// the chunk ("raw" order), wa(t) = 2t for t < 32 and 2(t - 32) + 1
// otherwise, so that each of the two access instructions covers one
// contiguous run, and one v_permlane32_swap per dword (lanes 32..63 of the
// first register trade with lanes 0..31 of the second) turns raw order into
// words 2t and 2t + 1 (group order). The swap is its own inverse. Element-wise
// work can stay in raw order (load_raw / store_raw); only values that feed
// an ordered sum need to_groups. Every call that swaps must be made with the
// whole wave active: the swap reads other lanes' registers.
template <int DT>
struct Grouped {
    __device__ __forceinline__ static Pack<DT> load_raw(const void* b, int64_t c0, int t, int h)
    {
        return t < h ? Pack<DT>::load(b, c0 + t) : Pack<DT>::zero();
    }
    __device__ __forceinline__ static Pack<DT> load_stream_raw(const void* b, int64_t c0, int t,
                                                               int h)
    {
        return t < h ? Pack<DT>::load_stream(b, c0 + t) : Pack<DT>::zero();
    }
    __device__ __forceinline__ static void store_stream_raw(const Pack<DT>& p, void* b,
                                                            int64_t c0, int t, int h)
    {
        if (t < h)
            p.store_stream(b, c0 + t);
    }
    // load_raw / load_stream_raw without a branch around the load: the index
    // is clamped to the row's last pack (c0 + h - 1, which every row has) and
    // the zeros are selected afterwards. A branch per load made the compiler
    // wait for one pack's loads before issuing the next pack's.
    template <bool STREAM>
    __device__ __forceinline__ static Pack<DT> load_clamped(const void* b, int64_t c0, int t, int h)
    {
        const int tc = t < h ? t : h - 1;
        Pack<DT> p = STREAM ? Pack<DT>::load_stream(b, c0 + tc) : Pack<DT>::load(b, c0 + tc);
        const bool in = t < h;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            p.v[d] = in ? p.v[d] : 0u;
        return p;
    }
    __device__ __forceinline__ static Pack<DT> to_groups(const Pack<DT>& p) { return p; }
    __device__ __forceinline__ static Pack<DT> to_raw(const Pack<DT>& p) { return p; }
    __device__ __forceinline__ static Pack<DT> load_stream(const void* b, int64_t c0, int t, int h)
    {
        return load_stream_raw(b, c0, t, h);
    }
    // load_raw from a row staged in LDS as 16-byte words in memory order;
    // the index is clamped into the row and zeros selected past its end (no
    // branch, so a wave's reads can all be issued before the first use)
    __device__ __forceinline__ static Pack<DT> lds_raw(const u32x4* w, int c0, int t, int h)
    {
        Pack<DT> p;
        p.v = w[c0 + (t < h ? t : h - 1)];
        const bool in = t < h;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            p.v[d] = in ? p.v[d] : 0u;
        return p;
    }
};

template <>
struct Grouped<kF32> {
    __device__ __forceinline__ static int wa(int t) { return t < 32 ? 2 * t : 2 * (t - 32) + 1; }
    __device__ __forceinline__ static Pack<kF32> swapped(const Pack<kF32>& p)
    {
        Pack<kF32> q;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const auto r = __builtin_amdgcn_permlane32_swap(p.a[k], p.b[k], false, false);
            q.a[k] = r[0];
            q.b[k] = r[1];
        }
        return q;
    }
    template <bool STREAM>
    __device__ __forceinline__ static Pack<kF32> load_any(const void* base, int64_t c0, int t,
                                                          int h)
    {
        const u32x4* q = static_cast<const u32x4*>(base) + 2 * c0;
        const int w = wa(t);
        const u32x4 z = {0, 0, 0, 0};
        Pack<kF32> p;
        p.a = w < 2 * h ? (STREAM ? load16_stream(q + w) : load16(q + w)) : z;
        p.b = 64 + w < 2 * h ? (STREAM ? load16_stream(q + 64 + w) : load16(q + 64 + w)) : z;
        return p;
    }
    // load_any without branches: word indexes clamped to the row's last word
    // (2(c0 + h) - 1), zeros selected afterwards
    template <bool STREAM>
    __device__ __forceinline__ static Pack<kF32> load_clamped(const void* base, int64_t c0, int t,
                                                              int h)
    {
        const u32x4* q = static_cast<const u32x4*>(base) + 2 * c0;
        const int w = wa(t);
        const int wb = 64 + w;
        const int last = 2 * h - 1;
        Pack<kF32> p;
        p.a = STREAM ? load16_stream(q + (w < 2 * h ? w : last)) : load16(q + (w < 2 * h ? w : last));
        p.b = STREAM ? load16_stream(q + (wb < 2 * h ? wb : last))
                     : load16(q + (wb < 2 * h ? wb : last));
        const bool ia = w < 2 * h, ib = wb < 2 * h;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            p.a[d] = ia ? p.a[d] : 0u;
            p.b[d] = ib ? p.b[d] : 0u;
        }
        return p;
    }
    __device__ __forceinline__ static Pack<kF32> load_raw(const void* b, int64_t c0, int t, int h)
    {
        return load_any<false>(b, c0, t, h);
    }
    __device__ __forceinline__ static Pack<kF32> load_stream_raw(const void* b, int64_t c0, int t,
                                                                 int h)
    {
        return load_any<true>(b, c0, t, h);
    }
    __device__ __forceinline__ static void store_stream_raw(const Pack<kF32>& p, void* base,
                                                            int64_t c0, int t, int h)
    {
        u32x4* q = static_cast<u32x4*>(base) + 2 * c0;
        const int w = wa(t);
        if (w < 2 * h)
            store16_stream(q + w, p.a);
        if (64 + w < 2 * h)
            store16_stream(q + 64 + w, p.b);
    }
    __device__ __forceinline__ static Pack<kF32> to_groups(const Pack<kF32>& p) { return swapped(p); }
    __device__ __forceinline__ static Pack<kF32> to_raw(const Pack<kF32>& p) { return swapped(p); }
    // load_raw from a row staged in LDS as 16-byte words in memory order
    __device__ __forceinline__ static Pack<kF32> lds_raw(const u32x4* w, int c0, int t, int h)
    {
        const u32x4* q = w + 2 * c0;
        const int a = wa(t);
        const u32x4 z = {0, 0, 0, 0};
        Pack<kF32> p;
        p.a = a < 2 * h ? q[a] : z;
        p.b = 64 + a < 2 * h ? q[64 + a] : z;
        return p;
    }
    __device__ __forceinline__ static Pack<kF32> load_stream(const void* b, int64_t c0, int t,
                                                             int h)
    {
        return swapped(load_any<true>(b, c0, t, h));
    }
};

// Single elements: the trailing n % 8 elements of a flat pack stream, and the
// narrowing of the span path (span.hpp).
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

// the storage value of v (one round-to-nearest-even for the 2-byte types)
template <int DT>
__device__ __forceinline__ uint32_t narrow_elem(float v)
{
    if constexpr (DT == kF32) {
        return __float_as_uint(v);
    } else if constexpr (DT == kF16) {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    } else {
        return pack_bf16(v, 0.0f) & 0xFFFFu;
    }
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v)
{
    if constexpr (DT == kF32)
        static_cast<float*>(base)[i] = v;
    else
        static_cast<uint16_t*>(base)[i] = (uint16_t)narrow_elem<DT>(v);
}

// ---- Modulation factors staged for many rows ---------------------------------
//
// The element path's staged rows (row_regs.hpp) hold 1 + scale already
// widened to binary32: two words per group of eight 2-byte elements
// (elements 0-3, then 4-7). It is the same binary32 sum that would
// otherwise be taken per element of every row, so results do not change;
// each row's apply then skips a widening and an add per element, which
// counts on that path's realigning, instruction-heavy rows.
template <int DT>
__device__ __forceinline__ void one_plus(const u32x4& s, u32x4& lo, u32x4& hi)
{
    static_assert(DT != kF32, "groups of eight 2-byte elements");
    Pack<DT> p;
    p.v = s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = __float_as_uint(1.0f + p.get(e));
        hi[e] = __float_as_uint(1.0f + p.get(4 + e));
    }
}

// (((x - mu) or x) * rr) * a + shift per element of a group, rounded once to
// the storage type; a = 1 + scale as one_plus stores it.
template <int DT, bool CENTER>
__device__ __forceinline__ Pack<DT> modulate_group(const Pack<DT>& x, float mu, float rr,
                                                   const u32x4& a_lo, const u32x4& a_hi,
                                                   const Pack<DT>& shift)
{
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float v = x.get(e);
        if constexpr (CENTER)
            v = v - mu;
        const float n = v * rr;
        const float a = __uint_as_float(e < 4 ? a_lo[e] : a_hi[e - 4]);
        const float m = n * a;
        o[e] = m + shift.get(e);
    }
    return Pack<DT>::make(o);
}

}  // namespace rga
