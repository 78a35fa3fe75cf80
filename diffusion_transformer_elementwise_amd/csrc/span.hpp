// Element spans at any element alignment, staged through LDS with 16-byte
// accesses.
//
// Used by the modulations' element kernels where a row does not fit the
// register-resident path (binary32 rows, rows longer than 8192 elements);
// every other element path realigns in registers (realign.hpp). Accessing a
// span element by element is bound by the access issue rate on MI355X
// (2-byte accesses measured at 2.4 TB/s, 16-byte ones at 6.6), so a wave
// moves a span of n elements through LDS instead:
//
//   load:  lanes read the aligned 16-byte words that hold the span (word w
//          by lane w mod 64: every instruction covers one contiguous run)
//          into a raw LDS buffer, so that element i of the span sits at byte
//          offset m + i * es, m being the span's start address mod 16. Every
//          word read holds at least one byte of the span, so it lies in
//          memory the caller owns pages of; the bytes outside the span are
//          read and ignored.
//   get / put: element i as binary32, widened from or narrowed to storage.
//   store: words of the raw buffer that lie wholly inside the span are
//          written with 16-byte stores, the partial first and last words
//          element by element, so no byte outside the span is written.
//
// Every function is called by the whole wave; put and get by any lanes.
// Between load and get, and between put and store, the caller separates
// the lanes' LDS accesses with a barrier.
#pragma once

#include "dtype.hpp"
#include "realign.hpp"

namespace rga {

template <int DT>
__device__ __forceinline__ float from_bits(uint32_t b)
{
    if constexpr (DT == kF32) {
        return __uint_as_float(b);
    } else if constexpr (DT == kF16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    } else {
        return __uint_as_float(b << 16);
    }
}

template <int DT, int MAXN>
struct Span {
    static constexpr int kEs = DT == kF32 ? 4 : 2;
    // raw words a span of up to MAXN elements can touch (start offset < 16)
    static constexpr int kWords = (15 + MAXN * kEs + 15) / 16;
    static constexpr int kPerLane = (kWords + 63) / 64;

    __device__ __forceinline__ static int offset(const void* p)
    {
        return (int)(reinterpret_cast<uintptr_t>(p) & 15u);
    }

    // words of a span in flight in registers (fetch), then written to LDS
    // (commit): a caller can fetch the next span before working on this one
    struct Words {
        u32x4 v[kPerLane];
        int count;
    };

    template <bool STREAM>
    __device__ __forceinline__ static Words fetch(const void* p, int n)
    {
        const int lane = threadIdx.x & 63;
        const u32x4* w0 = aligned_down(p);
        Words r;
        r.count = n > 0 ? (start_offset(p) + n * kEs + 15) >> 4 : 0;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int w = lane + 64 * k;
            r.v[k] = u32x4{0, 0, 0, 0};
            if (w < r.count)
                r.v[k] = STREAM ? load16_stream(w0 + w) : load16(w0 + w);
        }
        return r;
    }

    // Whole wave: write the span's words to LDS shifted so that element i
    // sits at byte i * es, i.e. group g of 8 elements in word g (2-byte
    // types) or words 2g, 2g + 1 (binary32), readable with aligned 16-byte
    // LDS reads that touch every bank (the unshifted layout puts the groups
    // of neighbouring lanes 16 bytes apart at one offset in their words: an
    // 8-way bank conflict). m is the span's start offset (wave-uniform).
    // Lane t's word w = t + 64k is joined with word w + 1, which lane t + 1
    // holds (a DPP wave shift left by one lane) or, for lane 63, lane 0 in
    // its next slot (a lane read into the shift's fill value). Bytes past
    // the span's end are garbage and never read as elements.
    __device__ __forceinline__ static void commit_aligned(const Words& r, int m, int n,
                                                          u32x4* raw)
    {
        const int lane = threadIdx.x & 63;
        const int na = (n * kEs + 15) >> 4;  // aligned words holding the span
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const u32x4 fill = (k + 1 < kPerLane) ? read_lane(r.v[k + 1 < kPerLane ? k + 1 : k], 0)
                                                  : u32x4{0, 0, 0, 0};
            const u32x4 nx = lane_from_next(r.v[k], fill);
            const u32x4 o = window_at(r.v[k], nx, m);
            const int w = lane + 64 * k;
            if (w < na)
                raw[w] = o;
        }
    }

    // Group g (elements 8g .. 8g + 7) of a span committed with commit_aligned.
    __device__ __forceinline__ static Pack<DT> group(const u32x4* raw, int g)
    {
        Pack<DT> p;
        if constexpr (DT == kF32) {
            p.a = raw[2 * g];
            p.b = raw[2 * g + 1];
        } else {
            p.v = raw[g];
        }
        return p;
    }

    __device__ __forceinline__ static void commit(const Words& r, u32x4* raw)
    {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int w = lane + 64 * k;
            if (w < r.count)
                raw[w] = r.v[k];
        }
    }

    template <bool STREAM>
    __device__ __forceinline__ static void load(const void* p, int n, u32x4* raw)
    {
        commit(fetch<STREAM>(p, n), raw);
    }

    __device__ __forceinline__ static float get(const u32x4* raw, int m, int i)
    {
        const unsigned char* b = reinterpret_cast<const unsigned char*>(raw) + m + i * kEs;
        if constexpr (DT == kF32)
            return *reinterpret_cast<const float*>(b);
        else
            return from_bits<DT>(*reinterpret_cast<const uint16_t*>(b));
    }

    __device__ __forceinline__ static void put(u32x4* raw, int m, int i, float v)
    {
        unsigned char* b = reinterpret_cast<unsigned char*>(raw) + m + i * kEs;
        if constexpr (DT == kF32)
            *reinterpret_cast<float*>(b) = v;
        else
            *reinterpret_cast<uint16_t*>(b) = (uint16_t)narrow_elem<DT>(v);
    }

    template <bool STREAM>
    __device__ __forceinline__ static void store(void* p, int n, const u32x4* raw)
    {
        const int lane = threadIdx.x & 63;
        u32x4* w0 = aligned_down(p);
        const int m = start_offset(p);
        const int end = m + n * kEs;  // span bytes [m, end) of the raw buffer
        const int words = n > 0 ? (end + 15) >> 4 : 0;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int w = lane + 64 * k;
            if (w >= words)
                continue;
            const int lo = 16 * w;
            if (lo >= m && lo + 16 <= end) {
                if (STREAM)
                    store16_stream(w0 + w, raw[w]);
                else
                    w0[w] = raw[w];
            } else {
                const unsigned char* rb = reinterpret_cast<const unsigned char*>(raw);
                unsigned char* gb = reinterpret_cast<unsigned char*>(w0);
                const int b0 = lo > m ? lo : m;
                const int b1 = lo + 16 < end ? lo + 16 : end;
                for (int bo = b0; bo < b1; bo += kEs) {
                    if constexpr (DT == kF32)
                        *reinterpret_cast<float*>(gb + bo) = *reinterpret_cast<const float*>(rb + bo);
                    else
                        *reinterpret_cast<uint16_t*>(gb + bo) =
                            *reinterpret_cast<const uint16_t*>(rb + bo);
                }
            }
        }
    }
};

}  // namespace rga
