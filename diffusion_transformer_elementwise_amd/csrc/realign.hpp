// Runs of 2-byte elements at any element alignment, realigned in registers.
//
// A run of n elements starting at address p (start offset m = p mod 16) is
// read as the aligned 16-byte words that hold its bytes: lane t, slot k
// holds word t + 64k of that window (one contiguous wave-wide access per
// slot); word 64K, which only a run of exactly 64K groups can reach with
// m > 0, is held by every lane. realign_in then turns the words into
// groups: lane t, slot k holds elements 8(t + 64k) .. 8(t + 64k) + 7 of the
// run, by joining its word with the next one (which lane t + 1 holds: a DPP
// wave shift left by one lane, lane 63 taking lane 0 of the next slot) and
// cutting 16 bytes at offset m (alignbyte). store_run does the reverse for
// an output at its own start offset: word w of the output window joins
// groups w - 1 (a DPP wave shift right) and w, interior words go out with
// 16-byte stores and the two partial edge words element by element, so no
// byte outside the run is written.
//
// Two forms of the cut: window_at takes the offset at run time (selects pick
// the dwords), window_c<O> has it fixed (the picks are free). realign_in and
// store_run branch once per run on the wave-uniform offset (dispatch_offset)
// to code for that offset, which pays off over a row's many slots; the
// chunked kernels cut one word per lane and keep window_at, where a branch
// between the loads and their use cost more than the selects.
//
// Every word read holds at least one byte of the run, so it lies in memory
// the caller owns pages of; the other bytes are read and ignored. Groups
// past the run's end hold garbage that callers neither store nor sum.
//
// Every function is called by the whole wave with wave-uniform arguments.
#pragma once

#include "dtype.hpp"

namespace rga {

// One of four values by a wave-uniform index (q1, q2 its bits), as selects
// on values: indexing a local array with a select would put the array in
// scratch memory.
__device__ __forceinline__ uint32_t pick4(bool q1, bool q2, uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3)
{
    const uint32_t lo = q1 ? a1 : a0;
    const uint32_t hi = q1 ? a3 : a2;
    return q2 ? hi : lo;
}

// Bytes o .. o + 15 of the 32-byte window (c, n), 0 <= o < 16, o
// wave-uniform: the dword shift o >> 2 picks dwords with selects on a
// uniform condition (no branches), then alignbyte shifts by o & 3 bytes.
__device__ __forceinline__ u32x4 window_at(const u32x4& c, const u32x4& n, int o)
{
    const bool q1 = (o & 4) != 0, q2 = (o & 8) != 0;
    const int sh = o & 3;
    const uint32_t s0 = pick4(q1, q2, c[0], c[1], c[2], c[3]);
    const uint32_t s1 = pick4(q1, q2, c[1], c[2], c[3], n[0]);
    const uint32_t s2 = pick4(q1, q2, c[2], c[3], n[0], n[1]);
    const uint32_t s3 = pick4(q1, q2, c[3], n[0], n[1], n[2]);
    const uint32_t s4 = pick4(q1, q2, n[0], n[1], n[2], n[3]);
    return u32x4{__builtin_amdgcn_alignbyte(s1, s0, sh), __builtin_amdgcn_alignbyte(s2, s1, sh),
                 __builtin_amdgcn_alignbyte(s3, s2, sh), __builtin_amdgcn_alignbyte(s4, s3, sh)};
}

// The same cut for a compile-time O: fixed dword picks, and alignbyte only
// when O is not a multiple of 4 (2-byte elements at an odd element offset).
template <int O>
__device__ __forceinline__ u32x4 window_c(const u32x4& c, const u32x4& n)
{
    static_assert(O >= 0 && O < 16, "byte offset inside a word");
    const uint32_t s[8] = {c[0], c[1], c[2], c[3], n[0], n[1], n[2], n[3]};
    constexpr int q = O >> 2, sh = O & 3;
    if constexpr (sh == 0)
        return u32x4{s[q], s[q + 1], s[q + 2], s[q + 3]};
    else
        return u32x4{__builtin_amdgcn_alignbyte(s[q + 1], s[q], sh),
                     __builtin_amdgcn_alignbyte(s[q + 2], s[q + 1], sh),
                     __builtin_amdgcn_alignbyte(s[q + 3], s[q + 2], sh),
                     __builtin_amdgcn_alignbyte(s[q + 4], s[q + 3], sh)};
}

// A byte offset as a type: O in 0..15, or -1 for one known only at run time.
template <int O>
struct Offset {
    static constexpr int value = O;
};

// window_c<O> where the offset is fixed, else window_at with the run-time o.
template <int O>
__device__ __forceinline__ u32x4 window_o(const u32x4& c, const u32x4& n, int o)
{
    if constexpr (O >= 0)
        return window_c<O>(c, n);
    else
        return window_at(c, n, o);
}

// f(Offset<o>{}) for a wave-uniform byte offset o: one scalar branch, then
// straight-line code for that offset, where window_at spends 15 selects
// per word on an offset known only at run time. Runs of 2- and 4-byte
// elements at element-aligned addresses have even offsets; an odd one
// (not reachable through the library's calls) takes the run-time form.
template <typename F>
__device__ __forceinline__ void dispatch_offset(int o, F&& f)
{
    switch (o) {
    case 0: f(Offset<0>{}); break;
    case 2: f(Offset<2>{}); break;
    case 4: f(Offset<4>{}); break;
    case 6: f(Offset<6>{}); break;
    case 8: f(Offset<8>{}); break;
    case 10: f(Offset<10>{}); break;
    case 12: f(Offset<12>{}); break;
    case 14: f(Offset<14>{}); break;
    default: f(Offset<-1>{}); break;
    }
}

// DPP wave shifts by one lane; a lane with no source keeps `fill`.
__device__ __forceinline__ u32x4 lane_from_next(const u32x4& v, const u32x4& fill)
{
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        o[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)fill[d], (int)v[d], 0x130 /* wave_shl1 */,
                                                     0xF, 0xF, false);
    return o;
}

__device__ __forceinline__ u32x4 lane_from_prev(const u32x4& v, const u32x4& fill)
{
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        o[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)fill[d], (int)v[d], 0x138 /* wave_shr1 */,
                                                     0xF, 0xF, false);
    return o;
}

__device__ __forceinline__ u32x4 read_lane(const u32x4& v, int lane)
{
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        o[d] = (uint32_t)__builtin_amdgcn_readlane((int)v[d], lane);
    return o;
}

__device__ __forceinline__ int start_offset(const void* p)
{
    return (int)(reinterpret_cast<uintptr_t>(p) & 15u);
}

// The 16-byte word holding p's first byte. Derived from p by pointer
// arithmetic (not through an integer) so the compiler keeps the global
// address space and emits global rather than flat accesses.
__device__ __forceinline__ const u32x4* aligned_down(const void* p)
{
    return reinterpret_cast<const u32x4*>(static_cast<const char*>(p) - start_offset(p));
}

__device__ __forceinline__ u32x4* aligned_down(void* p)
{
    return reinterpret_cast<u32x4*>(static_cast<char*>(p) - start_offset(p));
}

// The position of p's aligned window word 0 within its 128-byte line
// (0..7 words). Access instructions that start at window word 64j - lead
// cover whole lines: an instruction that straddles nine lines instead of
// eight costs the memory system one more request per instruction, and a
// line two workgroups (often on different XCDs, with their own L2s) each
// touch part of is fetched twice.
__device__ __forceinline__ int line_lead(const void* p)
{
    return (int)((reinterpret_cast<uintptr_t>(p) >> 4) & 7u);
}

// Word i at w0, which every lane of the wave reads (a run's extra word),
// through the vector memory path: at a wave-uniform index the compiler
// would issue a scalar load instead, which reads the line through the
// scalar cache apart from the run's vector loads of it.
__device__ __forceinline__ u32x4 load16_uniform(const u32x4* w0, int i)
{
    __asm__ volatile("" : "+v"(i));
    return load16(w0 + i);
}

// Words of a run of n >= 1 2-byte elements at p into w[0..K) and extra, at
// a wave-uniform phase s (0..7): lane t, slot k holds window word
// 64k + t - s, and extra (every lane) word 64K - s. With s the window's
// line_lead each slot's access instruction covers whole 128-byte lines;
// realign_in then leaves group 64k + t - s in lane t, slot k.
template <int K, bool STREAM>
__device__ __forceinline__ void load_run(const void* p, int n, u32x4 (&w)[K], u32x4& extra,
                                         int phase = 0)
{
    const int lane = threadIdx.x & 63;
    const int m = start_offset(p);
    const u32x4* w0 = aligned_down(p);
    const int count = (m + 2 * n + 15) >> 4;  // n >= 1
    // indexes outside the window re-read its first or last word (a clamp
    // rather than a branch, which would wait for each load before the
    // next): those values only reach elements outside the run, never summed
    // nor stored
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = lane + 64 * k - phase;
        const int ic = i < 0 ? 0 : (i < count ? i : count - 1);
        w[k] = STREAM ? load16_stream(w0 + ic) : load16(w0 + ic);
    }
    const int ie = 64 * K - phase;
    extra = load16_uniform(w0, ie < count ? ie : count - 1);
}

// Slots of a run from which realign_in uses the run-time cut (register use;
// measured on MI355X at 12 and 16 slots: only 16 gained).
constexpr int kRealignRuntimeSlots = 16;

// Words of slots k0 .. k0 + KB - 1 of the run into w[0..KB) (as load_run),
// and in extra the word that completes the last of them: slot k0 + KB's
// first word, or the window's last word.
template <int KB, bool STREAM>
__device__ __forceinline__ void load_run_at(const void* p, int n, int k0, u32x4 (&w)[KB],
                                            u32x4& extra)
{
    const int lane = threadIdx.x & 63;
    const int m = start_offset(p);
    const u32x4* w0 = aligned_down(p);
    const int count = (m + 2 * n + 15) >> 4;  // n >= 1
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        const int i = lane + 64 * (k0 + j);
        const int ic = i < count ? i : count - 1;
        w[j] = STREAM ? load16_stream(w0 + ic) : load16(w0 + ic);
    }
    const int ie = 64 * (k0 + KB);
    extra = load16_uniform(w0, ie < count ? ie : count - 1);
}

// Words -> groups, in place (m = the run's start offset).
template <int K>
__device__ __forceinline__ void realign_in(u32x4 (&w)[K], const u32x4& extra, int m)
{
    // at 16 slots the run-time cut: the branch to code for each offset held
    // ~60 more registers there (1 wave per SIMD instead of 2, 17-22 % slower)
    if constexpr (K >= kRealignRuntimeSlots) {
        if (m == 0)
            return;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const u32x4 fill = (k + 1 < K) ? read_lane(w[k + 1 < K ? k + 1 : k], 0) : extra;
            w[k] = window_at(w[k], lane_from_next(w[k], fill), m);
        }
        return;
    }
    dispatch_offset(m, [&](auto off) {
        constexpr int O = decltype(off)::value;
        if constexpr (O != 0) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const u32x4 fill = (k + 1 < K) ? read_lane(w[k + 1 < K ? k + 1 : k], 0) : extra;
                w[k] = window_o<O>(w[k], lane_from_next(w[k], fill), m);
            }
        }
    });
}

// Groups of a run at phase s (load_run): lane t, slot k holds group
// 64k + t - s.
template <int K, bool STREAM>
__device__ __forceinline__ void load_groups(const void* p, int n, u32x4 (&g)[K], int phase = 0)
{
    u32x4 extra;
    load_run<K, STREAM>(p, n, g, extra, phase);
    realign_in<K>(g, extra, start_offset(p));
}

// The bytes of output word i inside the run [mo, end) of the window at
// w0, as 2-byte stores (every element size here is a multiple of 2 and
// every run boundary a multiple of the element size): the chunked kernels'
// edge words (few, and compact code where it is inlined at many sites).
__device__ __forceinline__ void put_partial(u32x4* w0, int64_t i, const u32x4& v, int64_t mo,
                                            int64_t end)
{
    const int64_t lo = 16 * i;
    unsigned char* gb = reinterpret_cast<unsigned char*>(w0);
    const int b0 = (int)((lo > mo ? lo : mo) - lo);
    const int b1 = (int)((lo + 16 < end ? lo + 16 : end) - lo);
    for (int j = b0; j < b1; j += 2) {
        const uint32_t dw = j < 8 ? (j < 4 ? v[0] : v[1]) : (j < 12 ? v[2] : v[3]);
        *reinterpret_cast<uint16_t*>(gb + lo + j) = (uint16_t)(dw >> (8 * (j & 2)));
    }
}

// The same bytes with the widest aligned stores that fit them: a 2-byte
// store up to a 4-byte boundary, a 4-byte one up to an 8-byte boundary, an
// 8-byte one, then what is left (at most four store instructions where two
// bytes at a time took up to seven; they cover any run of up to 14 bytes,
// and a partial word holds at most 14): the register rows' first and last
// words, one lane each per row. (Inlined into the chunked kernels' many
// store sites instead, it grew the 8-wave LDS row kernel by a third.)
__device__ __forceinline__ void put_partial_wide(u32x4* w0, int64_t i, const u32x4& v, int64_t mo,
                                                 int64_t end)
{
    const int64_t lo = 16 * i;
    unsigned char* gb = reinterpret_cast<unsigned char*>(w0) + lo;
    int b = (int)((lo > mo ? lo : mo) - lo);
    const int b1 = (int)((lo + 16 < end ? lo + 16 : end) - lo);
    // the dword holding byte j of the word
    auto dw = [&](int j) { return j < 8 ? (j < 4 ? v[0] : v[1]) : (j < 12 ? v[2] : v[3]); };
    if ((b & 2) != 0 && b < b1) {
        *reinterpret_cast<uint16_t*>(gb + b) = (uint16_t)(dw(b) >> 16);
        b += 2;
    }
    if ((b & 4) != 0 && b + 4 <= b1) {
        *reinterpret_cast<uint32_t*>(gb + b) = dw(b);
        b += 4;
    }
    if (b + 8 <= b1) {
        *reinterpret_cast<uint2*>(gb + b) = make_uint2(dw(b), dw(b + 4));
        b += 8;
    }
    if (b + 4 <= b1) {
        *reinterpret_cast<uint32_t*>(gb + b) = dw(b);
        b += 4;
    }
    if (b < b1)
        *reinterpret_cast<uint16_t*>(gb + b) = (uint16_t)dw(b);
}

// Output word i of the run [mo, end): one 16-byte store when it lies wholly
// inside the run, else its bytes inside the run (none for i < 0).
template <bool STREAM>
__device__ __forceinline__ void put_word(u32x4* w0, int64_t i, const u32x4& v, int64_t mo,
                                         int64_t end)
{
    const int64_t lo = 16 * i;
    if (lo >= end)
        return;
    if (lo >= mo && lo + 16 <= end) {
        if (STREAM)
            store16_stream(w0 + i, v);
        else
            w0[i] = v;
        return;
    }
    put_partial(w0, i, v, mo, end);
}

// Groups at phase s (lane t, slot k: group 64k + t - s) -> the n elements
// of a run at p: output word w joins groups w - 1 and w (cut at 16 - mo), so
// lane t, slot k forms word 64k + t - s (whole 128-byte lines per slot when
// s is the output window's line_lead). Whole words are stored in the slot
// loop; the run's first word (when mo > 0) and last word (when the run does
// not end on a word boundary) are the only partial ones and are written
// after it. The phase is below 64, so word 0 is in slot 0; the last word's
// slot is known to the whole wave, so neither is picked out lane by lane
// in every slot.
template <int K, bool STREAM>
__device__ __forceinline__ void store_run(void* p, int n, const u32x4 (&g)[K], int phase = 0)
{
    if (n <= 0)
        return;
    const int lane = threadIdx.x & 63;
    const int mo = start_offset(p);
    u32x4* w0 = aligned_down(p);
    const int end = mo + 2 * n;
    const int words = (end + 15) >> 4;
    const int wl = words - 1;
    const int kl = (wl + phase) >> 6;  // the slot of word wl (K: the tail below)
    u32x4 first = u32x4{0, 0, 0, 0}, last = u32x4{0, 0, 0, 0};
    dispatch_offset(mo, [&](auto off) {
        constexpr int O = decltype(off)::value;
        // the cut at 16 - mo, fixed with mo
        constexpr int C = O > 0 ? 16 - O : -1;
        u32x4 fill = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            u32x4 v = g[k];
            if constexpr (O != 0)
                v = window_o<C>(lane_from_prev(g[k], fill), g[k], 16 - mo);
            fill = read_lane(g[k], 63);
            const int w = lane + 64 * k - phase;
            if (16 * w >= mo && 16 * w + 16 <= end) {
                if (STREAM)
                    store16_stream(w0 + w, v);
                else
                    w0[w] = v;
            }
            if (k == 0)
                first = v;
            if (k == kl)
                last = v;
        }
        // word 64K - s (only reached when mo > 0): the tail of the last
        // slot's lane 63 group
        if constexpr (O != 0)
            if (kl == K)
                last = window_o<C>(fill, u32x4{0, 0, 0, 0}, 16 - mo);
    });
    const bool last_partial = (end & 15) != 0;
    if (lane == phase && mo != 0)
        put_partial_wide(w0, 0, first, mo, end);
    if (last_partial && lane == ((wl + phase) & 63) && !(wl == 0 && mo != 0))
        put_partial_wide(w0, wl, last, mo, end);
}

// ---- Output-aligned chunks -----------------------------------------------
//
// An element-wise result over a run of nbytes bytes written at po is cut
// into chunks of 64 words of po's aligned window: lane t of the chunk that
// starts at window word wbase owns output word wbase + t (words before the
// window's start are owned by no one and not written). Only the window's first and last words can be
// partial, so only they are written element by element, every other word
// is one 16-byte store, and no two waves write the same word. An input run
// at its own start offset mi is read so that each lane gets the input bytes
// that line up with its output word: for d = mi - mo, output bytes
// [16w - mo, 16w - mo + 16) of the run are input window bytes
// [16w + d, 16w + d + 16), i.e. words w + floor(d / 16) and the next one
// (a DPP shift brings the next lane's word; lane 63 takes one more word
// loaded by every lane), cut at d mod 16. Indexes outside the input's
// window are clamped to its first or last word; the bytes they supply fall
// outside the run.
// The same byte-level realignment serves every element size.

__device__ __forceinline__ int64_t window_words(const void* p, int64_t nbytes)
{
    return nbytes > 0 ? (start_offset(p) + nbytes + 15) >> 4 : 0;
}


// The words an input supplies to lane t of chunk j, fetched (every load
// issued, none waited on) so that a caller can fetch all its inputs before
// realigning any: a branch between fetches made the compiler wait for each
// input's loads before issuing the next input's.
struct ChunkWords {
    u32x4 cur, extra;
    int sh;
};

template <bool STREAM>
__device__ __forceinline__ ChunkWords fetch_for_chunk(const void* p, int64_t nbytes, int mo,
                                                      int64_t wbase)
{
    const int lane = threadIdx.x & 63;
    const int mi = start_offset(p);
    const u32x4* w0 = aligned_down(p);
    const int64_t count = window_words(p, nbytes);
    const int d = mi - mo;
    const int64_t q0 = wbase + (d < 0 ? -1 : 0);
    // indexes clamped into the input's window (no branch around the loads);
    // a clamped word only supplies bytes outside the run
    const int64_t i = q0 + lane;
    const int64_t ic = i < 0 ? 0 : (i < count ? i : count - 1);
    const int64_t ie = q0 + 64;
    ChunkWords r;
    r.cur = STREAM ? load16_stream(w0 + ic) : load16(w0 + ic);
    r.extra = load16(w0 + (ie < 0 ? 0 : (ie < count ? ie : count - 1)));
    r.sh = d < 0 ? d + 16 : d;
    return r;
}

// One word per lane: the run-time cut (selects) measured faster here than a
// branch to code for the offset, which slowed a chunked gated add by half.
__device__ __forceinline__ u32x4 chunk_word(const ChunkWords& w)
{
    return w.sh == 0 ? w.cur : window_at(w.cur, lane_from_next(w.cur, w.extra), w.sh);
}

template <bool STREAM>
__device__ __forceinline__ u32x4 load_for_chunk(const void* p, int64_t nbytes, int mo,
                                                int64_t wbase)
{
    return chunk_word(fetch_for_chunk<STREAM>(p, nbytes, mo, wbase));
}

template <bool STREAM>
__device__ __forceinline__ void store_chunk(void* p, int64_t nbytes, int64_t wbase, const u32x4& v)
{
    const int lane = threadIdx.x & 63;
    const int mo = start_offset(p);
    put_word<STREAM>(aligned_down(p), wbase + lane, v, mo, mo + nbytes);
}

// Elements of a 16-byte word: 8 of a 2-byte type, 4 binary32.
template <int DT>
struct Word {
    static constexpr int kN = DT == kF32 ? 4 : 8;
    __device__ __forceinline__ static float get(const u32x4& w, int e)
    {
        if constexpr (DT == kF32) {
            return __uint_as_float(w[e]);
        } else {
            Pack<DT> p;
            p.v = w;
            return p.get(e);
        }
    }
    __device__ __forceinline__ static u32x4 make(const float* f)
    {
        if constexpr (DT == kF32)
            return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                         __float_as_uint(f[3])};
        else
            return Pack<DT>::make(f).v;
    }
};

}  // namespace rga
