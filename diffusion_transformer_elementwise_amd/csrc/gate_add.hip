// Gated residual add, out = x + u * g, over contiguous [B, L, D]
// ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path for LTX2",
// "Motivation": full gate [B, L, D] or a gate row broadcast over L; its test
// list adds dtype coverage and tail shapes).
//
// Per element: p = u * g and s = x + p in binary32 (no contraction: the
// library is built with -ffp-contract=off), then one rounding to the storage
// type (bf16, binary16 or binary32; see dtype.hpp).
//
// Fast path (D % 8 == 0, every pointer 16-byte aligned). Launch shape,
// measured on MI355X: one wave64 per workgroup, one 8-element pack per lane
// and stream, nontemporal loads and stores. Many short waves spread over the
// 256 CUs keep the HBM request stream even; more packs per lane, larger
// workgroups and persistent grids all measured slower. Which 8 elements a
// lane holds does not matter here, so binary32 packs are lane-interleaved
// (Interleaved in dtype.hpp) for contiguous wave-wide accesses.
//
// Element path (any D, pointers aligned to the element size): the same
// arithmetic over chunks of the output's aligned 16-byte words, every input
// realigned to the output in registers (realign.hpp), for shapes the pack
// path cannot take.
//
// Every thread reads its own elements before writing them and no element
// depends on another, so out may alias x or u (and g in full mode).
#include "dtype.hpp"
#include "launch.hpp"
#include "realign.hpp"

#include <rga.h>
#include <rga_measure.h>

namespace rga {
namespace {

constexpr int kBlock = 64;   // one wave per workgroup

template <int DT>
__device__ __forceinline__ Pack<DT> gate_add8(const Pack<DT>& x,
                                              const Pack<DT>& u,
                                              const Pack<DT>& g)
{
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = u.get(e) * g.get(e);
        o[e] = x.get(e) + p;
    }
    return Pack<DT>::make(o);
}

// Full gate: a flat stream of n8 = floor(n / 8) packs plus n % 8 trailing
// elements (n = B*L*D; rows play no part). Workgroup w takes the chunk of
// packs 64w .. 64w + h - 1 (h = 64 but for the last chunk), lane t its share
// of it (see Interleaved); lane h of the last chunk (in a workgroup of its
// own when n8 is a multiple of 64) takes the trailing elements one by one.
template <int DT>
__global__ __launch_bounds__(kBlock) void gate_add_full_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t n8, int tail)
{
    const int64_t c0 = (int64_t)blockIdx.x * kBlock;
    const int t = threadIdx.x;
    const int h = (n8 - c0 < kBlock) ? (int)(n8 - c0) : kBlock;
    if (t < h) {
        using I = Interleaved<DT>;
        const Pack<DT> xv = I::load_stream(x, c0, t, h);
        const Pack<DT> uv = I::load_stream(u, c0, t, h);
        const Pack<DT> gv = I::load_stream(g, c0, t, h);
        I::store_stream(gate_add8<DT>(xv, uv, gv), out, c0, t, h);
    } else if (t == h && c0 + h == n8) {
        for (int e = 0; e < tail; ++e) {
            const int64_t i = 8 * n8 + e;
            const float p = load_elem<DT>(u, i) * load_elem<DT>(g, i);
            store_elem<DT>(out, i, load_elem<DT>(x, i) + p);
        }
    }
}

// Broadcast gate [B, 1, D]. Grid: x = (row l of the batch) * chunks + chunk,
// y = batch b, where a chunk is up to 64 packs of a row. The lanes of a
// chunk take its packs as in the full kernel; the matching gate packs come
// from row b of g, which stays in the caches while the streams of x, u and
// out pass through. With 2-byte storage, chunk c of a row covers its packs
// 64c - s .. 64c - s + 63, s the position of the output row's first pack in
// its 128-byte line (0 for rows of a multiple of 64 packs in a line-aligned
// tensor), so that each access instruction covers whole lines: on MI355X a
// 16-byte-aligned copy whose instructions each straddle one line more
// fetched 12.5 % more from HBM and ran 10-26 % slower. The launch gives
// each row enough chunks for that shift.
template <int DT>
__global__ __launch_bounds__(kBlock) void gate_add_bcast_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t L,
    uint32_t vpr, uint32_t chunks)
{
    const uint32_t l = blockIdx.x / chunks;
    const uint32_t chunk = blockIdx.x - l * chunks;
    const int t = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + l) * vpr;
    if constexpr (DT != kF32) {
        const int lead =
            (int)((reinterpret_cast<uintptr_t>(static_cast<const u32x4*>(out) + row) >> 4) & 7u);
        const int p = (int)(chunk * kBlock) + t - lead;
        if (p < 0 || p >= (int)vpr)
            return;
        const Pack<DT> xv = Pack<DT>::load_stream(x, row + p);
        const Pack<DT> uv = Pack<DT>::load_stream(u, row + p);
        const Pack<DT> gv = Pack<DT>::load(g, b * vpr + p);
        gate_add8<DT>(xv, uv, gv).store_stream(out, row + p);
    } else {
        const uint32_t col0 = chunk * kBlock;
        const int h = (vpr - col0 < (uint32_t)kBlock) ? (int)(vpr - col0) : kBlock;
        if (t >= h)
            return;
        const int64_t c0 = row + col0;
        using I = Interleaved<DT>;
        const Pack<DT> xv = I::load_stream(x, c0, t, h);
        const Pack<DT> uv = I::load_stream(u, c0, t, h);
        const Pack<DT> gv = I::load(g, b * vpr + col0, t, h);
        I::store_stream(gate_add8<DT>(xv, uv, gv), out, c0, t, h);
    }
}

// Chunks per row of gate_add_bcast_kernel: every row's packs at its line
// shift (up to 7 packs, 0 for rows that all start on a line).
uint32_t bcast_chunks(const void* out, int64_t D, int es)
{
    const int64_t vpr = D / 8;
    if (es == 4)
        return (uint32_t)((vpr + kBlock - 1) / kBlock);
    const bool rows_on_lines = (D * es) % 128 == 0;
    const int64_t lead = rows_on_lines ? (int64_t)((reinterpret_cast<uintptr_t>(out) >> 4) & 7u) : 7;
    return (uint32_t)((vpr + lead + kBlock - 1) / kBlock);
}

// Measurement variants of the bf16 broadcast-gate add (rga_gate_add_variant
// in rga_measure.h), same arithmetic and result as gate_add_bcast_kernel:
//   T rows per wave: the wave takes one 64-pack column chunk of T consecutive
//     rows and loads its gate pack once for all of them (the row tile of the
//     residual-gate page's Nsight Compute check); T = 1 is the library's
//     shape. Grid: x = (row tile) * chunks + chunk, y = batch.
//   SP, the stores' cache policy: RGA_STORE_NT (nontemporal, the library's),
//     RGA_STORE_PLAIN (default policy: lines stay dirty in the L2) or
//     RGA_STORE_DEVICE (device scope: written through the L2 into the
//     memory-side cache, which may keep them; a buffer store with the SC1
//     bit, whose descriptor covers exactly the chunk's valid bytes).
template <int SP>
__device__ __forceinline__ void store_with_policy(void* out, int64_t c0, int t, int h,
                                                  const u32x4& v)
{
    u32x4* p = static_cast<u32x4*>(out) + c0;
    if constexpr (SP == RGA_STORE_NT) {
        store16_stream(p + t, v);
    } else if constexpr (SP == RGA_STORE_PLAIN) {
        store16(p + t, v);
    } else {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(p, (short)0, h * 16, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, t * 16, 0, 16 /* SC1 */);
    }
}

template <int T, int SP>
__global__ __launch_bounds__(kBlock) void gate_add_bcast_rows_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t L,
    uint32_t vpr, uint32_t chunks)
{
    const uint32_t tile = blockIdx.x / chunks;
    const uint32_t chunk = blockIdx.x - tile * chunks;
    const uint32_t col0 = chunk * kBlock;
    const int t = threadIdx.x;
    const int h = (vpr - col0 < (uint32_t)kBlock) ? (int)(vpr - col0) : kBlock;
    if (t >= h)
        return;
    const int64_t b = blockIdx.y;
    const int64_t l0 = (int64_t)tile * T;
    const Pack<kBF16> gv = Pack<kBF16>::load(g, b * vpr + col0 + t);
    Pack<kBF16> xv[T], uv[T];
#pragma unroll
    for (int r = 0; r < T; ++r) {
        if (l0 + r < L) {
            const int64_t c0 = (b * L + l0 + r) * vpr + col0;
            xv[r] = Pack<kBF16>::load_stream(x, c0 + t);
            uv[r] = Pack<kBF16>::load_stream(u, c0 + t);
        }
    }
#pragma unroll
    for (int r = 0; r < T; ++r) {
        if (l0 + r < L)
            store_with_policy<SP>(out, (b * L + l0 + r) * vpr + col0, t, h,
                                  gate_add8<kBF16>(xv[r], uv[r], gv).v);
    }
}

template <int DT>
__device__ __forceinline__ u32x4 gate_add_word(const u32x4& x, const u32x4& u, const u32x4& g)
{
    using W = Word<DT>;
    float o[W::kN];
#pragma unroll
    for (int e = 0; e < W::kN; ++e) {
        const float p = W::get(u, e) * W::get(g, e);
        o[e] = W::get(x, e) + p;
    }
    return W::make(o);
}

// Element path (realign.hpp): a run of elements is cut into chunks of 64
// 16-byte words of the output's aligned window (whole 128-byte lines), one
// chunk per workgroup;
// each input is read realigned to the output's byte positions, so a lane
// computes the elements of exactly one output word.
template <int DT, bool G_STREAM>
__device__ __forceinline__ void gate_add_chunk(const void* x, const void* u, const void* g,
                                               void* out, int64_t nbytes, int64_t j)
{
    const int mo = start_offset(out);
    const int64_t wbase = 64 * j - line_lead(out);
    if (wbase >= window_words(out, nbytes))
        return;
    const ChunkWords fx = fetch_for_chunk<true>(x, nbytes, mo, wbase);
    const ChunkWords fu = fetch_for_chunk<true>(u, nbytes, mo, wbase);
    const ChunkWords fg = fetch_for_chunk<G_STREAM>(g, nbytes, mo, wbase);
    store_chunk<true>(out, nbytes, wbase,
                      gate_add_word<DT>(chunk_word(fx), chunk_word(fu), chunk_word(fg)));
}

template <int DT>
__device__ __forceinline__ const void* elem_ptr(const void* p, int64_t i)
{
    return static_cast<const char*>(p) + i * (DT == kF32 ? 4 : 2);
}

template <int DT>
__device__ __forceinline__ void* elem_ptr(void* p, int64_t i)
{
    return static_cast<char*>(p) + i * (DT == kF32 ? 4 : 2);
}

// Full gate: the flat B*L*D elements are one run; grid x = chunk.
template <int DT>
__global__ __launch_bounds__(kBlock) void gate_add_generic_full_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t nbytes)
{
    gate_add_chunk<DT, true>(x, u, g, out, nbytes, blockIdx.x);
}

// Broadcast gate: each row is a run, with row b of g as its gate run; grid
// x = (row l) * chunks per row + chunk, y = batch b. (Folding a ragged row's
// last word or two into another workgroup's loop measured slower: that
// workgroup then waits out two load-to-store latencies while holding its
// slot.)
template <int DT>
__global__ __launch_bounds__(kBlock) void gate_add_generic_bcast_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t L,
    int64_t D, uint32_t chunks)
{
    const uint32_t l = blockIdx.x / chunks;
    const uint32_t j = blockIdx.x - l * chunks;
    const int64_t b = blockIdx.y;
    const int64_t e0 = (b * L + l) * D;
    gate_add_chunk<DT, false>(elem_ptr<DT>(x, e0), elem_ptr<DT>(u, e0), elem_ptr<DT>(g, b * D),
                              elem_ptr<DT>(out, e0), D * (DT == kF32 ? 4 : 2), j);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunks of 64 output words that cover a run of nbytes at any start offset
// (at most 14 bytes into its first word), the first chunk starting up to 7
// words early (line_lead in realign.hpp).
int64_t element_chunks(int64_t nbytes) { return ceil_div(ceil_div(14 + nbytes, 16) + 7, 64); }

template <int DT>
hipError_t launch_typed(const void* x, const void* u, const void* g,
                        void* out, int64_t B, int64_t L, int64_t D,
                        int gate_mode, bool fast, hipStream_t stream)
{
    constexpr int es = DT == kF32 ? 4 : 2;
    if (!fast) {
        if (gate_mode == RGA_GATE_FULL) {
            int64_t nbytes = B * L * D * es;
            void* args[] = {&x, &u, &g, &out, &nbytes};
            return hipLaunchKernel(
                reinterpret_cast<const void*>(&gate_add_generic_full_kernel<DT>),
                dim3((uint32_t)element_chunks(nbytes)), dim3(kBlock), args, 0, stream);
        }
        uint32_t chunks = (uint32_t)element_chunks(D * es);
        void* args[] = {&x, &u, &g, &out, &L, &D, &chunks};
        return hipLaunchKernel(
            reinterpret_cast<const void*>(&gate_add_generic_bcast_kernel<DT>),
            dim3((uint32_t)(L * chunks), (uint32_t)B), dim3(kBlock), args, 0, stream);
    }
    if (gate_mode == RGA_GATE_FULL) {
        const int64_t n = B * L * D;
        int64_t n8 = n / 8;
        int tail = (int)(n % 8);
        void* args[] = {&x, &u, &g, &out, &n8, &tail};
        return hipLaunchKernel(
            reinterpret_cast<const void*>(&gate_add_full_kernel<DT>),
            dim3((uint32_t)ceil_div(n8 + (tail ? 1 : 0), kBlock)), dim3(kBlock), args, 0,
            stream);
    }
    uint32_t vpr = (uint32_t)(D / 8);
    uint32_t chunks = bcast_chunks(out, D, es);
    void* args[] = {&x, &u, &g, &out, &L, &vpr, &chunks};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&gate_add_bcast_kernel<DT>),
        dim3((uint32_t)(L * chunks), (uint32_t)B), dim3(kBlock), args, 0,
        stream);
}

}  // namespace

// AMD dispatch packets carry the grid size in work-items per dimension as
// 32-bit numbers; HIP grids stop at 65535 workgroups in y.
bool gate_add_grid_fits(int64_t B, int64_t L, int64_t D, int gate_mode, int es,
                        bool fast)
{
    const int64_t max_wg = (((int64_t)1 << 32) - 1) / kBlock;
    if (gate_mode == RGA_GATE_FULL)  // one flat grid dimension, B plays no part
        return fast ? ceil_div(B * L * D / 8 + 1, kBlock) <= max_wg
                    : element_chunks(B * L * D * es) <= max_wg;
    if (B > 65535)  // grid y
        return false;
    // the pack kernel's chunks per row, at most one more for the line shift
    return fast ? L * (ceil_div(D / 8, kBlock) + 1) <= max_wg
                : L * element_chunks(D * es) <= max_wg;
}

bool gate_add_variant_grid_fits(int64_t B, int64_t L, int64_t D, int rows_per_wave)
{
    const int64_t max_wg = (((int64_t)1 << 32) - 1) / kBlock;
    return B <= 65535 && ceil_div(L, rows_per_wave) * ceil_div(D / 8, kBlock) <= max_wg;
}

template <int T>
const void* variant_kernel(int store_policy)
{
    switch (store_policy) {
    case RGA_STORE_PLAIN:
        return reinterpret_cast<const void*>(&gate_add_bcast_rows_kernel<T, RGA_STORE_PLAIN>);
    case RGA_STORE_DEVICE:
        return reinterpret_cast<const void*>(&gate_add_bcast_rows_kernel<T, RGA_STORE_DEVICE>);
    default:
        return reinterpret_cast<const void*>(&gate_add_bcast_rows_kernel<T, RGA_STORE_NT>);
    }
}

hipError_t launch_gate_add_variant(const void* x, const void* u, const void* g, void* out,
                                   int64_t B, int64_t L, int64_t D, int rows_per_wave,
                                   int store_policy, hipStream_t stream)
{
    const void* k = rows_per_wave == 8   ? variant_kernel<8>(store_policy)
                    : rows_per_wave == 4 ? variant_kernel<4>(store_policy)
                    : rows_per_wave == 2 ? variant_kernel<2>(store_policy)
                                         : variant_kernel<1>(store_policy);
    uint32_t vpr = (uint32_t)(D / 8);
    uint32_t chunks = (uint32_t)ceil_div(vpr, kBlock);
    void* args[] = {&x, &u, &g, &out, &L, &vpr, &chunks};
    return hipLaunchKernel(k, dim3((uint32_t)(ceil_div(L, rows_per_wave) * chunks), (uint32_t)B),
                           dim3(kBlock), args, 0, stream);
}

hipError_t launch_gate_add(const void* x, const void* u, const void* g,
                           void* out, int64_t B, int64_t L, int64_t D,
                           int gate_mode, int dtype, bool fast,
                           hipStream_t stream)
{
    switch (dtype) {
    case RGA_DTYPE_F16:
        return launch_typed<kF16>(x, u, g, out, B, L, D, gate_mode, fast, stream);
    case RGA_DTYPE_F32:
        return launch_typed<kF32>(x, u, g, out, B, L, D, gate_mode, fast, stream);
    default:
        return launch_typed<kBF16>(x, u, g, out, B, L, D, gate_mode, fast, stream);
    }
}

}  // namespace rga
