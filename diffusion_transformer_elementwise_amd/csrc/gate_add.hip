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
// workgroups and persistent grids all measured slower.
//
// Generic path (any D, pointers aligned to the element size): one element per
// thread, same arithmetic, for shapes the fast path cannot take.
//
// Every thread reads its own elements before writing them and no element
// depends on another, so out may alias x or u (and g in full mode).
#include "dtype.hpp"
#include "launch.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;           // fast path: one wave per workgroup
constexpr int kGenericBlock = 256;   // generic path: elements per workgroup

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

// Full gate: a flat stream of n8 = B*L*D/8 packs; lane t of workgroup w
// takes pack w*64 + t.
template <int DT>
__global__ __launch_bounds__(kBlock) void gate_add_full_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n8)
        return;
    const Pack<DT> xv = Pack<DT>::load_stream(x, i);
    const Pack<DT> uv = Pack<DT>::load_stream(u, i);
    const Pack<DT> gv = Pack<DT>::load_stream(g, i);
    gate_add8<DT>(xv, uv, gv).store_stream(out, i);
}

// Broadcast gate [B, 1, D]. Grid: x = (row l of the batch) * chunks + chunk,
// y = batch b, where a chunk is 64 packs of a row. Lane t handles pack
// chunk*64 + t of row (b, l); its gate pack comes from row b of g, which
// stays in the caches while the streams of x, u and out pass through.
template <int DT>
__global__ __launch_bounds__(kBlock) void gate_add_bcast_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t L,
    uint32_t vpr, uint32_t chunks)
{
    const uint32_t l = blockIdx.x / chunks;
    const uint32_t chunk = blockIdx.x - l * chunks;
    const uint32_t col = chunk * kBlock + threadIdx.x;
    if (col >= vpr)
        return;
    const int64_t b = blockIdx.y;
    const int64_t i = (b * L + l) * vpr + col;
    const Pack<DT> xv = Pack<DT>::load_stream(x, i);
    const Pack<DT> uv = Pack<DT>::load_stream(u, i);
    const Pack<DT> gv = Pack<DT>::load(g, b * vpr + col);
    gate_add8<DT>(xv, uv, gv).store_stream(out, i);
}

// Generic: grid x = (row l) * cD + c, y = batch b; element d = c*256 + t.
template <int DT, bool FULL>
__global__ __launch_bounds__(kGenericBlock) void gate_add_generic_kernel(
    const void* x, const void* u, const void* g, void* out, int64_t L,
    int64_t D, uint32_t cD)
{
    const uint32_t l = blockIdx.x / cD;
    const uint32_t c = blockIdx.x - l * cD;
    const int64_t d = (int64_t)c * kGenericBlock + threadIdx.x;
    if (d >= D)
        return;
    const int64_t b = blockIdx.y;
    const int64_t i = (b * L + l) * D + d;
    const float p = load_elem<DT>(u, i) * load_elem<DT>(g, FULL ? i : b * D + d);
    const float s = load_elem<DT>(x, i) + p;
    store_elem<DT>(out, i, s);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int DT>
hipError_t launch_typed(const void* x, const void* u, const void* g,
                        void* out, int64_t B, int64_t L, int64_t D,
                        int gate_mode, bool fast, hipStream_t stream)
{
    if (!fast) {
        uint32_t cD = (uint32_t)ceil_div(D, kGenericBlock);
        void* args[] = {&x, &u, &g, &out, &L, &D, &cD};
        const void* k = gate_mode == RGA_GATE_FULL
                            ? reinterpret_cast<const void*>(&gate_add_generic_kernel<DT, true>)
                            : reinterpret_cast<const void*>(&gate_add_generic_kernel<DT, false>);
        return hipLaunchKernel(k, dim3((uint32_t)(L * cD), (uint32_t)B),
                               dim3(kGenericBlock), args, 0, stream);
    }
    if (gate_mode == RGA_GATE_FULL) {
        int64_t n8 = B * L * D / 8;
        void* args[] = {&x, &u, &g, &out, &n8};
        return hipLaunchKernel(
            reinterpret_cast<const void*>(&gate_add_full_kernel<DT>),
            dim3((uint32_t)ceil_div(n8, kBlock)), dim3(kBlock), args, 0,
            stream);
    }
    uint32_t vpr = (uint32_t)(D / 8);
    uint32_t chunks = (uint32_t)ceil_div(vpr, kBlock);
    void* args[] = {&x, &u, &g, &out, &L, &vpr, &chunks};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&gate_add_bcast_kernel<DT>),
        dim3((uint32_t)(L * chunks), (uint32_t)B), dim3(kBlock), args, 0,
        stream);
}

}  // namespace

// AMD dispatch packets carry the grid size in work-items per dimension as
// 32-bit numbers; HIP grids stop at 65535 workgroups in y.
bool gate_add_grid_fits(int64_t B, int64_t L, int64_t D, int gate_mode,
                        bool fast)
{
    const int64_t max_x = (((int64_t)1 << 32) - 1);
    if (B > 65535)
        return false;
    if (!fast)
        return L * ceil_div(D, kGenericBlock) <= max_x / kGenericBlock;
    const int64_t vpr = D / 8;
    if (gate_mode == RGA_GATE_FULL)
        return ceil_div(B * L * vpr, kBlock) <= max_x / kBlock;
    return L * ceil_div(vpr, kBlock) <= max_x / kBlock;
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
