// Gated residual add, out = x + u * g, over contiguous bf16 [B, L, D]
// ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path for LTX2",
// "Motivation": full gate [B, L, D] or a gate row broadcast over L).
//
// Per element: p = u * g and s = x + p in binary32 (no contraction: the
// library is built with -ffp-contract=off), then one bf16 rounding.
//
// Launch shape (measured on MI355X): one wave64 per workgroup, one 16-byte vector per lane and stream,
// nontemporal loads and stores. Many short waves spread over the 256 CUs
// keep the HBM request stream even; more vectors per lane, larger
// workgroups and persistent grids all measured slower. Every lane reads its
// own elements before writing them and no element depends on another, so
// out may alias x or u (and g in full mode).
#include "bf16x8.hpp"
#include "launch.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;  // one wave per workgroup

__device__ __forceinline__ u32x4 gate_add8(u32x4 x, u32x4 u, u32x4 g)
{
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p0 = bf16_lo(u[i]) * bf16_lo(g[i]);
        const float p1 = bf16_hi(u[i]) * bf16_hi(g[i]);
        const float s0 = bf16_lo(x[i]) + p0;
        const float s1 = bf16_hi(x[i]) + p1;
        o[i] = pack_bf16(s0, s1);
    }
    return o;
}

// Full gate: a flat stream of n8 = B*L*D/8 vectors; lane t of workgroup w
// takes vector w*64 + t.
__global__ __launch_bounds__(kBlock) void gate_add_full_kernel(
    const u32x4* x, const u32x4* u, const u32x4* g, u32x4* out, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n8)
        return;
    const u32x4 xv = load16_stream(x + i);
    const u32x4 uv = load16_stream(u + i);
    const u32x4 gv = load16_stream(g + i);
    store16_stream(out + i, gate_add8(xv, uv, gv));
}

// Broadcast gate [B, 1, D]. Grid: x = (row l of the batch) * chunks + chunk,
// y = batch b, where a chunk is 64 vectors (512 elements) of a row. Lane t
// handles column vector chunk*64 + t of row (b, l); its gate vector comes
// from row b of g, which stays in the caches (8 KiB for D = 4096) while the
// streams of x, u and out pass through.
__global__ __launch_bounds__(kBlock) void gate_add_bcast_kernel(
    const u32x4* x, const u32x4* u, const u32x4* g, u32x4* out, int64_t L,
    uint32_t vpr, uint32_t chunks)
{
    const uint32_t l = blockIdx.x / chunks;
    const uint32_t chunk = blockIdx.x - l * chunks;
    const uint32_t col = chunk * kBlock + threadIdx.x;
    if (col >= vpr)
        return;
    const int64_t b = blockIdx.y;
    const int64_t i = (b * L + l) * vpr + col;
    const u32x4 xv = load16_stream(x + i);
    const u32x4 uv = load16_stream(u + i);
    const u32x4 gv = load16(g + b * vpr + col);
    store16_stream(out + i, gate_add8(xv, uv, gv));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// AMD dispatch packets carry the grid size in work-items per dimension as
// 32-bit numbers; HIP grids stop at 65535 workgroups in y.
static constexpr int64_t kMaxBlocksX = (((int64_t)1 << 32) - 1) / kBlock;
static constexpr int64_t kMaxBlocksY = 65535;

bool gate_add_grid_fits(int64_t B, int64_t L, int64_t D, int gate_mode)
{
    const int64_t vpr = D / 8;
    if (gate_mode == RGA_GATE_FULL)
        return ceil_div(B * L * vpr, kBlock) <= kMaxBlocksX;
    return L * ceil_div(vpr, kBlock) <= kMaxBlocksX && B <= kMaxBlocksY;
}

hipError_t launch_gate_add(const void* x, const void* u, const void* g,
                           void* out, int64_t B, int64_t L, int64_t D,
                           int gate_mode, hipStream_t stream)
{
    const u32x4* xv = static_cast<const u32x4*>(x);
    const u32x4* uv = static_cast<const u32x4*>(u);
    const u32x4* gv = static_cast<const u32x4*>(g);
    u32x4* ov = static_cast<u32x4*>(out);
    if (gate_mode == RGA_GATE_FULL) {
        int64_t n8 = B * L * D / 8;
        void* args[] = {&xv, &uv, &gv, &ov, &n8};
        return hipLaunchKernel(
            reinterpret_cast<const void*>(&gate_add_full_kernel),
            dim3((uint32_t)ceil_div(n8, kBlock)), dim3(kBlock), args, 0,
            stream);
    }
    uint32_t vpr = (uint32_t)(D / 8);
    uint32_t chunks = (uint32_t)ceil_div(vpr, kBlock);
    void* args[] = {&xv, &uv, &gv, &ov, &L, &vpr, &chunks};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&gate_add_bcast_kernel),
        dim3((uint32_t)(L * chunks), (uint32_t)B), dim3(kBlock), args, 0,
        stream);
}

}  // namespace rga
