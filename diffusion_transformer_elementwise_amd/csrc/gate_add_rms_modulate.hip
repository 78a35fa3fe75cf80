// Residual update followed by the next adaLN modulation, in one pass:
//   x_out = x + u * g                                   (gated residual add)
//   y     = rms_norm(x_out, eps) * (1 + scale) + shift  (weightless RMSNorm)
// The two steps follow each other in a DiT block: the residual-gate update of
// hidden_states ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path for
// LTX2", "Motivation") and the modulation of the updated hidden_states before
// the next sub-layer (prhub summary of sglang PR #34172, "关键源码片段", the
// adaLN sites of LTX2TransformerBlock.forward). Run separately they move
// 10 bytes per element (x, u in, x_out out; x_out in, y out); fused, x_out is
// never read back: 8 bytes per element.
//
// Arithmetic is exactly that of the two separate operations: x_out is
// rounded to bf16 first, and the modulation works on the rounded values with
// the library's fixed reduction order (lane j accumulates groups j, j+64, ...
// of the row, then xor-distance lane exchanges 1..32), so the outputs are
// bit-identical to rga_residual_gate_add followed by rms_modulate.
//
// Launch shape (measured on MI355X): one wave per workgroup and one row per
// wave, nontemporal loads and stores; each x_out vector is stored as soon as
// it is formed, and scale and shift are read through the caches only in the
// apply phase, which keeps the wave at 79 registers for D = 4096. A
// broadcast gate row is read through the caches (it stays in L2), a full gate
// streams from HBM like x and u.
#include "bf16x8.hpp"
#include "launch.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;

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

// Grid: x = row l, y = batch b. G = ceil(D / 512) groups per lane; lanes
// past the row end hold zeros (they add +0 to a partial that is never -0
// and store nothing).
template <int G, bool FULL>
__global__ __launch_bounds__(kBlock) void gate_add_rms_modulate_kernel(
    const u32x4* x, const u32x4* u, const u32x4* g, const u32x4* scale,
    const u32x4* shift, float eps, float d_float, u32x4* x_out, u32x4* y,
    int64_t L, int vpr)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * vpr;
    const u32x4 zero = {0, 0, 0, 0};

    u32x4 xn[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int col = lane + 64 * i;
        if (col < vpr) {
            const u32x4 xv = load16_stream(x + row + col);
            const u32x4 uv = load16_stream(u + row + col);
            const u32x4 gv = FULL ? load16_stream(g + row + col)
                                  : load16(g + b * vpr + col);
            xn[i] = gate_add8(xv, uv, gv);
            store16_stream(x_out + row + col, xn[i]);
        } else {
            xn[i] = zero;
        }
    }

    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = bf16_lo(xn[i][w]);
            const float sa = a * a;
            acc = acc + sa;
            const float c = bf16_hi(xn[i][w]);
            const float sc2 = c * c;
            acc = acc + sc2;
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        acc = acc + __shfl_xor(acc, m);
    const float ms = acc / d_float;
    const float t = ms + eps;
    const float q = sqrtf(t);
    const float rr = 1.0f / q;

#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int col = lane + 64 * i;
        if (col >= vpr)
            continue;
        const u32x4 sc = load16(scale + b * vpr + col);
        const u32x4 sh = load16(shift + b * vpr + col);
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float n0 = bf16_lo(xn[i][w]) * rr;
            const float n1 = bf16_hi(xn[i][w]) * rr;
            const float a0 = 1.0f + bf16_lo(sc[w]);
            const float a1 = 1.0f + bf16_hi(sc[w]);
            const float m0 = n0 * a0;
            const float m1 = n1 * a1;
            const float y0 = m0 + bf16_lo(sh[w]);
            const float y1 = m1 + bf16_hi(sh[w]);
            o[w] = pack_bf16(y0, y1);
        }
        store16_stream(y + row + col, o);
    }
}

typedef void (*fused_kernel_t)(const u32x4*, const u32x4*, const u32x4*,
                               const u32x4*, const u32x4*, float, float,
                               u32x4*, u32x4*, int64_t, int);

template <bool FULL, int... Gs>
struct FusedTable {
    static fused_kernel_t get(int g)
    {
        fused_kernel_t table[] = {&gate_add_rms_modulate_kernel<Gs, FULL>...};
        return (g >= 1 && g <= (int)sizeof...(Gs)) ? table[g - 1] : nullptr;
    }
};

template <bool FULL>
using Table = FusedTable<FULL, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14,
                         15, 16>;
static_assert(RGA_RMS_MAX_D / 512 == 16, "table covers groups 1..16");

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool gate_add_rms_modulate_grid_fits(int64_t B, int64_t L, int64_t D)
{
    (void)D;
    return L <= (((int64_t)1 << 32) - 1) / kBlock && B <= 65535;
}

hipError_t launch_gate_add_rms_modulate(const void* x, const void* u,
                                        const void* g, const void* scale,
                                        const void* shift, float eps,
                                        void* x_out, void* y, int64_t B,
                                        int64_t L, int64_t D, int gate_mode,
                                        hipStream_t stream)
{
    int vpr = (int)(D / 8);
    const int groups = (int)ceil_div(vpr, 64);
    fused_kernel_t k = gate_mode == RGA_GATE_FULL ? Table<true>::get(groups)
                                                  : Table<false>::get(groups);
    if (k == nullptr)
        return hipErrorInvalidValue;
    const u32x4* xv = static_cast<const u32x4*>(x);
    const u32x4* uv = static_cast<const u32x4*>(u);
    const u32x4* gv = static_cast<const u32x4*>(g);
    const u32x4* sv = static_cast<const u32x4*>(scale);
    const u32x4* hv = static_cast<const u32x4*>(shift);
    u32x4* xo = static_cast<u32x4*>(x_out);
    u32x4* yo = static_cast<u32x4*>(y);
    float d_float = (float)D;
    void* args[] = {&xv, &uv, &gv, &sv, &hv, &eps, &d_float, &xo, &yo, &L, &vpr};
    return hipLaunchKernel(reinterpret_cast<const void*>(k),
                           dim3((uint32_t)L, (uint32_t)B),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace rga
