// Residual update followed by the next adaLN modulation, in one pass:
//   x_out = x + u * g                                   (gated residual add)
//   y     = rms_norm(x_out, eps) * (1 + scale) + shift  (weightless RMSNorm)
// The two steps follow each other in a DiT block: the residual-gate update of
// hidden_states ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path for
// LTX2", "Motivation") and the modulation of the updated hidden_states before
// the next sub-layer (prhub summary of sglang PR #34172, "关键源码片段", the
// adaLN sites of LTX2TransformerBlock.forward). Run separately they move
// 10 bytes per element (x, u in, x_out out; x_out in, y out) for bf16; fused,
// x_out is never read back: 8 bytes per element.
//
// Arithmetic is exactly that of the two separate operations: x_out is
// rounded to the storage type first, and the modulation works on the rounded
// values with the library's fixed reduction order (lane j accumulates groups
// j, j+64, ... of the row, then xor-distance lane exchanges 1..32), so the
// outputs are bit-identical to rga_residual_gate_add followed by
// rms_modulate.
//
// Fast path (D % 8 == 0, D <= RGA_RMS_MAX_D, 16-byte aligned pointers),
// launch shape measured on MI355X: one wave per workgroup and one row per
// wave, nontemporal loads and stores; each x_out pack is stored as soon as it
// is formed, and scale and shift are read only in the apply phase (through
// the caches for row modulation, streamed for per-token modulation), which
// keeps the wave at 79 registers for bf16 and D = 4096. A broadcast gate row
// is read through the caches (it stays in L2), a full gate streams from HBM
// like x and u.
//
// Generic path (any D, element-aligned pointers): the same operations in two
// passes over the row with element loads; the second pass re-reads x_out,
// which the same lane wrote in the first.
#include "dtype.hpp"
#include "launch.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;
constexpr int kStage = 2048;  // generic path: elements staged in LDS per step
constexpr int kSpan = 8;      // generic path: elements per lane in pass 2

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

// Grid: x = row l, y = batch b. G = packs per lane (at least ceil(D / 512));
// lanes past the row end hold zeros (they add +0 to a partial that is never
// -0 and store nothing).
template <int G, bool FULL, int DT, int MOD>
__global__ __launch_bounds__(kBlock) void gate_add_rms_modulate_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int vpr)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * vpr;

    // the residual update is element-wise: raw order (see Grouped); only the
    // rounded x' that feeds the ordered sum goes to group order. Every lane
    // runs every pack (binary32 packs trade data across lanes); packs past
    // the row end load as zeros and are not stored.
    using GP = Grouped<DT>;
    Pack<DT> xn[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int h = vpr - 64 * i;
        const Pack<DT> xv = GP::load_stream_raw(x, row + 64 * i, lane, h);
        const Pack<DT> uv = GP::load_stream_raw(u, row + 64 * i, lane, h);
        const Pack<DT> gv = FULL ? GP::load_stream_raw(g, row + 64 * i, lane, h)
                                 : GP::load_raw(g, b * vpr + 64 * i, lane, h);
        const Pack<DT> xr = gate_add8<DT>(xv, uv, gv);
        GP::store_stream_raw(xr, x_out, row + 64 * i, lane, h);
        xn[i] = GP::to_groups(xr);
    }

    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = xn[i].get(e);
            const float sa = a * a;
            acc = acc + sa;
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
        const int h = vpr - 64 * i;
        const Pack<DT> xr = GP::to_raw(xn[i]);
        const Pack<DT> sc = MOD == kModToken ? GP::load_stream_raw(scale, row + 64 * i, lane, h)
                                             : GP::load_raw(scale, b * vpr + 64 * i, lane, h);
        const Pack<DT> sh = MOD == kModToken ? GP::load_stream_raw(shift, row + 64 * i, lane, h)
                                             : GP::load_raw(shift, b * vpr + 64 * i, lane, h);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float n = xr.get(e) * rr;
            const float a = 1.0f + sc.get(e);
            const float m = n * a;
            o[e] = m + sh.get(e);
        }
        GP::store_stream_raw(Pack<DT>::make(o), y, row + 64 * i, lane, h);
    }
}

// Generic: one wave per row; grid x = row l, y = batch b. Pass 1 walks the
// row in stages of kStage elements: wave-contiguous loads (lane t takes
// elements 64e + t), x_out formed and stored, its rounded values staged in
// LDS, from where lane j adds up groups j, j + 64, ... of the stage in the
// fixed order. Pass 2 re-reads x_out (each lane the elements it wrote) and
// writes y.
template <bool FULL, int DT, int MOD>
__global__ __launch_bounds__(kBlock) void gate_add_rms_modulate_generic_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int64_t D)
{
    __shared__ float stage[kStage];
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t grow = FULL ? row : b * D;
    const int64_t mrow = (MOD == kModToken) ? row : b * D;

    float acc = 0.0f;
    for (int64_t s0 = 0; s0 < D; s0 += kStage) {
        float xv[kStage / kBlock], uv[kStage / kBlock], gv[kStage / kBlock];
#pragma unroll
        for (int e = 0; e < kStage / kBlock; ++e) {
            const int64_t d = s0 + e * kBlock + lane;
            const bool in = d < D;
            xv[e] = in ? load_elem_stream<DT>(x, row + d) : 0.0f;
            uv[e] = in ? load_elem_stream<DT>(u, row + d) : 0.0f;
            gv[e] = in ? (FULL ? load_elem_stream<DT>(g, grow + d) : load_elem<DT>(g, grow + d))
                       : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < kStage / kBlock; ++e) {
            const int64_t d = s0 + e * kBlock + lane;
            const float p = uv[e] * gv[e];
            const float sum = xv[e] + p;
            if (d < D)
                store_elem<DT>(x_out, row + d, sum);
            stage[e * kBlock + lane] = rounded<DT>(sum);
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < kStage / 512; ++m) {
            const int g0 = (lane + kBlock * m) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (s0 + g0 + e < D) {
                    const float a = stage[g0 + e];
                    const float sa = a * a;
                    acc = acc + sa;
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        acc = acc + __shfl_xor(acc, m);
    const float ms = acc / d_float;
    const float t = ms + eps;
    const float q = sqrtf(t);
    const float rr = 1.0f / q;

    for (int64_t s0 = 0; s0 < D; s0 += kBlock * kSpan) {
        float xv[kSpan], sv[kSpan], hv[kSpan];
#pragma unroll
        for (int e = 0; e < kSpan; ++e) {
            const int64_t d = s0 + e * kBlock + lane;
            const bool in = d < D;
            xv[e] = in ? load_elem<DT>(x_out, row + d) : 0.0f;
            sv[e] = in ? (MOD == kModToken ? load_elem_stream<DT>(scale, mrow + d)
                                           : load_elem<DT>(scale, mrow + d)) : 0.0f;
            hv[e] = in ? (MOD == kModToken ? load_elem_stream<DT>(shift, mrow + d)
                                           : load_elem<DT>(shift, mrow + d)) : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < kSpan; ++e) {
            const int64_t d = s0 + e * kBlock + lane;
            if (d < D) {
                const float n = xv[e] * rr;
                const float a = 1.0f + sv[e];
                const float m = n * a;
                store_elem_stream<DT>(y, row + d, m + hv[e]);
            }
        }
    }
}

typedef void (*fused_kernel_t)(const void*, const void*, const void*,
                               const void*, const void*, float, float, void*,
                               void*, int64_t, int);

constexpr int kLadder[] = {1, 2, 4, 6, 8, 12, 16};
static_assert(RGA_RMS_MAX_D / 512 == 16, "ladder tops out at RGA_RMS_MAX_D");

template <bool FULL, int DT, int MOD>
fused_kernel_t pick(int groups)
{
    fused_kernel_t t[] = {&gate_add_rms_modulate_kernel<1, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<2, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<4, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<6, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<8, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<12, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<16, FULL, DT, MOD>};
    for (int i = 0; i < 7; ++i)
        if (groups <= kLadder[i])
            return t[i];
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <bool FULL, int DT, int MOD>
hipError_t launch_typed(const void* x, const void* u, const void* g,
                        const void* scale, const void* shift, float eps,
                        void* x_out, void* y, int64_t B, int64_t L, int64_t D,
                        bool fast, hipStream_t stream)
{
    float d_float = (float)D;
    if (!fast) {
        void* args[] = {&x, &u, &g, &scale, &shift, &eps, &d_float, &x_out, &y, &L, &D};
        return hipLaunchKernel(
            reinterpret_cast<const void*>(&gate_add_rms_modulate_generic_kernel<FULL, DT, MOD>),
            dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args, 0, stream);
    }
    int vpr = (int)(D / 8);
    fused_kernel_t k = pick<FULL, DT, MOD>((int)ceil_div(vpr, 64));
    if (k == nullptr)
        return hipErrorInvalidValue;
    void* args[] = {&x, &u, &g, &scale, &shift, &eps, &d_float, &x_out, &y, &L, &vpr};
    return hipLaunchKernel(reinterpret_cast<const void*>(k),
                           dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args, 0,
                           stream);
}

template <int DT>
hipError_t launch_dt(const void* x, const void* u, const void* g,
                     const void* scale, const void* shift, float eps,
                     void* x_out, void* y, int64_t B, int64_t L, int64_t D,
                     int gate_mode, int mod_mode, bool fast, hipStream_t stream)
{
    const bool full = gate_mode == RGA_GATE_FULL;
    const bool token = mod_mode == RGA_MOD_TOKEN;
    if (full && token)
        return launch_typed<true, DT, kModToken>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream);
    if (full)
        return launch_typed<true, DT, kModRow>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream);
    if (token)
        return launch_typed<false, DT, kModToken>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream);
    return launch_typed<false, DT, kModRow>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream);
}

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
                                        int mod_mode, int dtype, bool fast,
                                        hipStream_t stream)
{
    switch (dtype) {
    case RGA_DTYPE_F16:
        return launch_dt<kF16>(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode, fast, stream);
    case RGA_DTYPE_F32:
        return launch_dt<kF32>(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode, fast, stream);
    default:
        return launch_dt<kBF16>(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode, fast, stream);
    }
}

}  // namespace rga
