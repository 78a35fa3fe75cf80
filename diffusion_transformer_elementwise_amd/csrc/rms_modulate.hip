// adaLN modulation with a weightless RMSNorm,
//   out = rms_norm(x, eps) * (1 + scale) + shift,
// over contiguous bf16 x [B, L, D] with scale and shift rows [B, 1, D]
// (prhub summary of sglang PR #34172, "关键源码片段": the expression and
// RMSNormNoWeight; "风险与影响": the fused kernel's one-ULP allowance).
//
// One wave64 owns one row at a time. Lane j loads the 16-byte groups
// k = j, j + 64, ..., (group k = elements 8k .. 8k+7), keeps them in
// registers, and accumulates their squares in increasing k and element
// order into one binary32 partial; the 64 partials are then combined with
// xor-distance lane exchanges 1, 2, ..., 32 (every lane ends with the same
// sum, because a + b == b + a bit for bit). That is the fixed order the
// library documents, so the result does not depend on the launch shape.
// Then r = 1 / sqrt(ss / D + eps) with IEEE division and square root, and
// each element becomes ((x * r) * (1 + scale)) + shift, rounded once to bf16.
//
// The row is read once from HBM and written once, with nontemporal loads
// and stores; scale and shift rows are loaded once per wave (two rows of one
// batch, one wave per workgroup: the shape that measured fastest on MI355X
// inside a chain of streaming kernels) and kept in registers. No LDS and no
// barrier: nothing crosses a wave.
#include "bf16x8.hpp"
#include "launch.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;      // one wave per workgroup
constexpr int kRowsPerWave = 2;
constexpr int kMaxGroups = RGA_RMS_MAX_D / 512;  // groups per lane

// G = groups per lane = ceil(D / 512). Lanes whose group index is past the
// row end load zeros, which add +0 to a partial that is never -0, so they
// change nothing.
// Grid: x = tile of kRowsPerWave rows, y = batch.
template <int G>
__global__ __launch_bounds__(kBlock) void rms_modulate_kernel(
    const u32x4* x, const u32x4* scale, const u32x4* shift, float eps,
    float d_float, u32x4* out, int64_t L, int vpr)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * kRowsPerWave;
    const int64_t r1 = (r0 + kRowsPerWave < L) ? r0 + kRowsPerWave : L;

    u32x4 sc[G], sh[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int col = lane + 64 * i;
        if (col < vpr) {
            sc[i] = load16(scale + b * vpr + col);
            sh[i] = load16(shift + b * vpr + col);
        } else {
            sc[i] = u32x4{0, 0, 0, 0};
            sh[i] = u32x4{0, 0, 0, 0};
        }
    }

    for (int64_t r = r0; r < r1; ++r) {
        const int64_t row = (b * L + r) * vpr;
        u32x4 xv[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int col = lane + 64 * i;
            xv[i] = (col < vpr) ? load16_stream(x + row + col)
                                : u32x4{0, 0, 0, 0};
        }

        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < G; ++i) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float a = bf16_lo(xv[i][w]);
                const float sa = a * a;
                acc = acc + sa;
                const float c = bf16_hi(xv[i][w]);
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
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float n0 = bf16_lo(xv[i][w]) * rr;
                const float n1 = bf16_hi(xv[i][w]) * rr;
                const float a0 = 1.0f + bf16_lo(sc[i][w]);
                const float a1 = 1.0f + bf16_hi(sc[i][w]);
                const float m0 = n0 * a0;
                const float m1 = n1 * a1;
                const float y0 = m0 + bf16_lo(sh[i][w]);
                const float y1 = m1 + bf16_hi(sh[i][w]);
                o[w] = pack_bf16(y0, y1);
            }
            store16_stream(out + row + col, o);
        }
    }
}

typedef void (*rms_kernel_t)(const u32x4*, const u32x4*, const u32x4*, float,
                             float, u32x4*, int64_t, int);

template <int... Gs>
struct KernelTable {
    static rms_kernel_t get(int g)
    {
        rms_kernel_t table[] = {&rms_modulate_kernel<Gs>...};
        return (g >= 1 && g <= (int)sizeof...(Gs)) ? table[g - 1] : nullptr;
    }
};

using Table = KernelTable<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15,
                          16>;
static_assert(kMaxGroups == 16, "table covers groups 1..16");

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool rms_modulate_grid_fits(int64_t B, int64_t L, int64_t D)
{
    (void)D;
    return ceil_div(L, kRowsPerWave) <= (((int64_t)1 << 32) - 1) / kBlock &&
           B <= 65535;
}

hipError_t launch_rms_modulate(const void* x, const void* scale,
                               const void* shift, float eps, void* out,
                               int64_t B, int64_t L, int64_t D,
                               hipStream_t stream)
{
    int vpr = (int)(D / 8);
    rms_kernel_t k = Table::get((int)ceil_div(vpr, 64));
    if (k == nullptr)
        return hipErrorInvalidValue;
    const u32x4* xv = static_cast<const u32x4*>(x);
    const u32x4* sv = static_cast<const u32x4*>(scale);
    const u32x4* hv = static_cast<const u32x4*>(shift);
    u32x4* ov = static_cast<u32x4*>(out);
    float d_float = (float)D;
    void* args[] = {&xv, &sv, &hv, &eps, &d_float, &ov, &L, &vpr};
    return hipLaunchKernel(reinterpret_cast<const void*>(k),
                           dim3((uint32_t)ceil_div(L, kRowsPerWave), (uint32_t)B),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace rga
