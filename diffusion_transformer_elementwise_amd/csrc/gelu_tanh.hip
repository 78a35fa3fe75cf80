// tanh-GELU over the FFN intermediate, out = gelu(x (+ bias)), x and out
// [rows, F] contiguous, bias an optional row [F] (prhub summary of sglang PR
// #34172, "关键源码片段": LTX2FeedForward.forward applies a tanh-approximated
// GELU to the output of proj_in; "实现拆解" item 1: it is one of the
// element-wise chains torch.compile fuses).
//
// gelu(h) = 0.5 h (1 + tanh(a)), a = sqrt(2/pi) (h + 0.044715 h^3), is
// evaluated as h * logistic(2a): 0.5 (1 + tanh(a)) equals 1 / (1 + e^-2a).
// With t = 2a and s = e^-|t| = 2^-|t log2 e| (never above 1, so never
// overflowing), logistic(t) is 1 / (1 + s) for t >= 0 and s / (1 + s) for
// t < 0, which keeps its relative accuracy where 1 + tanh(a) would cancel (h
// below about -4 in binary32). While t log2 e >= -126 the single form
// 1 / (1 + e^-t) is as accurate and cannot overflow, so a wave takes the
// split form only when one of its values lies below that (h below about
// -9.3). Every step is binary32 (the constants folded into t log2 e); the
// exponential is the hardware's v_exp_f32 (1 ulp), or the
// subnormal-preserving exp2f on the split form; the reciprocal is v_rcp_f32
// (1 ulp). The relative error of the
// binary32 result is at most about (6 + 4|t|) 2^-24, far inside half a bf16 or
// binary16 ULP, so after the one rounding to storage the result is the
// correctly rounded value or its neighbour. Limits: +inf -> +inf,
// -inf -> -0, NaN -> NaN; when logistic(t) underflows to 0 the result is a
// signed zero.
//
// At one pack per lane the kernel runs near both of its bounds on MI355X
// (HBM and the vector ALU, packed binary32 instructions being off), so the
// instruction count per element is kept low.
//
// With a bias row, h = x + bias in binary32 first (the bias add of a GEMM
// epilogue).
//
// Launch shapes follow the gated residual add (measured there on MI355X):
// one wave per workgroup, one 8-element pack per lane, nontemporal loads and
// stores; without a bias the tensor is one flat stream (the last lane adds
// the trailing rows*F % 8 elements), with a bias rows are cut into chunks of
// up to 64 packs; other layouts run over chunks of the output's aligned
// 16-byte words with the inputs realigned in registers (realign.hpp).
#include "dtype.hpp"
#include "launch.hpp"
#include "realign.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;

// tl = t log2(e) = h (kC1 + kC2 h^2), t = 2 sqrt(2/pi) (h + 0.044715 h^3);
// constants rounded to nearest binary32
constexpr float kC1 = 2.3022082f;    // 2 sqrt(2/pi) log2(e)
constexpr float kC2 = 0.10294324f;   // 2 sqrt(2/pi) 0.044715 log2(e)
// below this tl, 2^tl is subnormal (and 2^-tl beyond 2^126)
constexpr float kTinyExp = -126.0f;

__device__ __forceinline__ float exp_arg(float h)
{
    const float h2 = h * h;
    const float m = kC2 * h2;
    const float a = kC1 + m;
    return h * a;
}

// gelu(h) from tl, general form: s = 2^-|tl| <= 1 through exp2f, which keeps
// subnormal results; logistic = 1 / (1 + s) for tl >= 0, s / (1 + s) for
// tl < 0; a logistic factor that underflows to 0 gives a signed zero (also
// for h = -inf, where h * 0 would be NaN).
__device__ __forceinline__ float gelu_general(float h, float tl)
{
    const float s = exp2f(-fabsf(tl));
    const float r = __builtin_amdgcn_rcpf(1.0f + s);
    const float sig = (tl >= 0.0f) ? r : s * r;
    return (sig == 0.0f) ? copysignf(0.0f, h) : h * sig;
}

// gelu(h) from tl when tl >= kTinyExp (or NaN): 2^-tl <= 2^126 cannot
// overflow, so logistic = 1 / (1 + 2^-tl) needs no case split; for large tl
// the hardware exp may flush 2^-tl to 0, which leaves 1 + 2^-tl = 1 as
// before. h is then finite or +inf or NaN, and h * logistic is right for
// all of them.
__device__ __forceinline__ float gelu_common(float h, float tl)
{
    const float s = __builtin_amdgcn_exp2f(-tl);
    const float r = __builtin_amdgcn_rcpf(1.0f + s);
    return h * r;
}

__device__ __forceinline__ float gelu1(float h)
{
    return gelu_general(h, exp_arg(h));
}

template <int DT, bool BIAS>
__device__ __forceinline__ Pack<DT> gelu8(const Pack<DT>& x, const Pack<DT>& b)
{
    float h[8], tl[8], o[8];
    bool tiny = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = x.get(e);
        if constexpr (BIAS)
            h[e] = h[e] + b.get(e);
        tl[e] = exp_arg(h[e]);
        tiny = tiny || (tl[e] < kTinyExp);
    }
    // tl < kTinyExp (h below about -9.3, or -inf) is rare: the whole wave
    // takes the general form only when one of its lanes has such a value
    if (__any(tiny)) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = gelu_general(h[e], tl[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = gelu_common(h[e], tl[e]);
    }
    return Pack<DT>::make(o);
}

// No bias: n8 = floor(n / 8) packs plus n % 8 trailing elements; workgroup
// w takes the chunk of packs 64w .. 64w + h - 1, lane h of the last chunk
// the trailing elements.
template <int DT>
__global__ __launch_bounds__(kBlock) void gelu_tanh_flat_kernel(
    const void* x, void* out, int64_t n8, int tail)
{
    const int64_t c0 = (int64_t)blockIdx.x * kBlock;
    const int t = threadIdx.x;
    const int h = (n8 - c0 < kBlock) ? (int)(n8 - c0) : kBlock;
    if (t < h) {
        using I = Interleaved<DT>;
        const Pack<DT> xv = I::load_stream(x, c0, t, h);
        I::store_stream(gelu8<DT, false>(xv, xv), out, c0, t, h);
    } else if (t == h && c0 + h == n8) {
        for (int e = 0; e < tail; ++e) {
            const int64_t i = 8 * n8 + e;
            store_elem<DT>(out, i, gelu1(load_elem<DT>(x, i)));
        }
    }
}

// Bias row [F], F % 8 == 0: grid x = row * chunks + chunk, a chunk being up
// to 64 packs of a row; the bias packs stay in the caches.
template <int DT>
__global__ __launch_bounds__(kBlock) void gelu_tanh_bias_kernel(
    const void* x, const void* bias, void* out, uint32_t f8, uint32_t chunks)
{
    const uint32_t r = blockIdx.x / chunks;
    const uint32_t chunk = blockIdx.x - r * chunks;
    const uint32_t col0 = chunk * kBlock;
    const int t = threadIdx.x;
    const int h = (f8 - col0 < (uint32_t)kBlock) ? (int)(f8 - col0) : kBlock;
    if (t >= h)
        return;
    const int64_t c0 = (int64_t)r * f8 + col0;
    using I = Interleaved<DT>;
    const Pack<DT> xv = I::load_stream(x, c0, t, h);
    const Pack<DT> bv = I::load(bias, col0, t, h);
    I::store_stream(gelu8<DT, true>(xv, bv), out, c0, t, h);
}

// gelu8 for one 16-byte word of any storage type (8 or 4 elements).
template <int DT, bool BIAS>
__device__ __forceinline__ u32x4 gelu_word(const u32x4& x, const u32x4& b)
{
    using W = Word<DT>;
    float h[W::kN], tl[W::kN], o[W::kN];
    bool tiny = false;
#pragma unroll
    for (int e = 0; e < W::kN; ++e) {
        h[e] = W::get(x, e);
        if constexpr (BIAS)
            h[e] = h[e] + W::get(b, e);
        tl[e] = exp_arg(h[e]);
        tiny = tiny || (tl[e] < kTinyExp);
    }
    if (__any(tiny)) {
#pragma unroll
        for (int e = 0; e < W::kN; ++e)
            o[e] = gelu_general(h[e], tl[e]);
    } else {
#pragma unroll
        for (int e = 0; e < W::kN; ++e)
            o[e] = gelu_common(h[e], tl[e]);
    }
    return W::make(o);
}

// Element path (realign.hpp): chunks of 64 16-byte words of the output's
// aligned window, the input (and bias) read realigned to the output.
// Without a bias the rows * F elements are one run, grid x = chunk.
template <int DT>
__global__ __launch_bounds__(kBlock) void gelu_tanh_generic_flat_kernel(
    const void* x, void* out, int64_t nbytes)
{
    const int mo = start_offset(out);
    const int64_t wbase = 64 * (int64_t)blockIdx.x - line_lead(out);
    if (wbase >= window_words(out, nbytes))
        return;
    const u32x4 xv = load_for_chunk<true>(x, nbytes, mo, wbase);
    store_chunk<true>(out, nbytes, wbase, gelu_word<DT, false>(xv, xv));
}

// With a bias each row is a run, with the bias row beside it; grid x =
// row * chunks per row + chunk.
template <int DT>
__global__ __launch_bounds__(kBlock) void gelu_tanh_generic_bias_kernel(
    const void* x, const void* bias, void* out, int64_t F, uint32_t chunks)
{
    constexpr int es = DT == kF32 ? 4 : 2;
    const uint32_t r = blockIdx.x / chunks;
    const int64_t j = blockIdx.x - r * chunks;
    const int64_t nbytes = F * es;
    const void* px = static_cast<const char*>(x) + (int64_t)r * nbytes;
    void* po = static_cast<char*>(out) + (int64_t)r * nbytes;
    const int mo = start_offset(po);
    const int64_t wbase = 64 * j - line_lead(po);
    if (wbase >= window_words(po, nbytes))
        return;
    const ChunkWords fx = fetch_for_chunk<true>(px, nbytes, mo, wbase);
    const ChunkWords fb = fetch_for_chunk<false>(bias, nbytes, mo, wbase);
    store_chunk<true>(po, nbytes, wbase, gelu_word<DT, true>(chunk_word(fx), chunk_word(fb)));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunks of 64 output words that cover a run of nbytes at any start offset,
// the first chunk starting up to 7 words early (line_lead in realign.hpp).
int64_t element_chunks(int64_t nbytes) { return ceil_div(ceil_div(14 + nbytes, 16) + 7, 64); }

template <int DT>
hipError_t launch_typed(const void* x, const void* bias, void* out, int64_t rows, int64_t F,
                        bool fast, hipStream_t stream)
{
    if (fast && bias == nullptr) {
        const int64_t n = rows * F;
        int64_t n8 = n / 8;
        int tail = (int)(n % 8);
        void* args[] = {&x, &out, &n8, &tail};
        return hipLaunchKernel(reinterpret_cast<const void*>(&gelu_tanh_flat_kernel<DT>),
                               dim3((uint32_t)ceil_div(n8 + (tail ? 1 : 0), kBlock)),
                               dim3(kBlock), args, 0, stream);
    }
    if (fast) {
        uint32_t f8 = (uint32_t)(F / 8);
        uint32_t chunks = (uint32_t)ceil_div(f8, kBlock);
        void* args[] = {&x, &bias, &out, &f8, &chunks};
        return hipLaunchKernel(reinterpret_cast<const void*>(&gelu_tanh_bias_kernel<DT>),
                               dim3((uint32_t)(rows * chunks)), dim3(kBlock), args, 0, stream);
    }
    constexpr int es = DT == kF32 ? 4 : 2;
    if (bias == nullptr) {
        int64_t nbytes = rows * F * es;
        void* args[] = {&x, &out, &nbytes};
        return hipLaunchKernel(reinterpret_cast<const void*>(&gelu_tanh_generic_flat_kernel<DT>),
                               dim3((uint32_t)element_chunks(nbytes)), dim3(kBlock), args, 0,
                               stream);
    }
    uint32_t chunks = (uint32_t)element_chunks(F * es);
    void* args[] = {&x, &bias, &out, &F, &chunks};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gelu_tanh_generic_bias_kernel<DT>),
                           dim3((uint32_t)(rows * chunks)), dim3(kBlock), args, 0, stream);
}

}  // namespace

bool gelu_tanh_grid_fits(int64_t rows, int64_t F, bool has_bias, int es, bool fast)
{
    const int64_t max_wg = (((int64_t)1 << 32) - 1) / kBlock;
    if (fast && !has_bias)
        return ceil_div(rows * F / 8 + 1, kBlock) <= max_wg;
    if (fast)
        return rows * ceil_div(F / 8, kBlock) <= max_wg;
    if (!has_bias)
        return element_chunks(rows * F * es) <= max_wg;
    return rows * element_chunks(F * es) <= max_wg;
}

hipError_t launch_gelu_tanh(const void* x, const void* bias, void* out, int64_t rows,
                            int64_t F, int dtype, bool fast, hipStream_t stream)
{
    switch (dtype) {
    case RGA_DTYPE_F16:
        return launch_typed<kF16>(x, bias, out, rows, F, fast, stream);
    case RGA_DTYPE_F32:
        return launch_typed<kF32>(x, bias, out, rows, F, fast, stream);
    default:
        return launch_typed<kBF16>(x, bias, out, rows, F, fast, stream);
    }
}

}  // namespace rga
