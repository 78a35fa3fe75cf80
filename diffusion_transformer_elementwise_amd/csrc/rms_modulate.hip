// adaLN modulation of a normalized row,
//   out = norm(x, eps) * (1 + scale) + shift,
// over contiguous x [B, L, D] with scale and shift rows [B, 1, D] or per
// token [B, L, D], for two weightless norms:
//   RMSNorm: norm(x) = x / sqrt(mean(x^2) + eps) (prhub summary of sglang PR
//     #34172, "关键源码片段": the expression and RMSNormNoWeight; "风险与影响":
//     the fused kernel's one-ULP allowance);
//   LayerNorm: norm(x) = (x - mean) / sqrt(var + eps), biased variance (the
//     LN+modulate family that summary lists beside it, "实现拆解" items 2 and 4;
//     the pages do not describe it, the DiT adaLN form is taken).
//
// The fixed summation order: the row is cut into groups of 8 consecutive
// elements (the last group may be shorter); one wave64 owns the row; lane j
// accumulates groups j, j+64, ... in increasing group and element order into
// one binary32 partial; the 64 partials are combined with xor-distance lane
// exchanges 1, 2, ..., 32 (every lane ends with the same sum, because
// a + b == b + a bit for bit). RMSNorm sums the squares; LayerNorm first sums
// the values (mean = sum / D), then the squares of x - mean. Then
// r = 1 / sqrt(ss / D + eps) with IEEE division and square root, and each
// element becomes (((x or x - mean) * r) * (1 + scale)) + shift, rounded once
// to the storage type.
//
// Fast path (D % 8 == 0, D <= RGA_RMS_MAX_D, 16-byte aligned pointers): the
// row stays in registers (G packs per lane), read once from HBM and written
// once, with nontemporal loads and stores, one wave per row. With row
// modulation a workgroup holds two waves (two rows of one batch); it first
// stages that batch's scale and shift rows in LDS (from the L2: every
// workgroup reads the same rows), then each wave loads its row, reduces it
// and applies the modulation with scale and shift read from LDS. The launch
// asks for more LDS than the staging needs, to cap the workgroups per CU
// (row_wg_lds in launch.hpp); at [2,32640,4096] this form ran 168-174 us
// against 178-183 us for the former one (two rows per wave, scale and shift
// held in registers, 209 VGPRs), measured on MI355X in the same runs.
// Binary32 rows with row modulation keep the former form (one wave, two
// rows per wave, scale and shift held in registers), which measured faster
// there. Per-token modulation reads its scale and shift rows in the apply
// phase, one row per one-wave workgroup. The LayerNorm's second sum runs over the
// registers, so it costs arithmetic, not memory traffic. A binary32 pack is
// two words; they are moved with contiguous wave-wide accesses and one lane
// exchange (Grouped in dtype.hpp) rather than two adjacent words per lane,
// which left every access instruction half a cache line per lane.
//
// Element path (any D, element-aligned pointers), the same order: 2-byte
// rows of up to 8192 elements are read once and realigned in registers
// (realign.hpp, row_regs.hpp); binary32 rows and longer rows take each sum
// as one pass over the row, then the apply pass, moving spans of elements
// through LDS with 16-byte accesses (span.hpp).
//
// Apart from the row-modulation fast path (two waves sharing their staged
// scale and shift rows) and the LDS-staged element path, one wave per
// workgroup: no sum crosses a wave.
#include "dtype.hpp"
#include "launch.hpp"
#include "row_regs.hpp"
#include "span.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;  // one wave
constexpr int kStage = 1024;  // element path: elements staged in LDS per sum step
constexpr int kApply = 512;   // element path: elements per apply step

enum : int { kNormRms = 0, kNormLn = 1 };

// The 64 lane partials combined by xor-distance exchanges 1, 2, ..., 32;
// every lane ends with the same sum (a + b == b + a bit for bit).
__device__ __forceinline__ float wave_sum(float acc)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        acc = acc + __shfl_xor(acc, m);
    return acc;
}

// The same sums as wave_sum, bit for bit, with fewer round trips: exchanges
// 1 and 2 by DPP quad permutations, 4 and 8 by DPP half-row and row mirrors
// (once lanes 4q..4q+3 hold equal values, the mirror partner of a lane holds
// what its xor-4 partner holds; likewise for 8 once groups of 8 agree), and
// the exchanges at 16 and 32 from the four 16-lane sums read into scalars:
// lane j's (s[j] + s[j^16]) + (s[j^32] + s[j^48]) is (r0 + r1) + (r2 + r3) on
// every lane, as addition commutes. The whole wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_from(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float a)
{
    a = a + dpp_from<0xB1>(a);   // quad_perm [1,0,3,2]: lane ^ 1
    a = a + dpp_from<0x4E>(a);   // quad_perm [2,3,0,1]: lane ^ 2
    a = a + dpp_from<0x141>(a);  // row_half_mirror: the other quad of its 8
    a = a + dpp_from<0x140>(a);  // row_mirror: the other 8 of its 16
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float inv_std(float ss, float d_float, float eps)
{
    const float ms = ss / d_float;
    const float t = ms + eps;
    const float q = sqrtf(t);
    return 1.0f / q;
}

// Partial j of lane (j + s) mod 64 into lane j (ds_bpermute), for rows held
// at phase s: see row_factor.
__device__ __forceinline__ float partials_in_order(float acc, int lane, int phase)
{
    return __int_as_float(
        __builtin_amdgcn_ds_bpermute(((lane + phase) & 63) << 2, __float_as_int(acc)));
}

// The normalisation factor of one row held as G packs per lane at phase s
// (lane t, pack i holds group 64i + t - s; packs outside the row hold zeros,
// which add +0 to a partial that is never -0 and are left out of the
// LayerNorm's sum of squared deviations). Lane t's packs in increasing i are
// the groups of partial j = (t - s) mod 64 in increasing order; with s > 0
// (PHASED) the 64 partials are rotated back to lane order before the
// exchanges, so every sum is the fixed order's bit for bit. Returns r; *mu
// is the LayerNorm mean (0 for RMS).
template <int G, int DT, int NORM, bool DPP, bool PHASED = false>
__device__ __forceinline__ float row_factor(const Pack<DT> (&xv)[G], int lane, int vpr,
                                            float eps, float d_float, float* mu_out,
                                            int phase = 0)
{
    float mu = 0.0f;
    if constexpr (NORM == kNormLn) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < G; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc = acc + xv[i].get(e);
        }
        if constexpr (PHASED)
            acc = partials_in_order(acc, lane, phase);
        mu = (DPP ? wave_sum_dpp(acc) : wave_sum(acc)) / d_float;
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        if (NORM == kNormLn && (lane + 64 * i - phase >= vpr || lane + 64 * i < phase))
            continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = xv[i].get(e);
            if constexpr (NORM == kNormLn)
                a = a - mu;
            const float sa = a * a;
            acc = acc + sa;
        }
    }
    if constexpr (PHASED)
        acc = partials_in_order(acc, lane, phase);
    *mu_out = mu;
    return inv_std(DPP ? wave_sum_dpp(acc) : wave_sum(acc), d_float, eps);
}

template <int DT, int NORM>
__device__ __forceinline__ Pack<DT> modulate_pack(const Pack<DT>& xr, float mu, float rr,
                                                  const Pack<DT>& s_, const Pack<DT>& h_)
{
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float v = xr.get(e);
        if constexpr (NORM == kNormLn)
            v = v - mu;
        const float n = v * rr;
        const float a = 1.0f + s_.get(e);
        const float m = n * a;
        o[e] = m + h_.get(e);
    }
    return Pack<DT>::make(o);
}

// 16-byte LDS words per pack of the row
constexpr int staged_words_per_pack(int var) { return var == kSchedOnePlus ? 3 : 2; }

// The batch's scale and shift rows (vpr <= 64 G words each) into the
// dynamic LDS: every load issued before any LDS write (one round trip to the
// L2, not one per word a thread stages), at most kS words of each per
// thread, indexes clamped and writes guarded. As stored at [0, vpr) and
// [vpr, 2 vpr); with ONE_PLUS, 1 + scale at [0, 2 vpr) (elements 0-3, then
// 4-7 of each pack) and the shift row at [2 vpr, 3 vpr).
template <int G, int DT, bool ONE_PLUS>
__device__ __forceinline__ void stage_scale_shift(u32x4* staged, const u32x4* sc,
                                                  const u32x4* sh, int vpr)
{
    constexpr int kS = (64 * G + kBlock * kRowWaves - 1) / (kBlock * kRowWaves);
    u32x4 sv[kS], hv[kS];
#pragma unroll
    for (int j = 0; j < kS; ++j) {
        const int w = (int)threadIdx.x + kBlock * kRowWaves * j;
        const int wc = w < vpr ? w : vpr - 1;
        sv[j] = load16(sc + wc);
        hv[j] = load16(sh + wc);
    }
#pragma unroll
    for (int j = 0; j < kS; ++j) {
        const int w = (int)threadIdx.x + kBlock * kRowWaves * j;
        if (w < vpr) {
            if constexpr (ONE_PLUS) {
                u32x4 lo, hi;
                one_plus<DT>(sv[j], lo, hi);
                staged[w] = lo;
                staged[vpr + w] = hi;
                staged[2 * vpr + w] = hv[j];
            } else {
                staged[w] = sv[j];
                staged[vpr + w] = hv[j];
            }
        }
    }
}

// Row modulation, kRowWaves waves per workgroup, sched_rows_per_wave(VAR)
// rows per wave: rows kRowWaves * (R * blockIdx.x + j) + wave, j < R, of
// batch blockIdx.y. The batch's scale and shift rows are staged in the
// dynamic LDS (stage_scale_shift) before any row is loaded.
template <int G, int DT, int NORM, bool WHOLE, int VAR = kSchedLibrary>
__device__ __forceinline__ void modulate_staged_row(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    static_assert(DT != kF32, "2-byte rows: a pack is one word, raw order is group order");
    constexpr int R = sched_rows_per_wave(VAR);
    constexpr bool kOnePlus = VAR == kSchedOnePlus;
    extern __shared__ u32x4 staged[];
    const int lane = threadIdx.x & (kBlock - 1);
    const int64_t b = blockIdx.y;
    // the wave index as a per-lane value, as in the fused residual update's
    // staged kernel
    const int64_t r0 = (int64_t)blockIdx.x * kRowWaves * R + (threadIdx.x / kBlock);
    // WHOLE (D = 512 G): every lane's G packs lie in the row, no bounds at
    // all. Otherwise no branch around a load: the index is clamped into the
    // row and zeros are selected past its end (a branch per load made the
    // compiler wait for each load before issuing the next).
    // Other rows are held at the phase of their 128-byte lines (pack
    // 64i + t - s in lane t, pack i; row_factor), as far as the packs have
    // room for it, so that each access instruction covers whole lines.
    auto phase_of = [&](int64_t row) {
        if constexpr (WHOLE) {
            return 0;
        } else {
            const int lead = (int)((reinterpret_cast<uintptr_t>(static_cast<const u32x4*>(x) + row) >> 4) & 7u);
            const int room = 64 * G - vpr;
            return lead < room ? lead : room;
        }
    };
    auto load_row = [&](Pack<DT> (&xv)[G], int64_t row, int phase) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if constexpr (WHOLE) {
                xv[i] = Pack<DT>::load_stream(x, row + 64 * i + lane);
            } else {
                const int p = 64 * i + lane - phase;
                const int pc = p < 0 ? 0 : (p < vpr ? p : vpr - 1);
                xv[i] = Pack<DT>::load_stream(x, row + pc);
                const bool in = p >= 0 && p < vpr;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    xv[i].v[d] = in ? xv[i].v[d] : 0u;
            }
        }
    };
    Pack<DT> xv[G];
    float mu = 0.0f, rr = 0.0f;
    int phase = 0;
    if constexpr (VAR == kSchedLoadsFirst) {
        // a wave past the last row (odd L) loads the last row and stores
        // nothing
        const int64_t row = (b * L + (r0 < L ? r0 : L - 1)) * vpr;
        phase = phase_of(row);
        load_row(xv, row, phase);
    }
    stage_scale_shift<G, DT, kOnePlus>(staged, static_cast<const u32x4*>(scale) + b * vpr,
                                       static_cast<const u32x4*>(shift) + b * vpr, vpr);
    if constexpr (VAR == kSchedLoadsFirst)
        rr = row_factor<G, DT, NORM, true, !WHOLE>(xv, lane, vpr, eps, d_float, &mu, phase);
    __syncthreads();
    if (r0 >= L)
        return;
    if constexpr (VAR != kSchedLoadsFirst) {
        phase = phase_of((b * L + r0) * vpr);
        load_row(xv, (b * L + r0) * vpr, phase);
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t r = r0 + (int64_t)kRowWaves * j;
        const int64_t row = (b * L + r) * vpr;
        const bool more = j + 1 < R && r + kRowWaves < L;
        Pack<DT> xq[VAR == kSchedPrefetch ? G : 1];
        int phase_q = 0;
        if constexpr (VAR == kSchedPrefetch)
            if (more) {
                phase_q = phase_of(row + (int64_t)kRowWaves * vpr);
                load_row(xq, row + (int64_t)kRowWaves * vpr, phase_q);
            }
        if constexpr (VAR != kSchedLoadsFirst)
            rr = row_factor<G, DT, NORM, true, !WHOLE>(xv, lane, vpr, eps, d_float, &mu, phase);
        // element-wise; packs outside the row are not stored
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int p = 64 * i + lane - phase;  // the pack this lane holds
            // its scale and shift words (the index clamped into the row: packs
            // outside it are not stored)
            const int pc = WHOLE ? p : (p < 0 ? 0 : (p < vpr ? p : vpr - 1));
            Pack<DT> o;
            if constexpr (kOnePlus) {
                Pack<DT> h_;
                h_.v = staged[2 * vpr + pc];
                o = modulate_group<DT, NORM == kNormLn>(xv[i], mu, rr, staged[pc],
                                                        staged[vpr + pc], h_);
            } else {
                Pack<DT> s_, h_;
                s_.v = staged[pc];
                h_.v = staged[vpr + pc];
                o = modulate_pack<DT, NORM>(xv[i], mu, rr, s_, h_);
            }
            if constexpr (WHOLE) {
                o.store_stream(out, row + p);
            } else {
                if (p >= 0 && p < vpr)
                    o.store_stream(out, row + p);
            }
        }
        if (j + 1 < R) {
            if (!more)
                return;
            if constexpr (VAR == kSchedPrefetch) {
#pragma unroll
                for (int i = 0; i < G; ++i)
                    xv[i] = xq[i];
                phase = phase_q;
            } else {
                phase = phase_of(row + (int64_t)kRowWaves * vpr);
                load_row(xv, row + (int64_t)kRowWaves * vpr, phase);
            }
        }
    }
}

// Per-token modulation, one wave per workgroup and per row (nothing to share
// between rows): row blockIdx.x of batch blockIdx.y, its scale and shift rows
// read in the apply phase.
template <int G, int DT, int NORM>
__device__ __forceinline__ void modulate_token_row(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    const int lane = threadIdx.x;
    const int64_t row = ((int64_t)blockIdx.y * L + blockIdx.x) * vpr;
    Pack<DT> xv[G];
#pragma unroll
    for (int i = 0; i < G; ++i)
        xv[i] = Grouped<DT>::load_stream(x, row + 64 * i, lane, vpr - 64 * i);
    float mu;
    const float rr = row_factor<G, DT, NORM, false>(xv, lane, vpr, eps, d_float, &mu);
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int h = vpr - 64 * i;
        const Pack<DT> s_ = Grouped<DT>::load_stream_raw(scale, row + 64 * i, lane, h);
        const Pack<DT> h_ = Grouped<DT>::load_stream_raw(shift, row + 64 * i, lane, h);
        Grouped<DT>::store_stream_raw(
            modulate_pack<DT, NORM>(Grouped<DT>::to_raw(xv[i]), mu, rr, s_, h_), out,
            row + 64 * i, lane, h);
    }
}

// Row modulation of binary32 rows: one wave per workgroup, two rows per
// wave (rows 2 blockIdx.x, 2 blockIdx.x + 1 of batch blockIdx.y), the scale
// and shift rows held in registers across both. For these 16-byte-per-pair
// rows this form measured faster than the staged one (377 against 442 us
// at [2,32640,4096], MI355X, same run as the 2-byte gains).
template <int G, int DT, int NORM>
__device__ __forceinline__ void modulate_held_rows(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * 2;
    const int64_t r1 = (r0 + 2 < L) ? r0 + 2 : L;
    Pack<DT> sc[G], sh[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        sc[i] = Grouped<DT>::load_raw(scale, b * vpr + 64 * i, lane, vpr - 64 * i);
        sh[i] = Grouped<DT>::load_raw(shift, b * vpr + 64 * i, lane, vpr - 64 * i);
    }
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t row = (b * L + r) * vpr;
        Pack<DT> xv[G];
#pragma unroll
        for (int i = 0; i < G; ++i)
            xv[i] = Grouped<DT>::load_stream(x, row + 64 * i, lane, vpr - 64 * i);
        float mu;
        const float rr = row_factor<G, DT, NORM, false>(xv, lane, vpr, eps, d_float, &mu);
#pragma unroll
        for (int i = 0; i < G; ++i)
            Grouped<DT>::store_stream_raw(
                modulate_pack<DT, NORM>(Grouped<DT>::to_raw(xv[i]), mu, rr, sc[i], sh[i]), out,
                row + 64 * i, lane, vpr - 64 * i);
    }
}

// Launch shape of the fast path: workgroups of kRowWaves waves with staged
// rows for 2-byte row modulation, else one wave.
template <int DT, int MOD>
constexpr bool staged_rows()
{
    return MOD == kModRow && DT != kF32;
}

template <int G, int DT, int MOD, int NORM, bool WHOLE>
__device__ __forceinline__ void modulate_rows(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    if constexpr (staged_rows<DT, MOD>())
        modulate_staged_row<G, DT, NORM, WHOLE>(x, scale, shift, eps, d_float, out, L, vpr);
    else if constexpr (MOD == kModRow)
        modulate_held_rows<G, DT, NORM>(x, scale, shift, eps, d_float, out, L, vpr);
    else
        modulate_token_row<G, DT, NORM>(x, scale, shift, eps, d_float, out, L, vpr);
}

// Grid: x = pair of rows (row modulation) or row (per token), y = batch.
// WHOLE: D = 512 G (every lane's packs lie in the row; 2-byte row modulation)
template <int G, int DT, int MOD, bool WHOLE = false>
__global__ __launch_bounds__((staged_rows<DT, MOD>() ? kBlock * kRowWaves : kBlock)) void rms_modulate_kernel(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    modulate_rows<G, DT, MOD, kNormRms, WHOLE>(x, scale, shift, eps, d_float, out, L, vpr);
}

// The staged modulation in schedule SCHED (kSched*, launch.hpp), for
// measurement: bf16 rows of kSchedD = 4096 elements (G = 8, whole rows),
// RMSNorm, row modulation.
template <int SCHED>
__global__ __launch_bounds__(kBlock * kRowWaves) void rms_modulate_variant_kernel(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    modulate_staged_row<8, kBF16, kNormRms, true, SCHED>(x, scale, shift, eps, d_float, out, L,
                                                         vpr);
}

template <int G, int DT, int MOD, bool WHOLE = false>
__global__ __launch_bounds__((staged_rows<DT, MOD>() ? kBlock * kRowWaves : kBlock)) void ln_modulate_kernel(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int vpr)
{
    modulate_rows<G, DT, MOD, kNormLn, WHOLE>(x, scale, shift, eps, d_float, out, L, vpr);
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

// Element path, one wave per row. A sum in the fixed order walks the row in
// stages of kStage elements: the wave moves a stage into LDS with 16-byte
// accesses, realigned so that every group of 8 starts a 16-byte word
// (Span::commit_aligned in span.hpp), then lane j reads groups j, j + 64, ...
// of the stage with 16-byte LDS reads and adds them up in order. WHAT: 0 the
// values, 1 their squares, 2 the squares of value - mu.
template <int DT, int WHAT>
__device__ __forceinline__ float staged_sum(const void* x, int64_t row, int64_t D,
                                            float mu, u32x4* raw)
{
    using S = Span<DT, kStage>;
    const int lane = threadIdx.x;
    float acc = 0.0f;
    // the next stage's loads are in flight while this one is summed
    typename S::Words next = S::template fetch<false>(elem_ptr<DT>(x, row),
                                                      D < kStage ? (int)D : kStage);
    for (int64_t s0 = 0; s0 < D; s0 += kStage) {
        const int cnt = (D - s0 < kStage) ? (int)(D - s0) : kStage;
        const int m = S::offset(elem_ptr<DT>(x, row + s0));
        S::commit_aligned(next, m, cnt, raw);
        __syncthreads();
        const int64_t s1 = s0 + kStage;
        if (s1 < D)
            next = S::template fetch<false>(elem_ptr<DT>(x, row + s1),
                                            (D - s1 < kStage) ? (int)(D - s1) : kStage);
#pragma unroll
        for (int k = 0; k < kStage / 512; ++k) {
            const int g = lane + kBlock * k;
            if (8 * g >= cnt)
                continue;
            const Pack<DT> p = S::group(raw, g);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (8 * g + e < cnt) {
                    float a = p.get(e);
                    if constexpr (WHAT == 0) {
                        acc = acc + a;
                    } else {
                        if constexpr (WHAT == 2)
                            a = a - mu;
                        const float sa = a * a;
                        acc = acc + sa;
                    }
                }
            }
        }
        __syncthreads();
    }
    return wave_sum(acc);
}

// LDS of the two-pass kernels, taken from the launch's dynamic LDS: the
// staged-sum span, then the apply pass's x, scale, shift and out spans. (A
// static buffer would also be placed, unused, in every kernel of this file
// that uses dynamic LDS, 6-12 KB that limited the rows the LDS-staged
// kernels keep per CU.)
template <int DT>
constexpr int64_t generic_lds_bytes()
{
    return 16 * ((int64_t)Span<DT, kStage>::kWords + 4 * (int64_t)Span<DT, kApply>::kWords);
}

// The apply pass re-reads the row (mostly from L2) in spans of kApply
// elements, with scale and shift spans beside it, and writes out spans; the
// next span's loads are in flight while this one is computed and stored.
template <int DT, int MOD, int NORM>
__device__ __forceinline__ void modulate_row_generic(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int64_t D, u32x4* stage)
{
    using A = Span<DT, kApply>;
    u32x4* rx = stage + Span<DT, kStage>::kWords;
    u32x4* rs = rx + A::kWords;
    u32x4* rh = rs + A::kWords;
    u32x4* ro = rh + A::kWords;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t mrow = (MOD == kModToken) ? row : b * D;

    float mu = 0.0f;
    if constexpr (NORM == kNormLn)
        mu = staged_sum<DT, 0>(x, row, D, 0.0f, stage) / d_float;
    const float ss = staged_sum<DT, NORM == kNormLn ? 2 : 1>(x, row, D, mu, stage);
    const float rr = inv_std(ss, d_float, eps);

    constexpr bool kTok = MOD == kModToken;
    int cnt = D < kApply ? (int)D : kApply;
    typename A::Words nx = A::template fetch<true>(elem_ptr<DT>(x, row), cnt);
    typename A::Words ns = A::template fetch<kTok>(elem_ptr<DT>(scale, mrow), cnt);
    typename A::Words nh = A::template fetch<kTok>(elem_ptr<DT>(shift, mrow), cnt);
    for (int64_t s0 = 0; s0 < D; s0 += kApply) {
        cnt = (D - s0 < kApply) ? (int)(D - s0) : kApply;
        const int mx = A::offset(elem_ptr<DT>(x, row + s0));
        const int ms = A::offset(elem_ptr<DT>(scale, mrow + s0));
        const int mh = A::offset(elem_ptr<DT>(shift, mrow + s0));
        void* po = elem_ptr<DT>(out, row + s0);
        const int mo = A::offset(po);
        A::commit(nx, rx);
        A::commit(ns, rs);
        A::commit(nh, rh);
        __syncthreads();
        const int64_t s1 = s0 + kApply;
        if (s1 < D) {
            const int c1 = (D - s1 < kApply) ? (int)(D - s1) : kApply;
            nx = A::template fetch<true>(elem_ptr<DT>(x, row + s1), c1);
            ns = A::template fetch<kTok>(elem_ptr<DT>(scale, mrow + s1), c1);
            nh = A::template fetch<kTok>(elem_ptr<DT>(shift, mrow + s1), c1);
        }
        for (int i = threadIdx.x; i < cnt; i += kBlock) {
            float v = A::get(rx, mx, i);
            if constexpr (NORM == kNormLn)
                v = v - mu;
            const float n = v * rr;
            const float a = 1.0f + A::get(rs, ms, i);
            const float m = n * a;
            A::put(ro, mo, i, m + A::get(rh, mh, i));
        }
        __syncthreads();
        A::template store<true>(po, cnt, ro);
    }
}

// Grid: x = row l, y = batch b.
template <int DT, int MOD>
__global__ __launch_bounds__(kBlock) void rms_modulate_generic_kernel(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int64_t D)
{
    extern __shared__ u32x4 rowbuf[];  // generic_lds_bytes<DT>()
    modulate_row_generic<DT, MOD, kNormRms>(x, scale, shift, eps, d_float, out, L, D, rowbuf);
}

template <int DT, int MOD>
__global__ __launch_bounds__(kBlock) void ln_modulate_generic_kernel(
    const void* x, const void* scale, const void* shift, float eps,
    float d_float, void* out, int64_t L, int64_t D)
{
    extern __shared__ u32x4 rowbuf[];  // generic_lds_bytes<DT>()
    modulate_row_generic<DT, MOD, kNormLn>(x, scale, shift, eps, d_float, out, L, D, rowbuf);
}

// Element path for rows that fit in LDS but not in registers (binary32
// rows; 2-byte rows over 8192 elements): one workgroup of NW waves per row
// (lds_row_waves: about one per 4 KB of row), the row read from HBM once.
// The waves stage it into a dynamic LDS buffer (stage i by wave i mod NW, the
// wave's next stage in flight
// while one is committed), realigned so that element i sits at byte i * es
// (Span::commit_aligned); wave 0 takes the sums from LDS in the fixed order
// (lane j: groups j, j + 64, ...); all waves then apply over chunks of the
// output's aligned 16-byte words (realign.hpp), x taken from LDS at the
// output's byte positions (two aligned LDS words and a cut), scale and shift
// read realigned to them.
constexpr int kRowStage = 1024;  // elements staged per step
// dynamic LDS per workgroup, less room for the few static bytes
constexpr int64_t kMaxRowLds = 65536 - 256;

// LDS bytes the staged row needs: its aligned words plus two words that a
// cut at the row's end may touch (their bytes are never used).
int64_t row_lds_bytes(int64_t D, int es) { return ((D * es + 15) / 16 + 2) * 16; }

// sum over the staged row of x (what 0), x^2 (1) or (x - mu)^2 (2), by one wave
template <int DT>
__device__ __forceinline__ float lds_row_sum(const u32x4* rowbuf, int n, float mu, int what)
{
    const int lane = threadIdx.x & 63;
    const int groups = (n + 7) >> 3;
    float acc = 0.0f;
    // batches of U groups wholly inside the row: the U reads are issued
    // before any is added (one LDS round trip per batch rather than per
    // group); the additions keep the fixed order. The rest, masked, below.
    constexpr int U = DT == kF32 ? 4 : 8;
    const int n_whole = n >> 3;
    int g = lane;
    for (; g + kBlock * (U - 1) < n_whole; g += kBlock * U) {
        Pack<DT> p[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            p[u] = Span<DT, kRowStage>::group(rowbuf, g + kBlock * u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = p[u].get(e);
                if (what == 0) {
                    acc = acc + a;
                } else {
                    if (what == 2)
                        a = a - mu;
                    const float sa = a * a;
                    acc = acc + sa;
                }
            }
        }
    }
    for (; g < groups; g += kBlock) {
        const Pack<DT> p = Span<DT, kRowStage>::group(rowbuf, g);
        const bool whole = 8 * g + 8 <= n;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (whole || 8 * g + e < n) {
                float a = p.get(e);
                if (what == 0) {
                    acc = acc + a;
                } else {
                    if (what == 2)
                        a = a - mu;
                    const float sa = a * a;
                    acc = acc + sa;
                }
            }
        }
    }
    return wave_sum(acc);
}

template <int DT, int MOD, int NORM, int NW>
__global__ __launch_bounds__(kBlock * NW) void modulate_lds_kernel(
    const void* x, const void* scale, const void* shift, float eps, float d_float,
    void* out, int64_t L, int64_t D)
{
    extern __shared__ u32x4 rowbuf[];
    __shared__ float factors[2];
    using S = Span<DT, kRowStage>;
    constexpr int es = DT == kF32 ? 4 : 2;
    constexpr bool kTok = MOD == kModToken;
    constexpr int kStride = kRowStage * NW;
    // the wave index as a per-lane value (wave_in_group() would make it
    // scalar): the compiler then schedules this kernel as its timings
    // were taken with
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t mrow = kTok ? row : b * D;
    const int n = (int)D;

    const int first = wave * kRowStage;
    if (first < n) {
        typename S::Words next = S::template fetch<true>(
            elem_ptr<DT>(x, row + first), (n - first < kRowStage) ? n - first : kRowStage);
        for (int s0 = first; s0 < n; s0 += kStride) {
            const int cnt = (n - s0 < kRowStage) ? n - s0 : kRowStage;
            const int m = S::offset(elem_ptr<DT>(x, row + s0));
            const typename S::Words cur = next;
            const int s1 = s0 + kStride;
            if (s1 < n)
                next = S::template fetch<true>(elem_ptr<DT>(x, row + s1),
                                               (n - s1 < kRowStage) ? n - s1 : kRowStage);
            S::commit_aligned(cur, m, cnt, rowbuf + s0 * es / 16);
        }
    }
    __syncthreads();
    if (wave == 0) {
        float mu = 0.0f;
        if constexpr (NORM == kNormLn)
            mu = lds_row_sum<DT>(rowbuf, n, 0.0f, 0) / d_float;
        const float rr =
            inv_std(lds_row_sum<DT>(rowbuf, n, mu, NORM == kNormLn ? 2 : 1), d_float, eps);
        if (lane == 0) {
            factors[0] = mu;
            factors[1] = rr;
        }
    }
    __syncthreads();
    const float mu = factors[0];
    const float rr = factors[1];

    void* po = elem_ptr<DT>(out, row);
    const int mo = start_offset(po);
    const int64_t nbytes = D * es;
    const int64_t words = window_words(po, nbytes);
    const int sh = (16 - mo) & 15;
    // rowbuf holds (nbytes + 15) / 16 + 2 words: q and q + 1 stay inside for
    // q <= qmax; lanes past the row's last word are clamped (not stored)
    const int qmax = (int)((nbytes + 15) / 16);
    const int lead = line_lead(po);
    // one branch on the row's LDS cut (uniform for the row) around the whole
    // apply loop, so the x words are cut with fixed dword picks
    dispatch_offset(sh, [&](auto off) {
        constexpr int O = decltype(off)::value;
        for (int64_t c = wave; 64 * c - lead < words; c += NW) {
            const int64_t wbase = 64 * c - lead;  // chunks of whole 128-byte output lines
            // output word w holds row bytes [16w - mo, 16w - mo + 16); words
            // before the row (w < 0) read clamped words and are not stored
            int q = (int)((16 * (wbase + lane) - mo) >> 4);
            q = q < -1 ? -1 : (q < qmax ? q : qmax);
            u32x4 xw = rowbuf[q < 0 ? 0 : q];
            if constexpr (O != 0)
                xw = window_o<O>(xw, rowbuf[q + 1], sh);
            const ChunkWords fsw =
                fetch_for_chunk<kTok>(elem_ptr<DT>(scale, mrow), nbytes, mo, wbase);
            const ChunkWords fhw =
                fetch_for_chunk<kTok>(elem_ptr<DT>(shift, mrow), nbytes, mo, wbase);
            const u32x4 sw = chunk_word(fsw);
            const u32x4 hw = chunk_word(fhw);
            using W = Word<DT>;
            float o[W::kN];
#pragma unroll
            for (int e = 0; e < W::kN; ++e) {
                float v = W::get(xw, e);
                if constexpr (NORM == kNormLn)
                    v = v - mu;
                const float nv = v * rr;
                const float a = 1.0f + W::get(sw, e);
                const float mm = nv * a;
                o[e] = mm + W::get(hw, e);
            }
            store_chunk<true>(po, nbytes, wbase, W::make(o));
        }
    });
}

// Element path for 2-byte types with D <= 512 * K: one wave per row, the
// row read once and realigned in registers (realign.hpp) so lane t, slot k
// holds group t + 64k, which is the fixed order's assignment (row_regs.hpp).
// Scale and shift are realigned the same way and the result is realigned
// to the output's offset.
// Row modulation of 2-byte rows held in registers: kRowWaves waves per
// workgroup, one row each (rows kRowWaves * blockIdx.x + wave of batch
// blockIdx.y). Before any row is loaded, wave 0 stages the batch's 1 + scale
// in binary32 and wave 1 its shift row in the dynamic LDS, as groups in
// planes of P = ceil(D / 8) words (row_regs.hpp): 1 + scale elements 0-3 at
// [0, P), 4-7 at [P, 2P), shift at [2P, 3P).
template <int K, int DT, int NORM>
__global__ __launch_bounds__(kBlock * kRowWaves) void modulate_regs_staged_kernel(
    const void* x, const void* scale, const void* shift, float eps, float d_float,
    void* out, int64_t L, int64_t D)
{
    extern __shared__ u32x4 staged[];
    const int wave = wave_in_group();
    const int64_t b = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * kRowWaves + wave;
    const int n = (int)D;
    const int planes = (n + 7) >> 3;
    constexpr int kNorm = NORM == kNormLn ? regs::kLn : regs::kRms;
    static_assert(kRowWaves == 2, "one staged row per wave");
    u32x4* h_st = staged + 2 * planes;
    if (wave == 0)
        regs::stage_one_plus<K, DT>(staged, staged + planes, elem_ptr<DT>(scale, b * D), n);
    else
        regs::stage_row<K>(h_st, elem_ptr<DT>(shift, b * D), n);
    __syncthreads();
    if (r >= L)
        return;
    const int64_t row = (b * L + r) * D;
    const void* px = elem_ptr<DT>(x, row);
    // the row at the phase of its 128-byte lines (each access instruction
    // covering whole lines), as far as the slots have room for it
    const int room = 64 * K - planes;
    const int phase = line_lead(px) < room ? line_lead(px) : room;
    u32x4 xv[K];
    load_groups<K, true>(px, n, xv, phase);
    float mu, rr;
    regs::row_factors<K, DT, kNorm>(xv, n, d_float, eps, &mu, &rr, phase);
    regs::apply_store_staged<K, DT, kNorm, true>(xv, staged, staged + planes, h_st, n, mu, rr,
                                                 elem_ptr<DT>(out, row), phase);
}

template <int K, int DT, int MOD, int NORM>
__global__ __launch_bounds__(kBlock) void modulate_regs_kernel(
    const void* x, const void* scale, const void* shift, float eps, float d_float,
    void* out, int64_t L, int64_t D)
{
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t mrow = (MOD == kModToken) ? row : b * D;
    const int n = (int)D;
    constexpr int kNorm = NORM == kNormLn ? regs::kLn : regs::kRms;

    u32x4 xv[K];
    load_groups<K, true>(elem_ptr<DT>(x, row), n, xv);
    float mu, rr;
    regs::row_factors<K, DT, kNorm>(xv, n, d_float, eps, &mu, &rr);
    regs::apply_store<K, DT, MOD == kModToken, kNorm>(xv, elem_ptr<DT>(scale, mrow),
                                                      elem_ptr<DT>(shift, mrow), n, mu, rr,
                                                      elem_ptr<DT>(out, row));
}

typedef void (*rms_kernel_t)(const void*, const void*, const void*, float,
                             float, void*, int64_t, int);

// Packs per lane are taken from a ladder (the smallest entry >= ceil(D/512)).
constexpr int kLadder[] = {1, 2, 4, 6, 8, 9, 12, 16};
static_assert(RGA_RMS_MAX_D / 512 == 16, "ladder tops out at RGA_RMS_MAX_D");

template <int NORM, int G, int DT, int MOD, bool WHOLE>
constexpr rms_kernel_t fast_kernel()
{
    return NORM == kNormLn ? &ln_modulate_kernel<G, DT, MOD, WHOLE>
                           : &rms_modulate_kernel<G, DT, MOD, WHOLE>;
}

// the kernel for rows of `groups` packs per lane; `whole`: the row is
// exactly 64 * groups packs (D = 512 G), every lane's packs in the row
template <int NORM, int DT, int MOD>
rms_kernel_t pick(int groups, bool whole)
{
    constexpr bool kW = staged_rows<DT, MOD>();  // only the staged rows have a WHOLE form
    rms_kernel_t t[] = {fast_kernel<NORM, 1, DT, MOD, false>(), fast_kernel<NORM, 2, DT, MOD, false>(),
                        fast_kernel<NORM, 4, DT, MOD, false>(), fast_kernel<NORM, 6, DT, MOD, false>(),
                        fast_kernel<NORM, 8, DT, MOD, false>(), fast_kernel<NORM, 9, DT, MOD, false>(),
                        fast_kernel<NORM, 12, DT, MOD, false>(), fast_kernel<NORM, 16, DT, MOD, false>()};
    rms_kernel_t w[] = {fast_kernel<NORM, 1, DT, MOD, kW>(), fast_kernel<NORM, 2, DT, MOD, kW>(),
                        fast_kernel<NORM, 4, DT, MOD, kW>(), fast_kernel<NORM, 6, DT, MOD, kW>(),
                        fast_kernel<NORM, 8, DT, MOD, kW>(), fast_kernel<NORM, 9, DT, MOD, kW>(),
                        fast_kernel<NORM, 12, DT, MOD, kW>(), fast_kernel<NORM, 16, DT, MOD, kW>()};
    static_assert(sizeof(kLadder) / sizeof(kLadder[0]) == 8, "one kernel per ladder entry");
    for (int i = 0; i < 8; ++i)
        if (groups <= kLadder[i])
            return (whole && groups == kLadder[i]) ? w[i] : t[i];
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Dynamic LDS of a row-modulation fast-path workgroup (row_wg_lds in
// launch.hpp): the staged scale and shift rows; a row of at most
// RGA_RMS_MAX_D binary32 elements stages 64 KB, one workgroup's limit.
int64_t staged_row_lds(int64_t row_bytes, int wg_per_cu)
{
    return row_wg_lds(row_bytes, 2 * row_bytes, kModRowBudget, wg_per_cu);
}

// Element-path slots per lane for 2-byte rows held in registers: the
// smallest entry >= ceil(ceil(D / 8) / 64); rows past the last entry (and
// binary32 rows) take the LDS-staged kernels.
using regs::kRegsLadder;

template <int NORM, int K, int DT, int MOD>
const void* regs_kernel()
{
    return reinterpret_cast<const void*>(&modulate_regs_kernel<K, DT, MOD, NORM>);
}

template <int NORM, int K, int DT>
const void* regs_staged_kernel()
{
    return reinterpret_cast<const void*>(&modulate_regs_staged_kernel<K, DT, NORM>);
}

// the register-row kernel of a row of `slots` slots: K from the ladder
int pick_regs_slots(int64_t slots)
{
    for (int i = 0; i < 8; ++i)
        if (slots <= kRegsLadder[i])
            return kRegsLadder[i];
    return 0;
}

template <int NORM, int DT>
const void* pick_regs_staged(int K)
{
    switch (K) {
    case 1: return regs_staged_kernel<NORM, 1, DT>();
    case 2: return regs_staged_kernel<NORM, 2, DT>();
    case 4: return regs_staged_kernel<NORM, 4, DT>();
    case 6: return regs_staged_kernel<NORM, 6, DT>();
    case 8: return regs_staged_kernel<NORM, 8, DT>();
    case 9: return regs_staged_kernel<NORM, 9, DT>();
    case 12: return regs_staged_kernel<NORM, 12, DT>();
    default: return regs_staged_kernel<NORM, 16, DT>();
    }
}

template <int NORM, int DT, int MOD>
const void* pick_regs(int64_t slots)
{
    const void* t[] = {regs_kernel<NORM, 1, DT, MOD>(), regs_kernel<NORM, 2, DT, MOD>(),
                       regs_kernel<NORM, 4, DT, MOD>(), regs_kernel<NORM, 6, DT, MOD>(),
                       regs_kernel<NORM, 8, DT, MOD>(), regs_kernel<NORM, 9, DT, MOD>(),
                       regs_kernel<NORM, 12, DT, MOD>(), regs_kernel<NORM, 16, DT, MOD>()};
    for (int i = 0; i < 8; ++i)
        if (slots <= kRegsLadder[i])
            return t[i];
    return nullptr;
}

template <int DT, int MOD, int NORM>
const void* lds_kernel(int w)
{
    switch (w) {
    case 2: return reinterpret_cast<const void*>(&modulate_lds_kernel<DT, MOD, NORM, 2>);
    case 4: return reinterpret_cast<const void*>(&modulate_lds_kernel<DT, MOD, NORM, 4>);
    default: return reinterpret_cast<const void*>(&modulate_lds_kernel<DT, MOD, NORM, 8>);
    }
}

template <int NORM, int DT, int MOD>
hipError_t launch_typed(const void* x, const void* scale, const void* shift,
                        float eps, void* out, int64_t B, int64_t L, int64_t D,
                        bool fast, hipStream_t stream, int wg_per_cu)
{
    float d_float = (float)D;
    if (!fast) {
        void* args[] = {&x, &scale, &shift, &eps, &d_float, &out, &L, &D};
        if constexpr (DT != kF32) {
            const int64_t slots = ceil_div(ceil_div(D, 8), 64);
            const int K = pick_regs_slots(slots);
            if (K > 0 && MOD == kModRow) {
                // two rows per workgroup with 1 + scale and the shift row
                // staged once (three planes of ceil(D / 8) words),
                // occupancy capped
                return hipLaunchKernel(pick_regs_staged<NORM, DT>(K),
                                       dim3((uint32_t)ceil_div(L, kRowWaves), (uint32_t)B),
                                       dim3(kBlock * kRowWaves), args,
                                       (size_t)row_wg_lds(2 * D, 3 * 16 * ceil_div(D, 8),
                                                          kModElemRowBudget, wg_per_cu),
                                       stream);
            }
            const void* rk = pick_regs<NORM, DT, MOD>(slots);
            if (rk != nullptr)
                return hipLaunchKernel(rk, dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args, 0,
                                       stream);
        }
        const int64_t lds = row_lds_bytes(D, DT == kF32 ? 4 : 2);
        if (lds <= kMaxRowLds) {
            const int w = lds_row_waves(D * (DT == kF32 ? 4 : 2));
            return hipLaunchKernel(lds_kernel<DT, MOD, NORM>(w), dim3((uint32_t)L, (uint32_t)B),
                                   dim3(kBlock * w), args, (size_t)lds, stream);
        }
        const void* k = NORM == kNormLn
                            ? reinterpret_cast<const void*>(&ln_modulate_generic_kernel<DT, MOD>)
                            : reinterpret_cast<const void*>(&rms_modulate_generic_kernel<DT, MOD>);
        return hipLaunchKernel(k, dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args,
                               (size_t)generic_lds_bytes<DT>(), stream);
    }
    int vpr = (int)(D / 8);
    rms_kernel_t k = pick<NORM, DT, MOD>((int)ceil_div(vpr, 64), vpr % 64 == 0);
    if (k == nullptr)
        return hipErrorInvalidValue;
    void* args[] = {&x, &scale, &shift, &eps, &d_float, &out, &L, &vpr};
    if constexpr (MOD == kModToken)
        return hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((uint32_t)L, (uint32_t)B),
                               dim3(kBlock), args, 0, stream);
    if constexpr (!staged_rows<DT, MOD>())
        return hipLaunchKernel(reinterpret_cast<const void*>(k),
                               dim3((uint32_t)ceil_div(L, 2), (uint32_t)B), dim3(kBlock), args, 0,
                               stream);
    return hipLaunchKernel(reinterpret_cast<const void*>(k),
                           dim3((uint32_t)ceil_div(L, kRowWaves), (uint32_t)B),
                           dim3(kBlock * kRowWaves), args,
                           (size_t)staged_row_lds(D * (DT == kF32 ? 4 : 2), wg_per_cu), stream);
}

template <int NORM, int DT>
hipError_t launch_mod(const void* x, const void* scale, const void* shift,
                      float eps, void* out, int64_t B, int64_t L, int64_t D,
                      int mod_mode, bool fast, hipStream_t stream, int wg_per_cu)
{
    return mod_mode == RGA_MOD_TOKEN
               ? launch_typed<NORM, DT, kModToken>(x, scale, shift, eps, out, B, L, D, fast,
                                                   stream, wg_per_cu)
               : launch_typed<NORM, DT, kModRow>(x, scale, shift, eps, out, B, L, D, fast,
                                                 stream, wg_per_cu);
}

template <int NORM>
hipError_t launch_norm(const void* x, const void* scale, const void* shift, float eps,
                       void* out, int64_t B, int64_t L, int64_t D, int mod_mode,
                       int dtype, bool fast, hipStream_t stream, int wg_per_cu)
{
    switch (dtype) {
    case RGA_DTYPE_F16:
        return launch_mod<NORM, kF16>(x, scale, shift, eps, out, B, L, D, mod_mode, fast,
                                      stream, wg_per_cu);
    case RGA_DTYPE_F32:
        return launch_mod<NORM, kF32>(x, scale, shift, eps, out, B, L, D, mod_mode, fast,
                                      stream, wg_per_cu);
    default:
        return launch_mod<NORM, kBF16>(x, scale, shift, eps, out, B, L, D, mod_mode, fast,
                                       stream, wg_per_cu);
    }
}

}  // namespace

// Grid x holds at most L workgroups (one or two rows each on the fast path,
// one row on the element paths); its size in work-items, L times the
// workgroup size, must fit 32 bits: 64 lanes, or 64 lds_row_waves(D * es)
// for the LDS-staged rows (binary32 rows and 2-byte rows over the register
// limit that fit the LDS buffer).
bool rms_modulate_grid_fits(int64_t B, int64_t L, int64_t D, int es, bool fast)
{
    if (B > 65535)
        return false;
    const bool regs = es == 2 && ceil_div(ceil_div(D, 8), 64) <= kRegsLadder[7];
    const bool lds = !fast && !regs && row_lds_bytes(D, es) <= kMaxRowLds;
    const int64_t wg = lds ? kBlock * lds_row_waves(D * es) : kBlock;
    const int64_t limit = ((int64_t)1 << 32) - 1;  // work-items of one launch
    // the staged row kernels: ceil(L / 2) workgroups of two waves (an odd
    // L at the one-wave bound would ask for 2^32 work-items)
    if (!lds && ceil_div(L, kRowWaves) > limit / (kBlock * kRowWaves))
        return false;
    return L <= limit / wg;
}

hipError_t launch_rms_modulate(const void* x, const void* scale,
                               const void* shift, float eps, void* out,
                               int64_t B, int64_t L, int64_t D, int mod_mode,
                               int dtype, bool fast, hipStream_t stream, int wg_per_cu)
{
    return launch_norm<kNormRms>(x, scale, shift, eps, out, B, L, D, mod_mode, dtype, fast,
                                 stream, wg_per_cu);
}

hipError_t launch_modulate_variant(const void* x, const void* scale, const void* shift,
                                   float eps, void* out, int64_t B, int64_t L, int sched,
                                   hipStream_t stream)
{
    static_assert(kSchedD == 512 * 8, "whole rows of 8 packs per lane");
    const void* k = nullptr;
    switch (sched) {
    case kSchedLibrary: k = reinterpret_cast<const void*>(&rms_modulate_variant_kernel<kSchedLibrary>); break;
    case kSchedLoadsFirst: k = reinterpret_cast<const void*>(&rms_modulate_variant_kernel<kSchedLoadsFirst>); break;
    case kSchedOnePlus: k = reinterpret_cast<const void*>(&rms_modulate_variant_kernel<kSchedOnePlus>); break;
    case kSchedTwoRows: k = reinterpret_cast<const void*>(&rms_modulate_variant_kernel<kSchedTwoRows>); break;
    case kSchedPrefetch: k = reinterpret_cast<const void*>(&rms_modulate_variant_kernel<kSchedPrefetch>); break;
    default: return hipErrorInvalidValue;
    }
    float d_float = (float)kSchedD;
    int vpr = (int)(kSchedD / 8);
    void* args[] = {&x, &scale, &shift, &eps, &d_float, &out, &L, &vpr};
    const int64_t row_bytes = kSchedD * 2;
    return hipLaunchKernel(
        k, dim3((uint32_t)ceil_div(L, kRowWaves * sched_rows_per_wave(sched)), (uint32_t)B),
        dim3(kBlock * kRowWaves), args,
        (size_t)row_wg_lds(row_bytes, staged_words_per_pack(sched) * row_bytes, kModRowBudget, 0),
        stream);
}

hipError_t launch_ln_modulate(const void* x, const void* scale,
                              const void* shift, float eps, void* out,
                              int64_t B, int64_t L, int64_t D, int mod_mode,
                              int dtype, bool fast, hipStream_t stream)
{
    return launch_norm<kNormLn>(x, scale, shift, eps, out, B, L, D, mod_mode, dtype, fast,
                                stream, 0);
}

}  // namespace rga
