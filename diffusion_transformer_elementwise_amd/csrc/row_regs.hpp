// The modulation of one row of a 2-byte type held in registers as groups
// (realign.hpp: lane t, slot k holds elements 8(t + 64k) .. 8(t + 64k) + 7,
// the last group possibly past the row end), shared by the element paths of
// the modulation and of the fused residual update.
//
// Sums follow the library's fixed order: lane j accumulates groups j,
// j + 64, ... in increasing group and element order, then xor-distance lane
// exchanges 1, 2, ..., 32 combine the 64 partials; elements past the row end
// are skipped. Slots that every row of the instance fills (whole_slots) are
// summed without per-element masks.
//
// Called by the whole wave.
#pragma once

#include "realign.hpp"

namespace rga {
namespace regs {

enum : int { kRms = 0, kLn = 1 };

// The slot ladder of the register-resident rows: a row of n 2-byte elements
// runs with the smallest K here of at least ceil(ceil(n / 8) / 64) slots;
// longer rows are staged in LDS.
constexpr int kRegsLadder[] = {1, 2, 4, 6, 8, 9, 12, 16};

// Slots that every row run with K slots fills with whole groups: such a row
// has more than 512 times the ladder's previous entry elements (it would
// run with that entry otherwise), so its slots below that entry are whole.
template <int K>
constexpr int whole_slots()
{
    int prev = 0;
    for (const int k : kRegsLadder) {
        if (k == K)
            return prev;
        prev = k;
    }
    return 0;
}

__device__ __forceinline__ float wave_sum(float acc)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        acc = acc + __shfl_xor(acc, m);
    return acc;
}

// sum over the row of x (WHAT 0), x^2 (1) or (x - mu)^2 (2), the row held at
// phase s (lane t, slot k: group g = 64k + t - s; load_groups). Lane t
// accumulates its slots in increasing k, which are groups j, j + 64, ... of
// partial j = (t - s) mod 64 in increasing order (lanes t < s start at slot
// 1); one rotation of the 64 partials by s lanes puts partial j in lane j
// before the xor-distance exchanges, so the sum is that of the fixed order
// bit for bit at any phase. Elements outside the row (groups below 0 or
// past n) add +0 instead of their term, which leaves the partial as it
// was (a partial that starts at +0 never becomes -0), and the selection
// is branch-free (a branch per element cost more than the terms). Slots
// 1 .. whole_slots<K>() - 1 are whole at any phase (a row run with K slots
// has more than 512 times the ladder's previous entry elements) and take
// no selection, known at compile time; the others test wholeness once for
// the wave.
template <int K, int DT, int WHAT>
__device__ __forceinline__ float row_sum(const u32x4 (&xv)[K], int n, float mu, int phase = 0)
{
    constexpr int kWhole = whole_slots<K>();
    const int lane = threadIdx.x & 63;
    auto term = [&](const Pack<DT>& p, int e) {
        float a = p.get(e);
        if constexpr (WHAT == 0)
            return a;
        if constexpr (WHAT == 2)
            a = a - mu;
        return a * a;
    };
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        Pack<DT> p;
        p.v = xv[k];
        const int g = lane + 64 * k - phase;
        const bool whole = (k >= 1 && k < kWhole) ||
                           (64 * k >= phase && 512 * (k + 1) - 8 * phase <= n);
        if (whole) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc = acc + term(p, e);
        } else {
            // elements of this group inside the row (none below group 0)
            const int rem = g >= 0 ? n - 8 * g : 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = term(p, e);
                acc = acc + (e < rem ? t : 0.0f);
            }
        }
    }
    // partial j from lane (j + s) mod 64 (ds_bpermute; the identity at s = 0)
    acc = __int_as_float(
        __builtin_amdgcn_ds_bpermute(((lane + phase) & 63) << 2, __float_as_int(acc)));
    return wave_sum(acc);
}

// mean (LayerNorm; 0 for RMSNorm) and 1 / sqrt(mean square + eps)
template <int K, int DT, int NORM>
__device__ __forceinline__ void row_factors(const u32x4 (&xv)[K], int n, float d_float, float eps,
                                            float* mu, float* rr, int phase = 0)
{
    float m = 0.0f;
    if constexpr (NORM == kLn)
        m = row_sum<K, DT, 0>(xv, n, 0.0f, phase) / d_float;
    const float ss = row_sum<K, DT, NORM == kLn ? 2 : 1>(xv, n, m, phase);
    const float ms = ss / d_float;
    const float t = ms + eps;
    const float q = sqrtf(t);
    *mu = m;
    *rr = 1.0f / q;
}

// out = ((x - mu) * rr) * (1 + scale) + shift over the row, written at out
// realigned to its offset; scale and shift rows are read realigned to
// groups (streamed when per token). xv is overwritten.
template <int K, int DT, bool STREAM_MOD, int NORM>
__device__ __forceinline__ void apply_store(u32x4 (&xv)[K], const void* scale, const void* shift,
                                            int n, float mu, float rr, void* out)
{
    // keep the row packed across the reduction: the apply widens it again
    // (a few shifts) instead of holding 8 widened values per group
#pragma unroll
    for (int k = 0; k < K; ++k)
        __asm__ volatile("" : "+v"(xv[k]));
    // scale and shift all at once, or at 16 slots in batches of 4 (with the
    // run-time cut in realign_in, 284 -> 236 registers: 2 waves per SIMD);
    // each batch's loads of both rows issued before either is realigned
    constexpr int KB = K >= kRealignRuntimeSlots ? 4 : K;
    static_assert(K % KB == 0, "whole batches");
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += KB) {
        u32x4 sv[KB], hv[KB], se, he;
        load_run_at<KB, STREAM_MOD>(scale, n, k0, sv, se);
        load_run_at<KB, STREAM_MOD>(shift, n, k0, hv, he);
        realign_in<KB>(sv, se, start_offset(scale));
        realign_in<KB>(hv, he, start_offset(shift));
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            Pack<DT> xp, sp, hp;
            xp.v = xv[k0 + j];
            sp.v = sv[j];
            hp.v = hv[j];
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = xp.get(e);
                if constexpr (NORM == kLn)
                    v = v - mu;
                const float nv = v * rr;
                const float a = 1.0f + sp.get(e);
                const float m = nv * a;
                o[e] = m + hp.get(e);
            }
            xv[k0 + j] = Pack<DT>::make(o).v;
        }
    }
    store_run<K, true>(out, n, xv);
}

// Rows a workgroup shares (scale, shift, a broadcast gate) are staged once
// in LDS as groups instead of realigned by every wave for every row: the
// P = ceil(n / 8) groups of a row of n elements, group g at word g of a
// plane of P words. Slots from whole_slots<K>() on can reach past P; their
// indexes are clamped into the plane (the groups they stand for are
// neither summed nor stored).
template <int K>
__device__ __forceinline__ int staged_index(int k, int lane, int planes, int phase = 0)
{
    const int i = 64 * k + lane - phase;
    if (k >= 1 && k < whole_slots<K>())
        return i;
    return i < 0 ? 0 : (i < planes ? i : planes - 1);
}

// The groups of the row of n elements at p into the plane at dst.
template <int K>
__device__ __forceinline__ void stage_row(u32x4* dst, const void* p, int n)
{
    const int lane = threadIdx.x & 63;
    const int planes = (n + 7) >> 3;
    u32x4 g[K];
    load_groups<K, false>(p, n, g);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = 64 * k + lane;
        if (k < whole_slots<K>() || i < planes)
            dst[i] = g[k];
    }
}

// 1 + scale of the row of n elements at p, in binary32 (one_plus), into
// the planes a_lo (elements 0-3 of each group) and a_hi (4-7).
template <int K, int DT>
__device__ __forceinline__ void stage_one_plus(u32x4* a_lo, u32x4* a_hi, const void* p, int n)
{
    const int lane = threadIdx.x & 63;
    const int planes = (n + 7) >> 3;
    u32x4 g[K];
    load_groups<K, false>(p, n, g);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = 64 * k + lane;
        u32x4 lo, hi;
        one_plus<DT>(g[k], lo, hi);
        if (k < whole_slots<K>() || i < planes) {
            a_lo[i] = lo;
            a_hi[i] = hi;
        }
    }
}

// apply_store with the scale and shift rows staged in LDS: no per-row
// loads or realignment of them. ONE_PLUS: 1 + scale staged in binary32
// (stage_one_plus: a_lo, a_hi); otherwise the scale row as it is stored
// (stage_row at a_lo), 1 + scale formed per group with the same rounding.
template <int K, int DT, int NORM, bool ONE_PLUS>
__device__ __forceinline__ void apply_store_staged(u32x4 (&xv)[K], const u32x4* a_lo,
                                                   const u32x4* a_hi, const u32x4* h_lds, int n,
                                                   float mu, float rr, void* out, int phase = 0)
{
    const int lane = threadIdx.x & 63;
    const int planes = (n + 7) >> 3;
    // up to 9 slots the widened row fits beside the rest (one widening for
    // the sum and the apply: 1-2 % faster at D = 4100 on MI355X); longer
    // rows stay packed across the reduction, as in apply_store
    if constexpr (K > 9) {
#pragma unroll
        for (int k = 0; k < K; ++k)
            __asm__ volatile("" : "+v"(xv[k]));
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = staged_index<K>(k, lane, planes, phase);
        Pack<DT> xp, hp;
        xp.v = xv[k];
        hp.v = h_lds[i];
        if constexpr (ONE_PLUS) {
            xv[k] = modulate_group<DT, NORM == kLn>(xp, mu, rr, a_lo[i], a_hi[i], hp).v;
        } else {
            u32x4 lo, hi;
            one_plus<DT>(a_lo[i], lo, hi);
            xv[k] = modulate_group<DT, NORM == kLn>(xp, mu, rr, lo, hi, hp).v;
        }
    }
    store_run<K, true>(out, n, xv, phase);
}

}  // namespace regs
}  // namespace rga
