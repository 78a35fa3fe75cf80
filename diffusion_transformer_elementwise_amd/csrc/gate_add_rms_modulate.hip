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
// Pack path with row modulation of 2-byte rows (D % 8 == 0,
// D <= RGA_RMS_MAX_D, 16-byte aligned pointers, staged rows within one
// workgroup's 64 KB of LDS): two
// waves per workgroup, one row each. The workgroup first stages its batch's
// scale and shift rows, and a broadcast gate row, in LDS; then each wave
// loads x and u (and a full gate), forms x', stores it, reduces it and
// applies the modulation from LDS; the launch caps the workgroups per CU
// through the LDS it asks for (row_wg_lds in launch.hpp). Measured on MI355X
// at [2,32640,4096] inside a chain of the step's kernels: 349-350 us against
// 356 us for the register-row kernel of the element path, which 2-byte rows
// with row modulation took at any alignment before.
//
// Pack path with per-token modulation and for binary32 rows (kept as they
// were measured fastest), launch shape measured on MI355X: one wave per
// workgroup and one row per wave, nontemporal loads and stores. Every pack's x, u and g loads are
// issued before the first add, with no branch around a load (a branch per
// bounded load made the wave wait for each pack before issuing the next);
// each x_out pack is stored as soon as it is formed; scale and shift are read
// only for the apply phase, all packs before the first (through the caches
// for row modulation, streamed for per-token modulation). A broadcast gate
// row is read through the caches (it stays in L2), a full gate streams from
// HBM like x and u.
//
// Element path (any D, element-aligned pointers): for 2-byte rows of up to
// 8192 elements, one pass with the row realigned in registers (x_out is
// never read back); otherwise (binary32, longer rows) two passes over the
// row, moving spans of elements through LDS with 16-byte accesses, the
// second pass re-reading x_out.
#include "dtype.hpp"
#include "launch.hpp"
#include "row_regs.hpp"
#include "span.hpp"

#include <rga.h>

namespace rga {
namespace {

constexpr int kBlock = 64;
constexpr int kStage = 1024;  // element path: elements per span

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
    // every pack's loads are issued before the first add (no branch around a
    // load), so a wave keeps its whole row of x, u and g in flight
    using GP = Grouped<DT>;
    Pack<DT> xv[G], uv[G], gv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int h = vpr - 64 * i;
        xv[i] = GP::template load_clamped<true>(x, row + 64 * i, lane, h);
        uv[i] = GP::template load_clamped<true>(u, row + 64 * i, lane, h);
        gv[i] = FULL ? GP::template load_clamped<true>(g, row + 64 * i, lane, h)
                     : GP::template load_clamped<false>(g, b * vpr + 64 * i, lane, h);
    }
    Pack<DT> xn[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int h = vpr - 64 * i;
        const Pack<DT> xr = gate_add8<DT>(xv[i], uv[i], gv[i]);
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

    // the scale and shift rows likewise, before the first apply
    Pack<DT> scs[G], shs[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int h = vpr - 64 * i;
        scs[i] = MOD == kModToken ? GP::template load_clamped<true>(scale, row + 64 * i, lane, h)
                                  : GP::template load_clamped<false>(scale, b * vpr + 64 * i, lane, h);
        shs[i] = MOD == kModToken ? GP::template load_clamped<true>(shift, row + 64 * i, lane, h)
                                  : GP::template load_clamped<false>(shift, b * vpr + 64 * i, lane, h);
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int h = vpr - 64 * i;
        const Pack<DT> xr = GP::to_raw(xn[i]);
        const Pack<DT>& sc = scs[i];
        const Pack<DT>& sh = shs[i];
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

// The same sums as a xor butterfly over __shfl_xor, bit for bit: exchanges 1
// and 2 by DPP quad permutations, 4 and 8 by DPP half-row and row mirrors
// (once lanes 4q..4q+3 hold equal values the mirror partner of a lane holds
// what its xor-4 partner holds; likewise for 8 once groups of 8 agree), then
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

// Row modulation, kRowWaves waves per workgroup, sched_rows_per_wave(SCHED)
// rows per wave (launch.hpp; the library runs kSchedLibrary, one row per
// wave): rows kRowWaves * (R * blockIdx.x + j) + wave, j < R, of batch
// blockIdx.y. The dynamic LDS holds the batch's scale row at [0, vpr), its
// shift row at [vpr, 2 vpr) and, with a broadcast gate, its gate row at
// [2 vpr, 3 vpr), as 16-byte words in memory order; with kSchedOnePlus,
// 1 + scale in binary32 at [0, 2 vpr) (one_plus: elements 0-3, then 4-7 of
// each pack) and the shift and gate rows one plane further on. Lanes past
// the row end hold zeros (x' = +0 there, which adds +0 to the partial) and
// store nothing.
// WHOLE: D = 512 G (every lane's packs lie in the row): no bounds at all.
template <int G, bool FULL, int DT, bool WHOLE, int SCHED>
__device__ __forceinline__ void fused_staged_rows(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int vpr)
{
    static_assert(DT != kF32, "2-byte rows: a pack is one word, raw order is group order");
    constexpr int R = sched_rows_per_wave(SCHED);
    constexpr bool kOnePlus = SCHED == kSchedOnePlus;
    extern __shared__ u32x4 staged[];
    const int lane = threadIdx.x & (kBlock - 1);
    const int64_t b = blockIdx.y;
    // the wave index as a per-lane value (wave_in_group() would make it
    // scalar): the compiler then orders this loop's loads as the library's
    // timings were taken with
    const int64_t r0 = (int64_t)blockIdx.x * kRowWaves * R + (threadIdx.x / kBlock);
    u32x4* s_st = staged;
    u32x4* h_st = staged + (kOnePlus ? 2 : 1) * vpr;
    u32x4* g_st = staged + (kOnePlus ? 3 : 2) * vpr;

    // Rows other than WHOLE ones are held at the phase s of x's 128-byte
    // lines (lane t, pack i: pack 64i + t - s; as far as the packs have room
    // for it), so that each access instruction covers whole lines: the sum's
    // 64 partials are rotated back to lane order before the exchanges (bit
    // for bit the fixed order), and packs outside the row hold zeros and are
    // not stored.
    auto phase_of = [&](int64_t row) {
        if constexpr (WHOLE) {
            return 0;
        } else {
            const int lead = (int)((reinterpret_cast<uintptr_t>(static_cast<const u32x4*>(x) + row) >> 4) & 7u);
            const int room = 64 * G - vpr;
            return lead < room ? lead : room;
        }
    };
    auto load_pack = [&](const void* base, int64_t row, int i, int phase) {
        if constexpr (WHOLE) {
            return Pack<DT>::load_stream(base, row + 64 * i + lane);
        } else {
            const int p = 64 * i + lane - phase;
            const int pc = p < 0 ? 0 : (p < vpr ? p : vpr - 1);
            Pack<DT> v = Pack<DT>::load_stream(base, row + pc);
            const bool in = p >= 0 && p < vpr;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                v.v[d] = in ? v.v[d] : 0u;
            return v;
        }
    };
    auto load_row = [&](Pack<DT> (&xv)[G], Pack<DT> (&uv)[G], Pack<DT> (&gv)[FULL ? G : 1],
                        int64_t row, int phase) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            xv[i] = load_pack(x, row, i, phase);
            uv[i] = load_pack(u, row, i, phase);
            if constexpr (FULL)
                gv[i] = load_pack(g, row, i, phase);
        }
    };

    Pack<DT> xv[G], uv[G], gv[FULL ? G : 1];
    int phase = 0;
    if constexpr (SCHED == kSchedLoadsFirst) {
        // a wave past the last row (odd L) loads the last row and stores
        // nothing
        const int64_t row = (b * L + (r0 < L ? r0 : L - 1)) * vpr;
        phase = phase_of(row);
        load_row(xv, uv, gv, row, phase);
    }
    // the batch's rows, vpr <= 64 G words each: every load issued before any
    // LDS write (one round trip to the L2, not one per word a thread
    // stages), at most kS words of each per thread, indexes clamped and
    // writes guarded
    {
        constexpr int kS = (64 * G + kBlock * kRowWaves - 1) / (kBlock * kRowWaves);
        const u32x4* sc = static_cast<const u32x4*>(scale) + b * vpr;
        const u32x4* sh = static_cast<const u32x4*>(shift) + b * vpr;
        const u32x4* gr = static_cast<const u32x4*>(g) + b * vpr;
        u32x4 sv[kS], hv[kS], bv[FULL ? 1 : kS];
#pragma unroll
        for (int j = 0; j < kS; ++j) {
            const int w = (int)threadIdx.x + kBlock * kRowWaves * j;
            const int wc = w < vpr ? w : vpr - 1;
            sv[j] = load16(sc + wc);
            hv[j] = load16(sh + wc);
            if constexpr (!FULL)
                bv[FULL ? 0 : j] = load16(gr + wc);
        }
#pragma unroll
        for (int j = 0; j < kS; ++j) {
            const int w = (int)threadIdx.x + kBlock * kRowWaves * j;
            if (w < vpr) {
                if constexpr (kOnePlus) {
                    u32x4 lo, hi;
                    one_plus<DT>(sv[j], lo, hi);
                    s_st[w] = lo;
                    s_st[vpr + w] = hi;
                } else {
                    s_st[w] = sv[j];
                }
                h_st[w] = hv[j];
                if constexpr (!FULL)
                    g_st[w] = bv[FULL ? 0 : j];
            }
        }
    }
    __syncthreads();
    if (r0 >= L)
        return;
    if constexpr (SCHED != kSchedLoadsFirst) {
        phase = phase_of((b * L + r0) * vpr);
        load_row(xv, uv, gv, (b * L + r0) * vpr, phase);
    }

#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t r = r0 + (int64_t)kRowWaves * j;
        const int64_t row = (b * L + r) * vpr;
        const bool more = j + 1 < R && r + kRowWaves < L;
        constexpr int kQ = SCHED == kSchedPrefetch ? G : 1;
        Pack<DT> xq[kQ], uq[kQ], gq[FULL ? kQ : 1];
        int phase_q = 0;
        if constexpr (SCHED == kSchedPrefetch)
            if (more) {
                phase_q = phase_of(row + (int64_t)kRowWaves * vpr);
                load_row(xq, uq, gq, row + (int64_t)kRowWaves * vpr, phase_q);
            }

        Pack<DT> xn[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int p = 64 * i + lane - phase;  // the pack this lane holds
            const bool in = WHOLE || (p >= 0 && p < vpr);
            Pack<DT> gi;
            if constexpr (FULL) {
                gi = gv[FULL ? i : 0];
            } else if constexpr (WHOLE) {
                gi.v = g_st[p];
            } else {
                // zeros outside the row: x' = +0 there
                gi.v = g_st[p < 0 ? 0 : (p < vpr ? p : vpr - 1)];
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    gi.v[d] = in ? gi.v[d] : 0u;
            }
            const Pack<DT> xr = gate_add8<DT>(xv[i], uv[i], gi);
            if (in)
                xr.store_stream(x_out, row + p);
            xn[i] = xr;
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
        if constexpr (!WHOLE)
            acc = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane + phase) & 63) << 2,
                                                              __float_as_int(acc)));
        const float ms = wave_sum_dpp(acc) / d_float;
        const float t = ms + eps;
        const float q = sqrtf(t);
        const float rr = 1.0f / q;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int p = 64 * i + lane - phase;
            // scale and shift at the pack's index, clamped into the row for
            // packs outside it (not stored)
            const int pc = WHOLE ? p : (p < 0 ? 0 : (p < vpr ? p : vpr - 1));
            Pack<DT> o;
            if constexpr (kOnePlus) {
                Pack<DT> h_;
                h_.v = h_st[pc];
                o = modulate_group<DT, false>(xn[i], 0.0f, rr, s_st[pc], s_st[vpr + pc], h_);
            } else {
                Pack<DT> s_, h_;
                s_.v = s_st[pc];
                h_.v = h_st[pc];
                float of[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float n = xn[i].get(e) * rr;
                    const float a = 1.0f + s_.get(e);
                    const float m = n * a;
                    of[e] = m + h_.get(e);
                }
                o = Pack<DT>::make(of);
            }
            if (WHOLE || (p >= 0 && p < vpr))
                o.store_stream(y, row + p);
        }

        if (j + 1 < R) {
            if (!more)
                return;
            if constexpr (SCHED == kSchedPrefetch) {
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    xv[i] = xq[i];
                    uv[i] = uq[i];
                    if constexpr (FULL)
                        gv[FULL ? i : 0] = gq[FULL ? i : 0];
                }
                phase = phase_q;
            } else {
                phase = phase_of(row + (int64_t)kRowWaves * vpr);
                load_row(xv, uv, gv, row + (int64_t)kRowWaves * vpr, phase);
            }
        }
    }
}

template <int G, bool FULL, int DT, bool WHOLE>
__global__ __launch_bounds__(kBlock * kRowWaves) void gate_add_rms_modulate_staged_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int vpr)
{
    fused_staged_rows<G, FULL, DT, WHOLE, kSchedLibrary>(x, u, g, scale, shift, eps, d_float,
                                                         x_out, y, L, vpr);
}

// The staged fused call in schedule SCHED (kSched*, launch.hpp), for
// measurement: bf16 rows of kSchedD = 4096 elements (G = 8, whole rows),
// broadcast gate, row modulation.
template <int SCHED>
__global__ __launch_bounds__(kBlock * kRowWaves) void gate_add_rms_modulate_variant_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int vpr)
{
    fused_staged_rows<8, false, kBF16, true, SCHED>(x, u, g, scale, shift, eps, d_float, x_out,
                                                    y, L, vpr);
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

// Element path: one wave per row; grid x = row l, y = batch b. Spans of
// kStage elements move through LDS with 16-byte accesses (span.hpp). Pass 1
// forms x' for a span, stores it to x_out and, from its rounded value put in
// LDS at byte i * es (every group of 8 in whole 16-byte words), lane j adds
// up groups j, j + 64, ... of the span in the fixed order.
// Pass 2 re-reads x_out (written by other lanes of this wave: the barrier
// between the passes orders those writes before the reads) and writes y.
template <bool FULL, int DT, int MOD>
__global__ __launch_bounds__(kBlock) void gate_add_rms_modulate_generic_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int64_t D)
{
    using S = Span<DT, kStage>;
    // five spans from the launch's dynamic LDS (5 * kWords words): a static
    // buffer would also be placed, unused, in this file's LDS-staged kernel
    extern __shared__ u32x4 rowbuf[];
    u32x4* r0 = rowbuf;
    u32x4* r1 = r0 + S::kWords;
    u32x4* r2 = r1 + S::kWords;
    u32x4* r3 = r2 + S::kWords;
    u32x4* ra = r3 + S::kWords;  // the rounded x' at byte i * es, for the sum
    const int lane = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t grow = FULL ? row : b * D;
    const int64_t mrow = (MOD == kModToken) ? row : b * D;

    float acc = 0.0f;
    for (int64_t s0 = 0; s0 < D; s0 += kStage) {
        const int cnt = (D - s0 < kStage) ? (int)(D - s0) : kStage;
        const void* px = elem_ptr<DT>(x, row + s0);
        const void* pu = elem_ptr<DT>(u, row + s0);
        const void* pg = elem_ptr<DT>(g, grow + s0);
        void* po = elem_ptr<DT>(x_out, row + s0);
        S::template load<true>(px, cnt, r0);
        S::template load<true>(pu, cnt, r1);
        S::template load<FULL>(pg, cnt, r2);
        __syncthreads();
        const int mx = S::offset(px), mu = S::offset(pu), mg = S::offset(pg), mo = S::offset(po);
        for (int i = lane; i < cnt; i += kBlock) {
            const float p = S::get(r1, mu, i) * S::get(r2, mg, i);
            const float sum = S::get(r0, mx, i) + p;
            S::put(r3, mo, i, sum);
            S::put(ra, 0, i, sum);
        }
        __syncthreads();
        S::template store<true>(po, cnt, r3);
#pragma unroll
        for (int k = 0; k < kStage / 512; ++k) {
            const int gi = lane + kBlock * k;
            if (8 * gi >= cnt)
                continue;
            const Pack<DT> pk = S::group(ra, gi);  // the rounded x'
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (8 * gi + e < cnt) {
                    const float a = pk.get(e);
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

    for (int64_t s0 = 0; s0 < D; s0 += kStage) {
        const int cnt = (D - s0 < kStage) ? (int)(D - s0) : kStage;
        const void* px = elem_ptr<DT>(x_out, row + s0);
        const void* ps = elem_ptr<DT>(scale, mrow + s0);
        const void* ph = elem_ptr<DT>(shift, mrow + s0);
        void* py = elem_ptr<DT>(y, row + s0);
        S::template load<false>(px, cnt, r0);
        S::template load<MOD == kModToken>(ps, cnt, r1);
        S::template load<MOD == kModToken>(ph, cnt, r2);
        __syncthreads();
        const int mx = S::offset(px), ms2 = S::offset(ps), mh = S::offset(ph), my = S::offset(py);
        for (int i = lane; i < cnt; i += kBlock) {
            const float n = S::get(r0, mx, i) * rr;
            const float a = 1.0f + S::get(r1, ms2, i);
            const float m = n * a;
            S::put(r3, my, i, m + S::get(r2, mh, i));
        }
        __syncthreads();
        S::template store<true>(py, cnt, r3);
        __syncthreads();
    }
}

// 16 bytes of an LDS row buffer starting at byte pos, pos mod 16 = sh the
// same in every lane; word indexes are clamped to [0, qmax] (the clamped
// bytes are never used). O: sh fixed at compile time (0..15), or -1.
template <int O>
__device__ __forceinline__ u32x4 lds_bytes16(const u32x4* buf, int pos, int sh, int qmax)
{
    int q = pos >> 4;
    q = q < qmax ? q : qmax;
    const u32x4 c = buf[q < 0 ? 0 : q];
    if constexpr (O == 0)
        return c;
    else
        return window_o<O>(c, buf[q + 1 < 0 ? 0 : q + 1], sh);
}

// Element path for rows that fit in LDS but not in registers (binary32
// rows; 2-byte rows over 8192 elements): one workgroup of NW waves per row
// (lds_row_waves: about one per 4 KB of row), x, u and g read once. The waves form x' over chunks of x_out's aligned
// 16-byte words (each input read realigned to x_out, realign.hpp), store it
// and keep the words in a dynamic LDS buffer; wave 0 takes the fixed-order
// sum from LDS (group g is the 16 or 32 bytes at x_out's offset + g * 8 *
// es); all waves then write y over chunks of y's aligned words, x' taken
// from LDS realigned to y. x_out is never read back.
// dynamic LDS per workgroup, less room for the few static bytes
constexpr int64_t kMaxRowLds = 65536 - 256;

// LDS bytes of the row buffer: x_out's window words (at most one more than
// the row's aligned words) and two spare words a cut may touch.
int64_t row_lds_bytes(int64_t D, int es) { return ((D * es + 15) / 16 + 3) * 16; }

template <bool FULL, int DT, int MOD, int NW>
__global__ __launch_bounds__(kBlock * NW) void gate_add_rms_modulate_lds_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int64_t D)
{
    extern __shared__ u32x4 rowbuf[];
    __shared__ float factor;
    constexpr int es = DT == kF32 ? 4 : 2;
    constexpr bool kTok = MOD == kModToken;
    // the wave index as a per-lane value (wave_in_group() would make it
    // scalar): the compiler then schedules this kernel as its timings
    // were taken with
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t grow = FULL ? row : b * D;
    const int64_t mrow = kTok ? row : b * D;
    const int n = (int)D;
    const int64_t nbytes = D * es;
    using W = Word<DT>;

    void* pxo = elem_ptr<DT>(x_out, row);
    const int mxo = start_offset(pxo);
    const int64_t words_xo = window_words(pxo, nbytes);
    const int lead_xo = line_lead(pxo);
    for (int64_t c = wave; 64 * c - lead_xo < words_xo; c += NW) {
        const int64_t wbase = 64 * c - lead_xo;  // chunks of whole 128-byte lines
        const ChunkWords fxw = fetch_for_chunk<true>(elem_ptr<DT>(x, row), nbytes, mxo, wbase);
        const ChunkWords fuw = fetch_for_chunk<true>(elem_ptr<DT>(u, row), nbytes, mxo, wbase);
        const ChunkWords fgw = fetch_for_chunk<FULL>(elem_ptr<DT>(g, grow), nbytes, mxo, wbase);
        const u32x4 xw = chunk_word(fxw);
        const u32x4 uw = chunk_word(fuw);
        const u32x4 gw = chunk_word(fgw);
        float o[W::kN];
#pragma unroll
        for (int e = 0; e < W::kN; ++e) {
            const float p = W::get(uw, e) * W::get(gw, e);
            o[e] = W::get(xw, e) + p;
        }
        const u32x4 v = W::make(o);
        store_chunk<true>(pxo, nbytes, wbase, v);
        const int64_t w = wbase + lane;
        if (w >= 0 && w < words_xo)
            rowbuf[w] = v;
    }
    __syncthreads();

    // the buffer's row starts at byte mxo; it holds (nbytes + 15) / 16 + 3
    // words, so reading words q and q + 1 with q <= words_xo stays inside
    // (words past words_xo - 1 only supply bytes past the row)
    const int qmax = (int)words_xo;
    if (wave == 0) {
        const int groups = (n + 7) >> 3;
        float acc = 0.0f;
        // one branch on the buffer's offset (uniform) around the sum, so each
        // group read is cut with fixed dword picks
        dispatch_offset(mxo, [&](auto off) {
            constexpr int O = decltype(off)::value;
            auto group_at = [&](int gi) {
                Pack<DT> p;
                if constexpr (DT == kF32) {
                    p.a = lds_bytes16<O>(rowbuf, mxo + 32 * gi, mxo, qmax);
                    p.b = lds_bytes16<O>(rowbuf, mxo + 32 * gi + 16, mxo, qmax);
                } else {
                    p.v = lds_bytes16<O>(rowbuf, mxo + 16 * gi, mxo, qmax);
                }
                return p;
            };
            // batches of U groups wholly inside the row: the U reads are issued
            // before any is added (one LDS round trip per batch); the additions
            // keep the fixed order. The rest, masked, below.
            constexpr int U = DT == kF32 ? 4 : 8;
            const int n_whole = n >> 3;
            int gi = lane;
            for (; gi + kBlock * (U - 1) < n_whole; gi += kBlock * U) {
                Pack<DT> p[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    p[u] = group_at(gi + kBlock * u);
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float a = p[u].get(e);
                        const float sa = a * a;
                        acc = acc + sa;
                    }
                }
            }
            for (; gi < groups; gi += kBlock) {
                const Pack<DT> p = group_at(gi);
                const bool whole = 8 * gi + 8 <= n;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (whole || 8 * gi + e < n) {
                        const float a = p.get(e);
                        const float sa = a * a;
                        acc = acc + sa;
                    }
                }
            }
        });
#pragma unroll
        for (int m = 1; m < 64; m <<= 1)
            acc = acc + __shfl_xor(acc, m);
        const float ms = acc / d_float;
        const float t = ms + eps;
        const float q = sqrtf(t);
        if (lane == 0)
            factor = 1.0f / q;
    }
    __syncthreads();
    const float rr = factor;

    void* py = elem_ptr<DT>(y, row);
    const int my = start_offset(py);
    const int64_t words_y = window_words(py, nbytes);
    const int sh = (mxo - my) & 15;
    const int lead_y = line_lead(py);
    // one branch on the row's LDS cut (uniform) around the y loop
    dispatch_offset(sh, [&](auto off) {
        constexpr int O = decltype(off)::value;
        for (int64_t c = wave; 64 * c - lead_y < words_y; c += NW) {
            const int64_t wbase = 64 * c - lead_y;
            // y word w holds row bytes [16w - my, +16): buffer bytes from 16w - my + mxo
            const int pos = (int)(16 * (wbase + lane)) - my + mxo;
            const u32x4 xw = lds_bytes16<O>(rowbuf, pos, sh, qmax);
            const ChunkWords fsw =
                fetch_for_chunk<kTok>(elem_ptr<DT>(scale, mrow), nbytes, my, wbase);
            const ChunkWords fhw =
                fetch_for_chunk<kTok>(elem_ptr<DT>(shift, mrow), nbytes, my, wbase);
            const u32x4 sw = chunk_word(fsw);
            const u32x4 hw = chunk_word(fhw);
            float o[W::kN];
#pragma unroll
            for (int e = 0; e < W::kN; ++e) {
                const float nv = W::get(xw, e) * rr;
                const float a = 1.0f + W::get(sw, e);
                const float m = nv * a;
                o[e] = m + W::get(hw, e);
            }
            store_chunk<true>(py, nbytes, wbase, W::make(o));
        }
    });
}

// Element path for 2-byte types with D <= 512 * K: one wave per row. x, u
// and g are read once and realigned in registers (realign.hpp) to groups,
// x' is formed there, written to x_out realigned to its offset, and the
// rounded x' groups stay in registers for the modulation (row_regs.hpp), so
// x_out is never read back.
// Row modulation of 2-byte rows held in registers: kRowWaves waves per
// workgroup, one row each. Before any row is loaded the workgroup stages
// its batch's rows in the dynamic LDS once, as groups in planes of
// P = ceil(D / 8) words (row_regs.hpp): wave 0 the scale row as stored (at
// [0, P); 1 + scale is formed per group) and a broadcast gate row (at
// [2P, 3P)), wave 1 the shift row (at [P, 2P)). Staging the scale at its
// 2-byte size rather than widened leaves room for 6 workgroups per CU,
// where the widened staging allowed 4.
template <int K, bool FULL, int DT>
__global__ __launch_bounds__(kBlock * kRowWaves) void gate_add_rms_modulate_regs_staged_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int64_t D)
{
    extern __shared__ u32x4 staged[];
    const int wave = wave_in_group();
    const int64_t b = blockIdx.y;
    const int64_t r = (int64_t)blockIdx.x * kRowWaves + wave;
    const int n = (int)D;
    static_assert(kRowWaves == 2, "staged rows split over two waves");
    const int planes = (n + 7) >> 3;
    u32x4* h_st = staged + planes;
    u32x4* g_st = staged + 2 * planes;
    if (wave == 0) {
        regs::stage_row<K>(staged, elem_ptr<DT>(scale, b * D), n);
        if constexpr (!FULL)
            regs::stage_row<K>(g_st, elem_ptr<DT>(g, b * D), n);
    } else {
        regs::stage_row<K>(h_st, elem_ptr<DT>(shift, b * D), n);
    }
    __syncthreads();
    if (r >= L)
        return;
    const int64_t row = (b * L + r) * D;
    const int lane = threadIdx.x & (kBlock - 1);
    const void* px = elem_ptr<DT>(x, row);
    // every stream of the row at the phase of x's 128-byte lines (each
    // access instruction covering whole lines where the streams share x's
    // line position), as far as the slots have room for it
    const int room = 64 * K - planes;
    const int phase = line_lead(px) < room ? line_lead(px) : room;

    u32x4 xv[K];
    {
        // every input's loads issued before any is realigned
        u32x4 uv[K], gv[FULL ? K : 1], xe, ue, ge;
        const void* pu = elem_ptr<DT>(u, row);
        load_run<K, true>(px, n, xv, xe, phase);
        load_run<K, true>(pu, n, uv, ue, phase);
        if constexpr (FULL)
            load_run<K, true>(elem_ptr<DT>(g, row), n, gv, ge, phase);
        realign_in<K>(xv, xe, start_offset(px));
        realign_in<K>(uv, ue, start_offset(pu));
        if constexpr (FULL)
            realign_in<K>(gv, ge, start_offset(elem_ptr<DT>(g, row)));
#pragma unroll
        for (int k = 0; k < K; ++k) {
            Pack<DT> a, c, e;
            a.v = xv[k];
            c.v = uv[k];
            e.v = FULL ? gv[FULL ? k : 0] : g_st[regs::staged_index<K>(k, lane, planes, phase)];
            xv[k] = gate_add8<DT>(a, c, e).v;
        }
    }
    store_run<K, true>(elem_ptr<DT>(x_out, row), n, xv, phase);
    float mu, rr;
    regs::row_factors<K, DT, regs::kRms>(xv, n, d_float, eps, &mu, &rr, phase);
    regs::apply_store_staged<K, DT, regs::kRms, false>(xv, staged, nullptr, h_st, n, mu, rr,
                                                elem_ptr<DT>(y, row), phase);
}

template <int K, bool FULL, int DT, int MOD>
__global__ __launch_bounds__(kBlock) void gate_add_rms_modulate_regs_kernel(
    const void* x, const void* u, const void* g, const void* scale,
    const void* shift, float eps, float d_float, void* x_out, void* y,
    int64_t L, int64_t D)
{
    const int64_t b = blockIdx.y;
    const int64_t row = (b * L + blockIdx.x) * D;
    const int64_t grow = FULL ? row : b * D;
    const int64_t mrow = (MOD == kModToken) ? row : b * D;
    const int n = (int)D;

    u32x4 xv[K];
    {
        // every input's loads issued before any is realigned
        u32x4 uv[K], gv[K], xe, ue, ge;
        const void* px = elem_ptr<DT>(x, row);
        const void* pu = elem_ptr<DT>(u, row);
        const void* pg = elem_ptr<DT>(g, grow);
        load_run<K, true>(px, n, xv, xe);
        load_run<K, true>(pu, n, uv, ue);
        load_run<K, FULL>(pg, n, gv, ge);
        realign_in<K>(xv, xe, start_offset(px));
        realign_in<K>(uv, ue, start_offset(pu));
        realign_in<K>(gv, ge, start_offset(pg));
#pragma unroll
        for (int k = 0; k < K; ++k) {
            Pack<DT> a, c, e;
            a.v = xv[k];
            c.v = uv[k];
            e.v = gv[k];
            xv[k] = gate_add8<DT>(a, c, e).v;
        }
    }
    store_run<K, true>(elem_ptr<DT>(x_out, row), n, xv);
    float mu, rr;
    regs::row_factors<K, DT, regs::kRms>(xv, n, d_float, eps, &mu, &rr);
    regs::apply_store<K, DT, MOD == kModToken, regs::kRms>(xv, elem_ptr<DT>(scale, mrow),
                                                            elem_ptr<DT>(shift, mrow), n, mu, rr,
                                                            elem_ptr<DT>(y, row));
}

typedef void (*regs_kernel_t)(const void*, const void*, const void*, const void*, const void*,
                              float, float, void*, void*, int64_t, int64_t);

// Slots per lane for the register-resident element path: the smallest entry
// >= ceil(ceil(D / 8) / 64); longer rows (and binary32) take the LDS path.
using regs::kRegsLadder;

int pick_regs_slots(int64_t slots)
{
    for (int i = 0; i < 8; ++i)
        if (slots <= kRegsLadder[i])
            return kRegsLadder[i];
    return 0;
}

template <bool FULL, int DT>
const void* pick_regs_staged(int K)
{
    switch (K) {
    case 1: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<1, FULL, DT>);
    case 2: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<2, FULL, DT>);
    case 4: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<4, FULL, DT>);
    case 6: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<6, FULL, DT>);
    case 8: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<8, FULL, DT>);
    case 9: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<9, FULL, DT>);
    case 12: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<12, FULL, DT>);
    default: return reinterpret_cast<const void*>(&gate_add_rms_modulate_regs_staged_kernel<16, FULL, DT>);
    }
}

template <bool FULL, int DT, int MOD>
regs_kernel_t pick_regs(int64_t slots)
{
    regs_kernel_t t[] = {&gate_add_rms_modulate_regs_kernel<1, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<2, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<4, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<6, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<8, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<9, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<12, FULL, DT, MOD>,
                         &gate_add_rms_modulate_regs_kernel<16, FULL, DT, MOD>};
    for (int i = 0; i < 8; ++i)
        if (slots <= kRegsLadder[i])
            return t[i];
    return nullptr;
}

typedef void (*fused_kernel_t)(const void*, const void*, const void*,
                               const void*, const void*, float, float, void*,
                               void*, int64_t, int);

constexpr int kLadder[] = {1, 2, 4, 6, 8, 9, 12, 16};
constexpr int kLadderSize = sizeof(kLadder) / sizeof(kLadder[0]);
static_assert(RGA_RMS_MAX_D / 512 == 16, "ladder tops out at RGA_RMS_MAX_D");

template <bool FULL, int DT, int MOD>
fused_kernel_t pick(int groups)
{
    fused_kernel_t t[] = {&gate_add_rms_modulate_kernel<1, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<2, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<4, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<6, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<8, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<9, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<12, FULL, DT, MOD>,
                          &gate_add_rms_modulate_kernel<16, FULL, DT, MOD>};
    static_assert(sizeof(t) / sizeof(t[0]) == kLadderSize, "one kernel per ladder entry");
    for (int i = 0; i < kLadderSize; ++i)
        if (groups <= kLadder[i])
            return t[i];
    return nullptr;
}

template <int G, bool FULL, int DT>
const void* staged_kernel(bool whole)
{
    return whole ? reinterpret_cast<const void*>(&gate_add_rms_modulate_staged_kernel<G, FULL, DT, true>)
                 : reinterpret_cast<const void*>(&gate_add_rms_modulate_staged_kernel<G, FULL, DT, false>);
}

// the staged kernel for rows of `groups` packs per lane; `whole`: the row is
// exactly 64 * groups packs (D = 512 G)
template <bool FULL, int DT>
const void* pick_staged(int groups, bool whole)
{
    const void* t[] = {staged_kernel<1, FULL, DT>(false), staged_kernel<2, FULL, DT>(false),
                       staged_kernel<4, FULL, DT>(false), staged_kernel<6, FULL, DT>(false),
                       staged_kernel<8, FULL, DT>(false), staged_kernel<9, FULL, DT>(false),
                       staged_kernel<12, FULL, DT>(false), staged_kernel<16, FULL, DT>(false)};
    const void* w[] = {staged_kernel<1, FULL, DT>(true), staged_kernel<2, FULL, DT>(true),
                       staged_kernel<4, FULL, DT>(true), staged_kernel<6, FULL, DT>(true),
                       staged_kernel<8, FULL, DT>(true), staged_kernel<9, FULL, DT>(true),
                       staged_kernel<12, FULL, DT>(true), staged_kernel<16, FULL, DT>(true)};
    static_assert(sizeof(t) / sizeof(t[0]) == kLadderSize, "one kernel per ladder entry");
    for (int i = 0; i < kLadderSize; ++i)
        if (groups <= kLadder[i])
            return (whole && groups == kLadder[i]) ? w[i] : t[i];
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <bool FULL, int DT, int MOD>
const void* lds_kernel(int w)
{
    switch (w) {
    case 2: return reinterpret_cast<const void*>(&gate_add_rms_modulate_lds_kernel<FULL, DT, MOD, 2>);
    case 4: return reinterpret_cast<const void*>(&gate_add_rms_modulate_lds_kernel<FULL, DT, MOD, 4>);
    default: return reinterpret_cast<const void*>(&gate_add_rms_modulate_lds_kernel<FULL, DT, MOD, 8>);
    }
}

// Element path: register rows for 2-byte rows of up to 8192 elements, then
// the LDS-staged rows, then the two-pass kernel.
template <bool FULL, int DT, int MOD>
hipError_t launch_element(const void* x, const void* u, const void* g,
                          const void* scale, const void* shift, float eps,
                          void* x_out, void* y, int64_t B, int64_t L, int64_t D,
                          hipStream_t stream, int wg_per_cu)
{
    float d_float = (float)D;
    void* args[] = {&x, &u, &g, &scale, &shift, &eps, &d_float, &x_out, &y, &L, &D};
    if constexpr (DT != kF32 && MOD == kModRow) {
        const int K = pick_regs_slots(ceil_div(ceil_div(D, 8), 64));
        if (K > 0) {
            // two rows per workgroup with the scale, the shift (and a
            // broadcast gate) row staged once (planes of ceil(D / 8)
            // words), occupancy capped
            const int64_t stage = (FULL ? 2 : 3) * 16 * ceil_div(D, 8);
            return hipLaunchKernel(pick_regs_staged<FULL, DT>(K),
                                   dim3((uint32_t)ceil_div(L, kRowWaves), (uint32_t)B),
                                   dim3(kBlock * kRowWaves), args,
                                   (size_t)row_wg_lds(2 * D, stage, kFusedElemRowBudget,
                                                      wg_per_cu),
                                   stream);
        }
    }
    if constexpr (DT != kF32) {
        regs_kernel_t rk = pick_regs<FULL, DT, MOD>(ceil_div(ceil_div(D, 8), 64));
        if (rk != nullptr)
            return hipLaunchKernel(reinterpret_cast<const void*>(rk),
                                   dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args, 0,
                                   stream);
    }
    const int64_t lds = row_lds_bytes(D, DT == kF32 ? 4 : 2);
    if (lds <= kMaxRowLds) {
        const int w = lds_row_waves(D * (DT == kF32 ? 4 : 2));
        return hipLaunchKernel(lds_kernel<FULL, DT, MOD>(w), dim3((uint32_t)L, (uint32_t)B),
                               dim3(kBlock * w), args, (size_t)lds, stream);
    }
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&gate_add_rms_modulate_generic_kernel<FULL, DT, MOD>),
        dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args,
        (size_t)(5 * 16 * Span<DT, kStage>::kWords), stream);
}

template <bool FULL, int DT, int MOD>
hipError_t launch_typed(const void* x, const void* u, const void* g,
                        const void* scale, const void* shift, float eps,
                        void* x_out, void* y, int64_t B, int64_t L, int64_t D,
                        bool fast, hipStream_t stream, int wg_per_cu)
{
    constexpr int64_t es = DT == kF32 ? 4 : 2;
    const int64_t stage = (FULL ? 2 : 3) * D * es;
    if constexpr (DT != kF32 && MOD == kModRow) {
        if (fast && stage <= kMaxStagedLds) {
            float d_float = (float)D;
            int vpr = (int)(D / 8);
            const void* k = pick_staged<FULL, DT>((int)ceil_div(vpr, 64), vpr % 64 == 0);
            if (k == nullptr)
                return hipErrorInvalidValue;
            void* args[] = {&x, &u, &g, &scale, &shift, &eps, &d_float, &x_out, &y, &L, &vpr};
            return hipLaunchKernel(k, dim3((uint32_t)ceil_div(L, kRowWaves), (uint32_t)B),
                                   dim3(kBlock * kRowWaves), args,
                                   (size_t)row_wg_lds(D * es, stage, kFusedRowBudget, wg_per_cu),
                                   stream);
        }
    }
    // otherwise 2-byte rows with row modulation take the register-row kernel
    // (aligned or not: on MI355X it ran 1-3 % faster than the one-wave pack
    // kernel there, and 1-3 % slower with per-token modulation, which keeps
    // the pack kernel, as binary32 does)
    if constexpr (DT != kF32 && MOD == kModRow) {
        return launch_element<FULL, DT, MOD>(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                                             stream, wg_per_cu);
    } else {
        if (!fast)
            return launch_element<FULL, DT, MOD>(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                                                 stream, wg_per_cu);
        float d_float = (float)D;
        int vpr = (int)(D / 8);
        fused_kernel_t k = pick<FULL, DT, MOD>((int)ceil_div(vpr, 64));
        if (k == nullptr)
            return hipErrorInvalidValue;
        void* args[] = {&x, &u, &g, &scale, &shift, &eps, &d_float, &x_out, &y, &L, &vpr};
        return hipLaunchKernel(reinterpret_cast<const void*>(k),
                               dim3((uint32_t)L, (uint32_t)B), dim3(kBlock), args, 0,
                               stream);
    }
}

template <int DT>
hipError_t launch_dt(const void* x, const void* u, const void* g,
                     const void* scale, const void* shift, float eps,
                     void* x_out, void* y, int64_t B, int64_t L, int64_t D,
                     int gate_mode, int mod_mode, bool fast, hipStream_t stream, int w)
{
    const bool full = gate_mode == RGA_GATE_FULL;
    const bool token = mod_mode == RGA_MOD_TOKEN;
    if (full && token)
        return launch_typed<true, DT, kModToken>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream, w);
    if (full)
        return launch_typed<true, DT, kModRow>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream, w);
    if (token)
        return launch_typed<false, DT, kModToken>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream, w);
    return launch_typed<false, DT, kModRow>(x, u, g, scale, shift, eps, x_out, y, B, L, D, fast, stream, w);
}

}  // namespace

// Grid x is L workgroups of 64 lanes, or of 64 lds_row_waves(D * es) lanes for the
// LDS-staged rows; its size in work-items must fit 32 bits.
bool gate_add_rms_modulate_grid_fits(int64_t B, int64_t L, int64_t D, int es, bool fast)
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

hipError_t launch_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                                const void* shift, float eps, void* x_out, void* y, int64_t B,
                                int64_t L, int sched, hipStream_t stream)
{
    static_assert(kSchedD == 512 * 8, "whole rows of 8 packs per lane");
    const void* k = nullptr;
    switch (sched) {
    case kSchedLibrary: k = reinterpret_cast<const void*>(&gate_add_rms_modulate_variant_kernel<kSchedLibrary>); break;
    case kSchedLoadsFirst: k = reinterpret_cast<const void*>(&gate_add_rms_modulate_variant_kernel<kSchedLoadsFirst>); break;
    case kSchedOnePlus: k = reinterpret_cast<const void*>(&gate_add_rms_modulate_variant_kernel<kSchedOnePlus>); break;
    case kSchedTwoRows: k = reinterpret_cast<const void*>(&gate_add_rms_modulate_variant_kernel<kSchedTwoRows>); break;
    case kSchedPrefetch: k = reinterpret_cast<const void*>(&gate_add_rms_modulate_variant_kernel<kSchedPrefetch>); break;
    default: return hipErrorInvalidValue;
    }
    float d_float = (float)kSchedD;
    int vpr = (int)(kSchedD / 8);
    void* args[] = {&x, &u, &g, &scale, &shift, &eps, &d_float, &x_out, &y, &L, &vpr};
    const int64_t row_bytes = kSchedD * 2;
    // scale (two planes with kSchedOnePlus), shift and gate rows
    const int64_t stage = (sched == kSchedOnePlus ? 4 : 3) * row_bytes;
    return hipLaunchKernel(
        k, dim3((uint32_t)ceil_div(L, kRowWaves * sched_rows_per_wave(sched)), (uint32_t)B),
        dim3(kBlock * kRowWaves), args, (size_t)row_wg_lds(row_bytes, stage, kFusedRowBudget, 0),
        stream);
}

hipError_t launch_gate_add_rms_modulate(const void* x, const void* u,
                                        const void* g, const void* scale,
                                        const void* shift, float eps,
                                        void* x_out, void* y, int64_t B,
                                        int64_t L, int64_t D, int gate_mode,
                                        int mod_mode, int dtype, bool fast,
                                        hipStream_t stream, int wg_per_cu)
{
    switch (dtype) {
    case RGA_DTYPE_F16:
        return launch_dt<kF16>(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode, fast, stream, wg_per_cu);
    case RGA_DTYPE_F32:
        return launch_dt<kF32>(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode, fast, stream, wg_per_cu);
    default:
        return launch_dt<kBF16>(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode, fast, stream, wg_per_cu);
    }
}

}  // namespace rga
