// C ABI of the library (include/rga.h, include/rga_measure.h): host-side
// validation, then one kernel launch on the caller's stream.
//
// Validation order (the first failing rule decides the status):
//   1. RGA_ERR_INVALID_ARG: a negative dimension, a bad gate_mode, a
//      non-finite or negative eps, B*L*D*2 bytes overflowing int64;
//   2. RGA_OK without a launch when B*L*D == 0 (pointers may be NULL);
//   3. RGA_ERR_INVALID_ARG: a NULL pointer;
//   4. RGA_ERR_UNSUPPORTED: D % 8 != 0, a pointer not 16-byte aligned, D
//      above RGA_RMS_MAX_D (modulation), a grid beyond the dispatch limit;
//   5. RGA_ERR_ALIAS: out overlapping an input other than the exact in-place
//      aliases each call allows.
// The gate-add rejection of unsupported inputs mirrors the residual-gate
// page's test list ("unsupported input rejection"); the bf16-only contract
// mirrors the modulation page's guard that admits only bf16 tensors.
#include <rga.h>
#include <rga_measure.h>

#include <cmath>
#include <cstdint>

#include "launch.hpp"

namespace {

struct Range {
    uintptr_t lo;
    uintptr_t hi;  // exclusive
};

Range range_of(const void* p, int64_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// elems = B*L*D and bytes = 2*elems without int64 overflow.
bool sizes(int64_t B, int64_t L, int64_t D, int64_t* elems, int64_t* bytes)
{
    int64_t bl = 0;
    if (__builtin_mul_overflow(B, L, &bl))
        return false;
    if (__builtin_mul_overflow(bl, D, elems))
        return false;
    return !__builtin_mul_overflow(*elems, (int64_t)2, bytes);
}

}  // namespace

extern "C" {

int rga_check_residual_gate_add(const void* x, const void* u, const void* g,
                                const void* out, int64_t B, int64_t L,
                                int64_t D, int gate_mode)
{
    if (B < 0 || L < 0 || D < 0)
        return RGA_ERR_INVALID_ARG;
    if (gate_mode != RGA_GATE_FULL && gate_mode != RGA_GATE_BCAST)
        return RGA_ERR_INVALID_ARG;
    int64_t n = 0, bytes = 0;
    if (!sizes(B, L, D, &n, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !u || !g || !out)
        return RGA_ERR_INVALID_ARG;
    if (D % 8 != 0)
        return RGA_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(u) || !aligned16(g) || !aligned16(out))
        return RGA_ERR_UNSUPPORTED;
    if (!rga::gate_add_grid_fits(B, L, D, gate_mode))
        return RGA_ERR_UNSUPPORTED;

    const bool full = gate_mode == RGA_GATE_FULL;
    const int64_t gate_bytes = full ? bytes : B * D * 2;  // <= bytes
    const Range o = range_of(out, bytes);
    if (overlaps(o, range_of(x, bytes)) && out != x)
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(u, bytes)) && out != u)
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(g, gate_bytes)) && !(full && out == g))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int rga_check_rms_modulate(const void* x, const void* scale,
                           const void* shift, float eps, const void* out,
                           int64_t B, int64_t L, int64_t D)
{
    if (B < 0 || L < 0 || D < 0)
        return RGA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f)
        return RGA_ERR_INVALID_ARG;
    int64_t n = 0, bytes = 0;
    if (!sizes(B, L, D, &n, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !scale || !shift || !out)
        return RGA_ERR_INVALID_ARG;
    if (D % 8 != 0 || D > RGA_RMS_MAX_D)
        return RGA_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(scale) || !aligned16(shift) ||
        !aligned16(out))
        return RGA_ERR_UNSUPPORTED;
    if (!rga::rms_modulate_grid_fits(B, L, D))
        return RGA_ERR_UNSUPPORTED;

    const int64_t row_bytes = B * D * 2;
    const Range o = range_of(out, bytes);
    if (overlaps(o, range_of(x, bytes)) && out != x)
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(scale, row_bytes)))
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(shift, row_bytes)))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int rga_check_gate_add_rms_modulate(const void* x, const void* u,
                                    const void* g, const void* scale,
                                    const void* shift, float eps,
                                    const void* x_out, const void* y,
                                    int64_t B, int64_t L, int64_t D,
                                    int gate_mode)
{
    if (B < 0 || L < 0 || D < 0)
        return RGA_ERR_INVALID_ARG;
    if (gate_mode != RGA_GATE_FULL && gate_mode != RGA_GATE_BCAST)
        return RGA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f)
        return RGA_ERR_INVALID_ARG;
    int64_t n = 0, bytes = 0;
    if (!sizes(B, L, D, &n, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !u || !g || !scale || !shift || !x_out || !y)
        return RGA_ERR_INVALID_ARG;
    if (D % 8 != 0 || D > RGA_RMS_MAX_D)
        return RGA_ERR_UNSUPPORTED;
    const void* all[] = {x, u, g, scale, shift, x_out, y};
    for (const void* p : all)
        if (!aligned16(p))
            return RGA_ERR_UNSUPPORTED;
    if (!rga::gate_add_rms_modulate_grid_fits(B, L, D))
        return RGA_ERR_UNSUPPORTED;

    const bool full = gate_mode == RGA_GATE_FULL;
    const int64_t row_bytes = B * D * 2;
    const Range rows[] = {range_of(scale, row_bytes), range_of(shift, row_bytes)};
    const void* outs[] = {x_out, y};
    for (const void* o : outs) {
        const Range r = range_of(o, bytes);
        if (overlaps(r, range_of(x, bytes)) && o != x)
            return RGA_ERR_ALIAS;
        if (overlaps(r, range_of(u, bytes)) && o != u)
            return RGA_ERR_ALIAS;
        if (overlaps(r, range_of(g, full ? bytes : row_bytes)) && !(full && o == g))
            return RGA_ERR_ALIAS;
        for (const Range& q : rows)
            if (overlaps(r, q))
                return RGA_ERR_ALIAS;
    }
    if (overlaps(range_of(x_out, bytes), range_of(y, bytes)))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int rga_gate_add_rms_modulate(const void* x, const void* u, const void* g,
                              const void* scale, const void* shift, float eps,
                              void* x_out, void* y, int64_t B, int64_t L,
                              int64_t D, int gate_mode, hipStream_t stream)
{
    const int st = rga_check_gate_add_rms_modulate(
        x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return rga::launch_gate_add_rms_modulate(x, u, g, scale, shift, eps,
                                             x_out, y, B, L, D, gate_mode,
                                             stream) == hipSuccess
               ? RGA_OK
               : RGA_ERR_HIP;
}

int rga_residual_gate_add(const void* x, const void* u, const void* g,
                          void* out, int64_t B, int64_t L, int64_t D,
                          int gate_mode, hipStream_t stream)
{
    const int st =
        rga_check_residual_gate_add(x, u, g, out, B, L, D, gate_mode);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return rga::launch_gate_add(x, u, g, out, B, L, D, gate_mode, stream) ==
                   hipSuccess
               ? RGA_OK
               : RGA_ERR_HIP;
}

int rms_modulate(const void* x, const void* scale, const void* shift,
                 float eps, void* out, int64_t B, int64_t L, int64_t D,
                 hipStream_t stream)
{
    const int st = rga_check_rms_modulate(x, scale, shift, eps, out, B, L, D);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return rga::launch_rms_modulate(x, scale, shift, eps, out, B, L, D,
                                    stream) == hipSuccess
               ? RGA_OK
               : RGA_ERR_HIP;
}

// Shared rules of the measurement helpers for one destination range and an
// optional source range (NULL for the fill).
static int check_stream_args(const void* src, bool has_src, const void* dst,
                             int64_t nbytes)
{
    if (nbytes < 0)
        return RGA_ERR_INVALID_ARG;
    if (nbytes == 0)
        return RGA_OK;
    if (dst == nullptr || (has_src && src == nullptr))
        return RGA_ERR_INVALID_ARG;
    if (nbytes % 16 != 0 || !aligned16(dst) || (has_src && !aligned16(src)))
        return RGA_ERR_UNSUPPORTED;
    if (!rga::stream_grid_fits(nbytes / 16))
        return RGA_ERR_UNSUPPORTED;
    if (has_src && overlaps(range_of(src, nbytes), range_of(dst, nbytes)))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int rga_copy(const void* src, void* dst, int64_t nbytes, hipStream_t stream)
{
    const int st = check_stream_args(src, true, dst, nbytes);
    if (st != RGA_OK || nbytes == 0)
        return st;
    return rga::launch_copy(src, dst, nbytes / 16, stream) == hipSuccess
               ? RGA_OK
               : RGA_ERR_HIP;
}

int rga_fill(void* dst, int64_t nbytes, uint32_t value, hipStream_t stream)
{
    const int st = check_stream_args(nullptr, false, dst, nbytes);
    if (st != RGA_OK || nbytes == 0)
        return st;
    return rga::launch_fill(dst, nbytes / 16, value, stream) == hipSuccess
               ? RGA_OK
               : RGA_ERR_HIP;
}

int rga_read(const void* src, int64_t nbytes, void* sink, hipStream_t stream)
{
    int st = check_stream_args(nullptr, false, src, nbytes);
    if (st != RGA_OK || nbytes == 0)
        return st;
    if (sink == nullptr)
        return RGA_ERR_INVALID_ARG;
    if (!aligned16(sink))
        return RGA_ERR_UNSUPPORTED;
    if (overlaps(range_of(src, nbytes), range_of(sink, 16)))
        return RGA_ERR_ALIAS;
    return rga::launch_read(src, nbytes / 16, sink, stream) == hipSuccess
               ? RGA_OK
               : RGA_ERR_HIP;
}

const char* rga_status_string(int status)
{
    switch (status) {
    case RGA_OK:
        return "ok";
    case RGA_ERR_INVALID_ARG:
        return "invalid argument (negative or overflowing size, bad gate "
               "mode or eps, NULL pointer)";
    case RGA_ERR_UNSUPPORTED:
        return "unsupported input (D not a multiple of 8, pointer not "
               "16-byte aligned, D too large, or grid too large)";
    case RGA_ERR_ALIAS:
        return "output overlaps an input other than as an allowed in-place "
               "alias";
    case RGA_ERR_HIP:
        return "HIP runtime error at kernel launch";
    default:
        return "unknown status";
    }
}

}  // extern "C"
