// C ABI of the library (include/rga.h, include/rga_measure.h): host-side
// validation, then one kernel launch on the caller's stream.
//
// Validation order (the first failing rule decides the status):
//   1. RGA_ERR_INVALID_ARG: a negative dimension, a bad gate_mode, mod_mode
//      or dtype, a non-finite or negative eps, the byte size overflowing
//      int64;
//   2. RGA_OK without a launch when B*L*D == 0 (pointers may be NULL);
//   3. RGA_ERR_INVALID_ARG: a NULL pointer;
//   4. RGA_ERR_UNSUPPORTED: for the original calls D % 8 != 0 or a pointer
//      not 16-byte aligned; for the _ex calls a pointer not aligned to the
//      element size; a grid beyond the dispatch limit;
//   5. RGA_ERR_ALIAS: an output overlapping an input other than the exact
//      in-place aliases each call allows.
// Every call takes the 16-byte-pack kernels when every pointer is 16-byte
// aligned and D % 8 == 0 (any D for a full-gate add, which is one flat
// stream) and, for the modulation, D <= RGA_RMS_MAX_D; the element-wise
// kernels otherwise (for the original calls: modulation rows above
// RGA_RMS_MAX_D, staged in LDS). The fused call with 2-byte rows and row modulation
// always takes its register-row element kernel (the faster one there).
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

int elem_size(int dtype) { return dtype == RGA_DTYPE_F32 ? 4 : 2; }

bool valid_dtype(int dtype)
{
    return dtype == RGA_DTYPE_BF16 || dtype == RGA_DTYPE_F16 ||
           dtype == RGA_DTYPE_F32;
}

bool aligned_to(const void* p, int n)
{
    return (reinterpret_cast<uintptr_t>(p) & (uintptr_t)(n - 1)) == 0;
}

// Layout rule shared by the three operations. strict: the original calls
// (bf16 only, D % 8 == 0 and 16-byte alignment or RGA_ERR_UNSUPPORTED);
// otherwise pointers need only element alignment. *fast tells whether the
// 16-byte-pack kernels can run; max_d > 0 caps their D (the modulation holds
// a row in registers). A row above that cap is not an unsupported input: it
// runs the kernels that stage the row in LDS, in the same summation order.
int layout(const void* const* ptrs, int nptr, int64_t D, int es, bool strict,
           int64_t max_d, bool* fast)
{
    bool all16 = true;
    for (int i = 0; i < nptr; ++i) {
        if (!aligned_to(ptrs[i], es))
            return RGA_ERR_UNSUPPORTED;
        all16 = all16 && aligned16(ptrs[i]);
    }
    if (strict && !(all16 && D % 8 == 0))
        return RGA_ERR_UNSUPPORTED;
    *fast = all16 && D % 8 == 0 && (max_d <= 0 || D <= max_d);
    return RGA_OK;
}

int check_gate_add(const void* x, const void* u, const void* g,
                   const void* out, int64_t B, int64_t L, int64_t D,
                   int gate_mode, int dtype, bool strict, bool* fast)
{
    if (B < 0 || L < 0 || D < 0)
        return RGA_ERR_INVALID_ARG;
    if (gate_mode != RGA_GATE_FULL && gate_mode != RGA_GATE_BCAST)
        return RGA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return RGA_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    int64_t n = 0, bytes = 0;
    if (!sizes(B, L, D, &n, &bytes) || __builtin_mul_overflow(n, (int64_t)es, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !u || !g || !out)
        return RGA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, u, g, out};
    int st = layout(ptrs, 4, D, es, strict, 0, fast);
    if (st != RGA_OK)
        return st;
    // a full gate is one flat stream: the pack kernel takes any D (its last
    // lane adds the trailing B*L*D % 8 elements)
    if (!strict && gate_mode == RGA_GATE_FULL)
        *fast = aligned16(x) && aligned16(u) && aligned16(g) && aligned16(out);
    if (!rga::gate_add_grid_fits(B, L, D, gate_mode, es, *fast))
        return RGA_ERR_UNSUPPORTED;

    const bool full = gate_mode == RGA_GATE_FULL;
    const int64_t gate_bytes = full ? bytes : B * D * es;  // <= bytes
    const Range o = range_of(out, bytes);
    if (overlaps(o, range_of(x, bytes)) && out != x)
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(u, bytes)) && out != u)
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(g, gate_bytes)) && !(full && out == g))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int check_rms(const void* x, const void* scale, const void* shift, float eps,
              const void* out, int64_t B, int64_t L, int64_t D, int mod_mode,
              int dtype, bool strict, bool* fast)
{
    if (B < 0 || L < 0 || D < 0)
        return RGA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f)
        return RGA_ERR_INVALID_ARG;
    if (mod_mode != RGA_MOD_ROW && mod_mode != RGA_MOD_TOKEN)
        return RGA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return RGA_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    int64_t n = 0, bytes = 0;
    if (!sizes(B, L, D, &n, &bytes) || __builtin_mul_overflow(n, (int64_t)es, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !scale || !shift || !out)
        return RGA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, scale, shift, out};
    int st = layout(ptrs, 4, D, es, strict, RGA_RMS_MAX_D, fast);
    if (st != RGA_OK)
        return st;
    if (!rga::rms_modulate_grid_fits(B, L, D, es, *fast))
        return RGA_ERR_UNSUPPORTED;

    const int64_t mod_bytes = mod_mode == RGA_MOD_TOKEN ? bytes : B * D * es;
    const Range o = range_of(out, bytes);
    if (overlaps(o, range_of(x, bytes)) && out != x)
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(scale, mod_bytes)))
        return RGA_ERR_ALIAS;
    if (overlaps(o, range_of(shift, mod_bytes)))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int check_fused(const void* x, const void* u, const void* g,
                const void* scale, const void* shift, float eps,
                const void* x_out, const void* y, int64_t B, int64_t L,
                int64_t D, int gate_mode, int mod_mode, int dtype,
                bool strict, bool* fast)
{
    if (B < 0 || L < 0 || D < 0)
        return RGA_ERR_INVALID_ARG;
    if (gate_mode != RGA_GATE_FULL && gate_mode != RGA_GATE_BCAST)
        return RGA_ERR_INVALID_ARG;
    if (mod_mode != RGA_MOD_ROW && mod_mode != RGA_MOD_TOKEN)
        return RGA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return RGA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f)
        return RGA_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    int64_t n = 0, bytes = 0;
    if (!sizes(B, L, D, &n, &bytes) || __builtin_mul_overflow(n, (int64_t)es, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !u || !g || !scale || !shift || !x_out || !y)
        return RGA_ERR_INVALID_ARG;
    const void* ptrs[] = {x, u, g, scale, shift, x_out, y};
    int st = layout(ptrs, 7, D, es, strict, RGA_RMS_MAX_D, fast);
    if (st != RGA_OK)
        return st;
    if (!rga::gate_add_rms_modulate_grid_fits(B, L, D, es, *fast))
        return RGA_ERR_UNSUPPORTED;

    const bool full = gate_mode == RGA_GATE_FULL;
    const int64_t row_bytes = B * D * es;
    const int64_t mod_bytes = mod_mode == RGA_MOD_TOKEN ? bytes : row_bytes;
    const Range mods[] = {range_of(scale, mod_bytes), range_of(shift, mod_bytes)};
    const void* outs[] = {x_out, y};
    for (const void* o : outs) {
        const Range r = range_of(o, bytes);
        if (overlaps(r, range_of(x, bytes)) && o != x)
            return RGA_ERR_ALIAS;
        if (overlaps(r, range_of(u, bytes)) && o != u)
            return RGA_ERR_ALIAS;
        if (overlaps(r, range_of(g, full ? bytes : row_bytes)) && !(full && o == g))
            return RGA_ERR_ALIAS;
        for (const Range& q : mods)
            if (overlaps(r, q))
                return RGA_ERR_ALIAS;
    }
    if (overlaps(range_of(x_out, bytes), range_of(y, bytes)))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int check_gelu(const void* x, const void* bias, const void* out, int64_t rows,
               int64_t F, int dtype, bool* fast)
{
    if (rows < 0 || F < 0)
        return RGA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype))
        return RGA_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    int64_t n = 0, bytes = 0;
    if (__builtin_mul_overflow(rows, F, &n) || __builtin_mul_overflow(n, (int64_t)es, &bytes))
        return RGA_ERR_INVALID_ARG;
    if (n == 0)
        return RGA_OK;
    if (!x || !out)
        return RGA_ERR_INVALID_ARG;
    if (!aligned_to(x, es) || !aligned_to(out, es) || (bias && !aligned_to(bias, es)))
        return RGA_ERR_UNSUPPORTED;
    *fast = aligned16(x) && aligned16(out) && (!bias || (aligned16(bias) && F % 8 == 0));
    if (!rga::gelu_tanh_grid_fits(rows, F, bias != nullptr, es, *fast))
        return RGA_ERR_UNSUPPORTED;
    const Range o = range_of(out, bytes);
    if (overlaps(o, range_of(x, bytes)) && out != x)
        return RGA_ERR_ALIAS;
    if (bias && overlaps(o, range_of(bias, F * es)))
        return RGA_ERR_ALIAS;
    return RGA_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? RGA_OK : RGA_ERR_HIP; }

}  // namespace

extern "C" {

int rga_check_residual_gate_add(const void* x, const void* u, const void* g,
                                const void* out, int64_t B, int64_t L,
                                int64_t D, int gate_mode)
{
    bool fast = false;
    return check_gate_add(x, u, g, out, B, L, D, gate_mode, RGA_DTYPE_BF16,
                          true, &fast);
}

int rga_check_residual_gate_add_ex(const void* x, const void* u,
                                   const void* g, const void* out, int64_t B,
                                   int64_t L, int64_t D, int gate_mode,
                                   int dtype)
{
    bool fast = false;
    return check_gate_add(x, u, g, out, B, L, D, gate_mode, dtype, false,
                          &fast);
}

int rga_check_rms_modulate(const void* x, const void* scale,
                           const void* shift, float eps, const void* out,
                           int64_t B, int64_t L, int64_t D)
{
    bool fast = false;
    return check_rms(x, scale, shift, eps, out, B, L, D, RGA_MOD_ROW,
                     RGA_DTYPE_BF16, true, &fast);
}

int rga_check_rms_modulate_ex(const void* x, const void* scale,
                              const void* shift, float eps, const void* out,
                              int64_t B, int64_t L, int64_t D, int mod_mode,
                              int dtype)
{
    bool fast = false;
    return check_rms(x, scale, shift, eps, out, B, L, D, mod_mode, dtype,
                     false, &fast);
}

int rga_check_gate_add_rms_modulate(const void* x, const void* u,
                                    const void* g, const void* scale,
                                    const void* shift, float eps,
                                    const void* x_out, const void* y,
                                    int64_t B, int64_t L, int64_t D,
                                    int gate_mode)
{
    bool fast = false;
    return check_fused(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                       gate_mode, RGA_MOD_ROW, RGA_DTYPE_BF16, true, &fast);
}

int rga_check_gate_add_rms_modulate_ex(const void* x, const void* u,
                                       const void* g, const void* scale,
                                       const void* shift, float eps,
                                       const void* x_out, const void* y,
                                       int64_t B, int64_t L, int64_t D,
                                       int gate_mode, int mod_mode, int dtype)
{
    bool fast = false;
    return check_fused(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                       gate_mode, mod_mode, dtype, false, &fast);
}

static int gate_add(const void* x, const void* u, const void* g, void* out,
                    int64_t B, int64_t L, int64_t D, int gate_mode, int dtype,
                    bool strict, hipStream_t stream)
{
    bool fast = false;
    const int st = check_gate_add(x, u, g, out, B, L, D, gate_mode, dtype,
                                  strict, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_gate_add(x, u, g, out, B, L, D, gate_mode,
                                         dtype, fast, stream));
}

int rga_residual_gate_add(const void* x, const void* u, const void* g,
                          void* out, int64_t B, int64_t L, int64_t D,
                          int gate_mode, hipStream_t stream)
{
    return gate_add(x, u, g, out, B, L, D, gate_mode, RGA_DTYPE_BF16, true,
                    stream);
}

int rga_residual_gate_add_ex(const void* x, const void* u, const void* g,
                             void* out, int64_t B, int64_t L, int64_t D,
                             int gate_mode, int dtype, hipStream_t stream)
{
    return gate_add(x, u, g, out, B, L, D, gate_mode, dtype, false, stream);
}

static int rms(const void* x, const void* scale, const void* shift, float eps,
               void* out, int64_t B, int64_t L, int64_t D, int mod_mode,
               int dtype, bool strict, hipStream_t stream)
{
    bool fast = false;
    const int st = check_rms(x, scale, shift, eps, out, B, L, D, mod_mode,
                             dtype, strict, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_rms_modulate(x, scale, shift, eps, out, B, L,
                                             D, mod_mode, dtype, fast,
                                             stream));
}

int rms_modulate(const void* x, const void* scale, const void* shift,
                 float eps, void* out, int64_t B, int64_t L, int64_t D,
                 hipStream_t stream)
{
    return rms(x, scale, shift, eps, out, B, L, D, RGA_MOD_ROW,
               RGA_DTYPE_BF16, true, stream);
}

int rga_rms_modulate_ex(const void* x, const void* scale, const void* shift,
                        float eps, void* out, int64_t B, int64_t L, int64_t D,
                        int mod_mode, int dtype, hipStream_t stream)
{
    return rms(x, scale, shift, eps, out, B, L, D, mod_mode, dtype, false,
               stream);
}

int rga_check_ln_modulate(const void* x, const void* scale, const void* shift,
                          float eps, const void* out, int64_t B, int64_t L,
                          int64_t D, int mod_mode, int dtype)
{
    bool fast = false;
    return check_rms(x, scale, shift, eps, out, B, L, D, mod_mode, dtype, false, &fast);
}

int rga_ln_modulate(const void* x, const void* scale, const void* shift,
                    float eps, void* out, int64_t B, int64_t L, int64_t D,
                    int mod_mode, int dtype, hipStream_t stream)
{
    bool fast = false;
    const int st = check_rms(x, scale, shift, eps, out, B, L, D, mod_mode, dtype, false, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_ln_modulate(x, scale, shift, eps, out, B, L, D, mod_mode,
                                            dtype, fast, stream));
}

static int fused(const void* x, const void* u, const void* g,
                 const void* scale, const void* shift, float eps, void* x_out,
                 void* y, int64_t B, int64_t L, int64_t D, int gate_mode,
                 int mod_mode, int dtype, bool strict, hipStream_t stream)
{
    bool fast = false;
    const int st = check_fused(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                               gate_mode, mod_mode, dtype, strict, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_gate_add_rms_modulate(
        x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, mod_mode,
        dtype, fast, stream));
}

int rga_gate_add_rms_modulate(const void* x, const void* u, const void* g,
                              const void* scale, const void* shift, float eps,
                              void* x_out, void* y, int64_t B, int64_t L,
                              int64_t D, int gate_mode, hipStream_t stream)
{
    return fused(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode,
                 RGA_MOD_ROW, RGA_DTYPE_BF16, true, stream);
}

int rga_gate_add_rms_modulate_ex(const void* x, const void* u, const void* g,
                                 const void* scale, const void* shift,
                                 float eps, void* x_out, void* y, int64_t B,
                                 int64_t L, int64_t D, int gate_mode,
                                 int mod_mode, int dtype, hipStream_t stream)
{
    return fused(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode,
                 mod_mode, dtype, false, stream);
}

int rga_check_gelu_tanh(const void* x, const void* bias, const void* out,
                        int64_t rows, int64_t F, int dtype)
{
    bool fast = false;
    return check_gelu(x, bias, out, rows, F, dtype, &fast);
}

int rga_gelu_tanh(const void* x, const void* bias, void* out, int64_t rows,
                  int64_t F, int dtype, hipStream_t stream)
{
    bool fast = false;
    const int st = check_gelu(x, bias, out, rows, F, dtype, &fast);
    if (st != RGA_OK || rows == 0 || F == 0)
        return st;
    return launched(rga::launch_gelu_tanh(x, bias, out, rows, F, dtype, fast, stream));
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

static int check_stream(const void* const* src, int nsrc, const void* dst, int64_t nbytes,
                        int words_per_lane, const void* sink)
{
    if (nsrc < 0 || nsrc > 3 || nbytes < 0)
        return RGA_ERR_INVALID_ARG;
    if (words_per_lane != 1 && words_per_lane != 2 && words_per_lane != 4)
        return RGA_ERR_INVALID_ARG;
    if (nsrc == 0 && dst == nullptr)
        return RGA_ERR_INVALID_ARG;
    if (nbytes == 0)
        return RGA_OK;
    if (nsrc > 0 && src == nullptr)
        return RGA_ERR_INVALID_ARG;
    for (int k = 0; k < nsrc; ++k)
        if (src[k] == nullptr)
            return RGA_ERR_INVALID_ARG;
    if (dst == nullptr && sink == nullptr)
        return RGA_ERR_INVALID_ARG;
    if (nbytes % 16 != 0 || (dst && !aligned16(dst)) || (!dst && !aligned16(sink)))
        return RGA_ERR_UNSUPPORTED;
    for (int k = 0; k < nsrc; ++k)
        if (!aligned16(src[k]))
            return RGA_ERR_UNSUPPORTED;
    if (!rga::stream_grid_fits(nbytes / 16))
        return RGA_ERR_UNSUPPORTED;
    if (dst) {
        const Range d = range_of(dst, nbytes);
        for (int k = 0; k < nsrc; ++k)
            if (overlaps(d, range_of(src[k], nbytes)) && !(k == 0 && dst == src[0]))
                return RGA_ERR_ALIAS;
    } else {
        const Range s = range_of(sink, 16);
        for (int k = 0; k < nsrc; ++k)
            if (overlaps(s, range_of(src[k], nbytes)))
                return RGA_ERR_ALIAS;
    }
    return RGA_OK;
}

int rga_check_stream(const void* const* src, int nsrc, const void* dst, int64_t nbytes,
                     int words_per_lane, const void* sink)
{
    return check_stream(src, nsrc, dst, nbytes, words_per_lane, sink);
}

int rga_stream(const void* const* src, int nsrc, void* dst, int64_t nbytes,
               int words_per_lane, void* sink, hipStream_t stream)
{
    const int st = check_stream(src, nsrc, dst, nbytes, words_per_lane, sink);
    if (st != RGA_OK || nbytes == 0)
        return st;
    return launched(rga::launch_stream(src, nsrc, dst, nbytes / 16, words_per_lane, sink,
                                       stream));
}

static int check_gate_add_variant(const void* x, const void* u, const void* g,
                                  const void* out, int64_t B, int64_t L, int64_t D,
                                  int rows_per_wave, int store_policy)
{
    if (rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4 && rows_per_wave != 8)
        return RGA_ERR_INVALID_ARG;
    if (store_policy != RGA_STORE_NT && store_policy != RGA_STORE_PLAIN &&
        store_policy != RGA_STORE_DEVICE)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    const int st = check_gate_add(x, u, g, out, B, L, D, RGA_GATE_BCAST, RGA_DTYPE_BF16,
                                  true, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    if (!rga::gate_add_variant_grid_fits(B, L, D, rows_per_wave))
        return RGA_ERR_UNSUPPORTED;
    return RGA_OK;
}

int rga_check_gate_add_variant(const void* x, const void* u, const void* g, const void* out,
                               int64_t B, int64_t L, int64_t D, int rows_per_wave,
                               int store_policy)
{
    return check_gate_add_variant(x, u, g, out, B, L, D, rows_per_wave, store_policy);
}

int rga_gate_add_variant(const void* x, const void* u, const void* g, void* out,
                         int64_t B, int64_t L, int64_t D, int rows_per_wave,
                         int store_policy, hipStream_t stream)
{
    const int st = check_gate_add_variant(x, u, g, out, B, L, D, rows_per_wave, store_policy);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_gate_add_variant(x, u, g, out, B, L, D, rows_per_wave,
                                                 store_policy, stream));
}

int rga_check_modulate_occupancy(const void* x, const void* scale, const void* shift, float eps,
                                 const void* out, int64_t B, int64_t L, int64_t D, int dtype,
                                 int wg_per_cu)
{
    if (wg_per_cu < -1 || wg_per_cu > 16)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    return check_rms(x, scale, shift, eps, out, B, L, D, RGA_MOD_ROW, dtype, false, &fast);
}

int rga_modulate_occupancy(const void* x, const void* scale, const void* shift, float eps,
                           void* out, int64_t B, int64_t L, int64_t D, int dtype, int wg_per_cu,
                           hipStream_t stream)
{
    if (wg_per_cu < -1 || wg_per_cu > 16)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    const int st = check_rms(x, scale, shift, eps, out, B, L, D, RGA_MOD_ROW, dtype, false, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_rms_modulate(x, scale, shift, eps, out, B, L, D, RGA_MOD_ROW,
                                             dtype, fast, stream, wg_per_cu));
}

int rga_check_fused_occupancy(const void* x, const void* u, const void* g, const void* scale,
                              const void* shift, float eps, const void* x_out, const void* y,
                              int64_t B, int64_t L, int64_t D, int gate_mode, int dtype,
                              int wg_per_cu)
{
    if (wg_per_cu < -1 || wg_per_cu > 16)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    return check_fused(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, RGA_MOD_ROW,
                       dtype, false, &fast);
}

int rga_fused_occupancy(const void* x, const void* u, const void* g, const void* scale,
                        const void* shift, float eps, void* x_out, void* y, int64_t B,
                        int64_t L, int64_t D, int gate_mode, int dtype, int wg_per_cu,
                        hipStream_t stream)
{
    if (wg_per_cu < -1 || wg_per_cu > 16)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    const int st = check_fused(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode,
                               RGA_MOD_ROW, dtype, false, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_gate_add_rms_modulate(x, u, g, scale, shift, eps, x_out, y, B,
                                                      L, D, gate_mode, RGA_MOD_ROW, dtype, fast,
                                                      stream, wg_per_cu));
}

static int check_modulate_variant(const void* x, const void* scale, const void* shift,
                                  float eps, const void* out, int64_t B, int64_t L, int64_t D,
                                  int schedule)
{
    if (schedule < 0 || schedule >= rga::kSchedCount)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    const int st = check_rms(x, scale, shift, eps, out, B, L, D, RGA_MOD_ROW, RGA_DTYPE_BF16,
                             true, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return D == rga::kSchedD ? RGA_OK : RGA_ERR_UNSUPPORTED;
}

int rga_check_modulate_variant(const void* x, const void* scale, const void* shift, float eps,
                               const void* out, int64_t B, int64_t L, int64_t D, int schedule)
{
    return check_modulate_variant(x, scale, shift, eps, out, B, L, D, schedule);
}

int rga_modulate_variant(const void* x, const void* scale, const void* shift, float eps,
                         void* out, int64_t B, int64_t L, int64_t D, int schedule,
                         hipStream_t stream)
{
    const int st = check_modulate_variant(x, scale, shift, eps, out, B, L, D, schedule);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_modulate_variant(x, scale, shift, eps, out, B, L, schedule,
                                                 stream));
}

static int check_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                               const void* shift, float eps, const void* x_out, const void* y,
                               int64_t B, int64_t L, int64_t D, int schedule)
{
    if (schedule < 0 || schedule >= rga::kSchedCount)
        return RGA_ERR_INVALID_ARG;
    bool fast = false;
    const int st = check_fused(x, u, g, scale, shift, eps, x_out, y, B, L, D, RGA_GATE_BCAST,
                               RGA_MOD_ROW, RGA_DTYPE_BF16, true, &fast);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return D == rga::kSchedD ? RGA_OK : RGA_ERR_UNSUPPORTED;
}

int rga_check_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                            const void* shift, float eps, const void* x_out, const void* y,
                            int64_t B, int64_t L, int64_t D, int schedule)
{
    return check_fused_variant(x, u, g, scale, shift, eps, x_out, y, B, L, D, schedule);
}

int rga_fused_variant(const void* x, const void* u, const void* g, const void* scale,
                      const void* shift, float eps, void* x_out, void* y, int64_t B, int64_t L,
                      int64_t D, int schedule, hipStream_t stream)
{
    const int st = check_fused_variant(x, u, g, scale, shift, eps, x_out, y, B, L, D, schedule);
    if (st != RGA_OK || B == 0 || L == 0 || D == 0)
        return st;
    return launched(rga::launch_fused_variant(x, u, g, scale, shift, eps, x_out, y, B, L,
                                              schedule, stream));
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
        return "unsupported input (D not a multiple of 8 or pointer not "
               "16-byte aligned for a call without a storage type, pointer "
               "not aligned to the element size, or grid too large)";
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
