/*
 * rga.h — C ABI of the MI355X (gfx950) elementwise library for video
 * diffusion transformer blocks: the gated residual add, the adaLN modulation
 * after a weightless RMSNorm or LayerNorm over contiguous [B, L, D], and the
 * tanh-GELU of the FFN.
 *
 * Conventions shared by every call below:
 *   - Tensor pointers are DEVICE pointers (HIP device memory of the current
 *     device) to row-major contiguous values of the call's storage type,
 *     passed as void*: bf16 (bfloat16: sign, 8 exponent bits, 7 fraction
 *     bits, the upper half of a binary32) for the calls without a dtype
 *     argument, RGA_DTYPE_* for the others (one type for every tensor of a
 *     call). Row (b, l) of a [B, L, D] tensor starts at element (b*L + l)*D;
 *     the broadcast row of batch b of a [B, 1, D] tensor starts at b*D.
 *   - Ownership: the caller allocates and owns every buffer. The library
 *     allocates nothing, keeps no pointer after a call returns and holds no
 *     state between calls. Calls are asynchronous: they validate on the host,
 *     enqueue one kernel on `stream` (0 is the null stream) and return without
 *     synchronising; buffers must stay alive until that work completes.
 *     Calls may be made from several host threads at once.
 *   - Arithmetic: IEEE binary32 with round-to-nearest-even, no fused
 *     multiply-add, subnormals kept, then one rounding to the storage type
 *     (round-to-nearest-even; a NaN stays a NaN, its payload unspecified).
 *   - Errors: every call returns an RGA_* status and never throws or aborts.
 *     Validation runs before anything is enqueued; on any non-zero status
 *     nothing was enqueued except for RGA_ERR_HIP, which reports the HIP
 *     error of the launch itself. There is no fallback path inside the
 *     library: a caller that wants one decides on a non-zero status.
 *   - Sizes: every dimension >= 0; an empty tensor is a valid no-op (RGA_OK,
 *     nothing enqueued, pointers may then be NULL). The bf16 calls without a
 *     dtype argument need D % 8 == 0 and 16-byte aligned pointers (one
 *     128-bit access moves 8 elements), else RGA_ERR_UNSUPPORTED; the calls
 *     with a dtype argument take any D and pointers aligned to the element
 *     size, and run element-wise kernels where the 128-bit ones cannot.
 *   - Memory touched: every kernel reads and writes with aligned 128-bit
 *     accesses. For a tensor that does not start or end on a 16-byte
 *     boundary, the element-wise kernels also READ the bytes of the first
 *     and last 16-byte words that lie outside the tensor (those words hold
 *     at least one of its elements, so they sit in pages the caller owns);
 *     they never WRITE a byte outside an output tensor (partial words are
 *     written element by element). Concurrent writers of those neighbouring
 *     bytes are therefore safe.
 */
#ifndef RGA_H
#define RGA_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Gate layouts of rga_residual_gate_add. */
enum {
    RGA_GATE_FULL = 0,  /* g is [B, L, D] */
    RGA_GATE_BCAST = 1, /* g is [B, 1, D]: row b is used for every l */
};

/* Status codes. */
enum {
    RGA_OK = 0,
    RGA_ERR_INVALID_ARG = 1, /* negative dim, size overflow, bad gate_mode,
                                bad eps, NULL pointer with B*L*D > 0 */
    RGA_ERR_UNSUPPORTED = 2, /* D % 8 != 0 or a pointer not 16-byte aligned
                                (calls without a dtype), a pointer not
                                aligned to the element size (_ex calls),
                                grid too large */
    RGA_ERR_ALIAS = 3,       /* out overlaps an input other than as allowed */
    RGA_ERR_HIP = 4,         /* the HIP runtime rejected the launch */
};

/* Largest D whose modulation rows the 16-byte-pack kernels hold in
 * registers. Longer rows are not rejected: rms_modulate,
 * rga_gate_add_rms_modulate and the _ex calls run them with kernels that
 * stage each row in LDS (or, past 64 KB per row, read it twice), in the same
 * summation order, so the results do not depend on which kernel ran. */
#define RGA_RMS_MAX_D 8192

/* Storage types of the _ex calls (all tensors of a call share one type).
 * Arithmetic is binary32 for every type; one round-to-nearest-even to the
 * storage type at the end (none for binary32). */
enum {
    RGA_DTYPE_BF16 = 0,
    RGA_DTYPE_F16 = 1, /* IEEE binary16 */
    RGA_DTYPE_F32 = 2, /* IEEE binary32 */
};

/* Layouts of scale and shift in the _ex modulation calls. */
enum {
    RGA_MOD_ROW = 0,   /* [B, 1, D]: row b used for every l */
    RGA_MOD_TOKEN = 1, /* [B, L, D]: one row per token */
};

/*
 * Gated residual add: out = x + u * g.
 *
 * Source: "[KDA-Pilot] Add diffusion residual-gate CUDA fast path for LTX2"
 * (sglang PR #29361), section "Motivation": hidden_states plus update times
 * gate over contiguous [B, L, D] tensors, with a full gate or a gate
 * broadcast over L as [B, 1, D].
 *
 * Per element: p = u * g (binary32), s = x + p (binary32), out = bf16(s).
 *   x, u, out : [B, L, D]
 *   g         : [B, L, D] if gate_mode == RGA_GATE_FULL,
 *               [B, 1, D] if gate_mode == RGA_GATE_BCAST
 * Aliasing: out == x and out == u are allowed (in place), and out == g in
 * full mode; any other overlap of out with an input is RGA_ERR_ALIAS.
 * Inputs may overlap one another freely.
 */
int rga_residual_gate_add(const void* x, const void* u, const void* g,
                          void* out, int64_t B, int64_t L, int64_t D,
                          int gate_mode, hipStream_t stream);

/*
 * adaLN modulation with a weightless RMSNorm:
 *   out = rms_norm(x, eps) * (1 + scale) + shift.
 *
 * Source: prhub summary of sglang PR #34172 ("LTX-2 quality=high fused
 * RMSNorm+modulate"), sections "功能与动机" and "关键源码片段": the
 * per-block adaLN expression with RMSNormNoWeight, eps 1e-6 in its test.
 *
 *   x, out        : [B, L, D]
 *   scale, shift  : [B, 1, D]; row b is used for every l
 *   eps           : finite, >= 0 (else RGA_ERR_INVALID_ARG)
 *   D             : multiple of 8 (rows above RGA_RMS_MAX_D are staged in
 *                   LDS; same result)
 * Per row (b, l): ss = sum of x_d^2, r = 1 / sqrt(ss / D + eps); per element
 * y = ((x_d * r) * (1 + scale_d)) + shift_d, each step binary32, then bf16.
 * The sum of squares has one fixed order: the row is cut into groups of 8
 * consecutive elements, group k is accumulated (in element order, square
 * then add) into partial k mod 64 in increasing k, and the 64 partials are
 * combined pairwise by index distance 1, 2, 4, ..., 32 (partial j takes
 * partial j xor m). Results are therefore reproducible bit for bit.
 * Aliasing: out == x is allowed (in place); any other overlap of out with
 * an input is RGA_ERR_ALIAS.
 */
int rms_modulate(const void* x, const void* scale, const void* shift,
                 float eps, void* out, int64_t B, int64_t L, int64_t D,
                 hipStream_t stream);

/*
 * Residual update followed by the next modulation, in one pass:
 *   x_out = x + u * g                                 (as rga_residual_gate_add)
 *   y     = rms_norm(x_out, eps) * (1 + scale) + shift (as rms_modulate)
 *
 * Source: the two steps are adjacent in a DiT block — the residual-gate update
 * of hidden_states ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path
 * for LTX2", "Motivation") and the adaLN modulation of the updated
 * hidden_states before the next sub-layer (prhub summary of sglang PR #34172,
 * "关键源码片段", LTX2TransformerBlock.forward). Fused, x_out is never read
 * back: 8 bytes per element instead of 10.
 *
 *   x, u, x_out, y : [B, L, D]
 *   g              : [B, L, D] (RGA_GATE_FULL) or [B, 1, D] (RGA_GATE_BCAST)
 *   scale, shift   : [B, 1, D]
 *   eps            : finite, >= 0;  D: multiple of 8 (any size)
 * Results are bit-identical to rga_residual_gate_add(x, u, g, x_out) followed
 * by rms_modulate(x_out, scale, shift, eps, y): the modulation reads the
 * bf16-rounded x_out, with the same fixed reduction order.
 * Aliasing: x_out and y may each be exactly x or u (or g in full mode); they
 * must not overlap each other, scale, shift or a broadcast g (RGA_ERR_ALIAS).
 */
int rga_gate_add_rms_modulate(const void* x, const void* u, const void* g,
                              const void* scale, const void* shift, float eps,
                              void* x_out, void* y, int64_t B, int64_t L,
                              int64_t D, int gate_mode, hipStream_t stream);

/*
 * Extended forms: any storage type (RGA_DTYPE_*), any D >= 0, pointers aligned
 * to the element size (2 or 4 bytes; else RGA_ERR_UNSUPPORTED), per-token
 * modulation (RGA_MOD_TOKEN). Source: the residual-gate page
 * ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path for LTX2",
 * "Modifications") lists a correctness test over several storage types and
 * ragged tail shapes.
 * Same operations, aliasing rules and status codes as the calls above; with
 * RGA_DTYPE_BF16, RGA_MOD_ROW, D % 8 == 0, D <= RGA_RMS_MAX_D and 16-byte
 * aligned pointers they run the same kernels and give the same results.
 * Otherwise element-wise kernels with the same arithmetic and the same
 * summation order run (the last group of 8 may be shorter). For per-token
 * modulation scale and shift are [B, L, D] and must not overlap the outputs.
 */
int rga_residual_gate_add_ex(const void* x, const void* u, const void* g,
                             void* out, int64_t B, int64_t L, int64_t D,
                             int gate_mode, int dtype, hipStream_t stream);
int rga_rms_modulate_ex(const void* x, const void* scale, const void* shift,
                        float eps, void* out, int64_t B, int64_t L, int64_t D,
                        int mod_mode, int dtype, hipStream_t stream);
int rga_gate_add_rms_modulate_ex(const void* x, const void* u, const void* g,
                                 const void* scale, const void* shift,
                                 float eps, void* x_out, void* y, int64_t B,
                                 int64_t L, int64_t D, int gate_mode,
                                 int mod_mode, int dtype, hipStream_t stream);

/*
 * adaLN modulation with a weightless LayerNorm:
 *   out = ((x - mean) / sqrt(var + eps)) * (1 + scale) + shift.
 *
 * Source: prhub summary of sglang PR #34172, "实现拆解" items 2 and 4: an
 * LN+modulate fusion family (fused_ln_modulate) sits beside the
 * RMSNorm+modulate one; the pages do not describe it, and the library takes
 * the adaLN form of a DiT block with a LayerNorm without affine weight:
 * mean = sum(x) / D, var = sum((x - mean)^2) / D (biased; the deviations from
 * the binary32 mean).
 *
 * Same arguments, layouts, storage types, aliasing rules, status codes and
 * kernels' launch shapes as rga_rms_modulate_ex. Both sums use the fixed
 * order of the RMS sum of squares (groups of 8, partial k mod 64, pairwise by
 * index distance 1..32); then r = 1 / sqrt(var + eps) and each element
 * becomes (((x - mean) * r) * (1 + scale)) + shift, every step binary32, one
 * rounding to storage. Results are reproducible bit for bit.
 */
int rga_ln_modulate(const void* x, const void* scale, const void* shift,
                    float eps, void* out, int64_t B, int64_t L, int64_t D,
                    int mod_mode, int dtype, hipStream_t stream);

/*
 * tanh-GELU over the FFN intermediate: out = gelu(x + bias), bias optional.
 *
 * Source: prhub summary of sglang PR #34172, "关键源码片段"
 * (LTX2FeedForward.forward: the output of proj_in goes through a
 * tanh-approximated GELU, there folded into the GEMM's epilogue) and "实现拆解"
 * item 1 (the GELU is one of the element-wise chains torch.compile fuses).
 * The pages name the function without printing it; the library takes the
 * standard tanh approximation
 *   gelu(h) = 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))).
 *
 *   x, out : [rows, F] (any leading shape flattened into rows), storage dtype
 *   bias   : [F] or NULL; when given, h = x + bias in binary32 first
 *   dtype  : RGA_DTYPE_*; pointers aligned to the element size
 * Arithmetic: binary32 through the identity 0.5 (1 + tanh(a)) = 1 / (1 +
 * e^-2a) with e^-|2a| (no overflow, no cancellation), then one
 * round-to-nearest-even to storage. The result is within one ULP of the
 * correctly rounded value for bf16 and binary16 storage; for binary32
 * storage the relative error is at most (8 + 6|2a|) 2^-24 (plus 2^-146
 * absolute for results near the subnormal range). +inf -> +inf, -inf -> -0,
 * NaN -> NaN.
 * Aliasing: out == x is allowed (in place); out must not overlap bias.
 * Fast path: every pointer 16-byte aligned and (with a bias) F % 8 == 0.
 */
int rga_gelu_tanh(const void* x, const void* bias, void* out, int64_t rows,
                  int64_t F, int dtype, hipStream_t stream);

/*
 * Host-only validation of the arguments of the calls above, with the same
 * rules and the same status the call would return before launching.
 * Touches neither the device nor the pointed-to memory.
 */
int rga_check_residual_gate_add(const void* x, const void* u, const void* g,
                                const void* out, int64_t B, int64_t L,
                                int64_t D, int gate_mode);
int rga_check_rms_modulate(const void* x, const void* scale,
                           const void* shift, float eps, const void* out,
                           int64_t B, int64_t L, int64_t D);
int rga_check_gate_add_rms_modulate(const void* x, const void* u,
                                    const void* g, const void* scale,
                                    const void* shift, float eps,
                                    const void* x_out, const void* y,
                                    int64_t B, int64_t L, int64_t D,
                                    int gate_mode);
int rga_check_residual_gate_add_ex(const void* x, const void* u,
                                   const void* g, const void* out, int64_t B,
                                   int64_t L, int64_t D, int gate_mode,
                                   int dtype);
int rga_check_rms_modulate_ex(const void* x, const void* scale,
                              const void* shift, float eps, const void* out,
                              int64_t B, int64_t L, int64_t D, int mod_mode,
                              int dtype);
int rga_check_gate_add_rms_modulate_ex(const void* x, const void* u,
                                       const void* g, const void* scale,
                                       const void* shift, float eps,
                                       const void* x_out, const void* y,
                                       int64_t B, int64_t L, int64_t D,
                                       int gate_mode, int mod_mode,
                                       int dtype);

int rga_check_ln_modulate(const void* x, const void* scale, const void* shift,
                          float eps, const void* out, int64_t B, int64_t L,
                          int64_t D, int mod_mode, int dtype);
int rga_check_gelu_tanh(const void* x, const void* bias, const void* out,
                        int64_t rows, int64_t F, int dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* rga_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RGA_H */
