"""MI355X (gfx950) elementwise kernels for video diffusion transformer blocks.

Thin Python binding over the C ABI in ``include/rga.h`` (``librga.so``):
argument marshalling only. Every element of every result is computed by the
library's HIP kernels; torch supplies device memory and the current stream.
There is no CPU path: importing fails loudly when the library is not built.

    rga_residual_gate_add(x, u, g, out=None, gate_mode=None)   out = x + u*g
    rms_modulate(x, scale, shift, eps=1e-6, out=None)
        out = rms_norm(x, eps) * (1 + scale) + shift
    rga_gate_add_rms_modulate(x, u, g, scale, shift, eps=1e-6)
        x_out = x + u*g, then y = rms_norm(x_out, eps) * (1 + scale) + shift

Tensors are contiguous bf16 on one HIP device; x, u, out are [B, L, D]; g is
[B, L, D] (full) or [B, 1, D] (broadcast); scale and shift are [B, 1, D].

The ``_ex`` forms take bf16, float16 or float32 (one type per call), any D,
tensors starting at any element offset, and per-token scale/shift [B, L, D]:

    rga_residual_gate_add_ex(x, u, g, out=None, gate_mode=None)
    rga_rms_modulate_ex(x, scale, shift, eps=1e-6, out=None, mod_mode=None)
    rga_gate_add_rms_modulate_ex(x, u, g, scale, shift, eps=1e-6, x_out=None,
                                 y=None, gate_mode=None, mod_mode=None)

Modulation after a weightless LayerNorm, with the same options as the _ex
forms:

    rga_ln_modulate(x, scale, shift, eps=1e-6, out=None, mod_mode=None)

The FFN's tanh-GELU, any storage type, over the last dimension F:

    gelu_tanh(x, bias=None, out=None)   out = gelu(x + bias)

Measurement helpers (include/rga_measure.h): copy_, fill_, read_ (cache
flush), stream_ (read:write mix ceilings), gate_add_variant (the
broadcast-gate add in the shapes the library does not use),
modulate_occupancy / fused_occupancy (the row-modulation kernels at a chosen
number of workgroups per CU) and modulate_variant / fused_variant (those
kernels in other schedules, SCHED_*).
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F16,
    DTYPE_F32,
    GATE_BCAST,
    GATE_FULL,
    MOD_ROW,
    MOD_TOKEN,
    RGA_ERR_ALIAS,
    RGA_ERR_HIP,
    RGA_ERR_INVALID_ARG,
    RGA_ERR_UNSUPPORTED,
    RGA_OK,
    RGA_RMS_MAX_D,
    SCHED_LIBRARY,
    SCHED_LOADS_FIRST,
    SCHED_ONE_PLUS,
    SCHED_PREFETCH,
    SCHED_TWO_ROWS,
    STORE_DEVICE,
    STORE_NT,
    STORE_PLAIN,
    RGAError,
    check_gate_add_rms_modulate,
    check_gate_add_rms_modulate_ex,
    check_residual_gate_add,
    check_residual_gate_add_ex,
    check_rms_modulate,
    check_fused_occupancy,
    check_fused_variant,
    check_gate_add_variant,
    check_gelu_tanh,
    check_modulate_occupancy,
    check_modulate_variant,
    check_stream,
    check_ln_modulate,
    check_rms_modulate_ex,
    library,
    library_path,
    status_string,
)
from .ops import (  # noqa: F401
    copy_,
    fill_,
    fused_occupancy,
    fused_variant,
    gate_add_variant,
    modulate_occupancy,
    modulate_variant,
    stream_,
    gelu_tanh,
    read_,
    rga_gate_add_rms_modulate,
    rga_gate_add_rms_modulate_ex,
    rga_ln_modulate,
    rga_residual_gate_add,
    rga_residual_gate_add_ex,
    rga_rms_modulate_ex,
    rms_modulate,
)

__all__ = [
    "rga_residual_gate_add",
    "rms_modulate",
    "rga_gate_add_rms_modulate",
    "rga_residual_gate_add_ex",
    "rga_rms_modulate_ex",
    "rga_gate_add_rms_modulate_ex",
    "rga_ln_modulate",
    "gelu_tanh",
    "GATE_FULL",
    "GATE_BCAST",
    "RGAError",
    "library_path",
]
