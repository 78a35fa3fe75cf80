"""ctypes declarations of the C ABI (include/rga.h, include/rga_measure.h).

Loading happens at import: a missing or unloadable ``librga.so`` raises
ImportError, so nothing can run without the HIP library.

torch is imported first on purpose. The ROCm build of torch ships its own
HIP runtime (SONAME libamdhip64.so.7); once it is loaded, the dynamic linker
resolves librga.so's dependency on that SONAME to the same copy, so the
library launches on torch's streams and sees torch's allocations. Loaded the
other way round, the process would hold two HIP runtimes and torch's stream
handles would be foreign to the library.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL below)

_HERE = os.path.dirname(os.path.abspath(__file__))
_PATH = os.path.join(_HERE, "librga.so")

GATE_FULL = 0
GATE_BCAST = 1

DTYPE_BF16 = 0
DTYPE_F16 = 1
DTYPE_F32 = 2

MOD_ROW = 0
MOD_TOKEN = 1

RGA_OK = 0
RGA_ERR_INVALID_ARG = 1
RGA_ERR_UNSUPPORTED = 2
RGA_ERR_ALIAS = 3
RGA_ERR_HIP = 4

RGA_RMS_MAX_D = 8192

STORE_NT = 0
STORE_PLAIN = 1
STORE_DEVICE = 2

SCHED_LIBRARY = 0
SCHED_LOADS_FIRST = 1
SCHED_ONE_PLUS = 2
SCHED_TWO_ROWS = 3
SCHED_PREFETCH = 4


class RGAError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: status {status}: {status_string(status)}")


def library_path() -> str:
    return _PATH


def _load():
    if not os.path.exists(_PATH):
        raise ImportError(
            f"{_PATH} is not built; run __graft_entry__.build() "
            "(hipcc for gfx950). There is no CPU fallback.")
    try:
        lib = ctypes.CDLL(_PATH)
    except OSError as e:
        raise ImportError(f"cannot load {_PATH}: {e}") from e
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f32, u32 = ctypes.c_float, ctypes.c_uint32
    lib.rga_residual_gate_add.argtypes = [p, p, p, p, i64, i64, i64, i32, p]
    lib.rga_residual_gate_add.restype = i32
    lib.rms_modulate.argtypes = [p, p, p, f32, p, i64, i64, i64, p]
    lib.rms_modulate.restype = i32
    lib.rga_check_residual_gate_add.argtypes = [p, p, p, p, i64, i64, i64, i32]
    lib.rga_check_residual_gate_add.restype = i32
    lib.rga_check_rms_modulate.argtypes = [p, p, p, f32, p, i64, i64, i64]
    lib.rga_check_rms_modulate.restype = i32
    lib.rga_gate_add_rms_modulate.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64, i32, p]
    lib.rga_gate_add_rms_modulate.restype = i32
    lib.rga_check_gate_add_rms_modulate.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64, i32]
    lib.rga_check_gate_add_rms_modulate.restype = i32
    lib.rga_residual_gate_add_ex.argtypes = [p, p, p, p, i64, i64, i64, i32, i32, p]
    lib.rga_residual_gate_add_ex.restype = i32
    lib.rga_rms_modulate_ex.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, i32, p]
    lib.rga_rms_modulate_ex.restype = i32
    lib.rga_gate_add_rms_modulate_ex.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64,
                                                 i32, i32, i32, p]
    lib.rga_gate_add_rms_modulate_ex.restype = i32
    lib.rga_check_residual_gate_add_ex.argtypes = [p, p, p, p, i64, i64, i64, i32, i32]
    lib.rga_check_residual_gate_add_ex.restype = i32
    lib.rga_check_rms_modulate_ex.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, i32]
    lib.rga_check_rms_modulate_ex.restype = i32
    lib.rga_check_gate_add_rms_modulate_ex.argtypes = [p, p, p, p, p, f32, p, p, i64, i64,
                                                       i64, i32, i32, i32]
    lib.rga_check_gate_add_rms_modulate_ex.restype = i32
    lib.rga_ln_modulate.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, i32, p]
    lib.rga_ln_modulate.restype = i32
    lib.rga_check_ln_modulate.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, i32]
    lib.rga_check_ln_modulate.restype = i32
    lib.rga_gelu_tanh.argtypes = [p, p, p, i64, i64, i32, p]
    lib.rga_gelu_tanh.restype = i32
    lib.rga_check_gelu_tanh.argtypes = [p, p, p, i64, i64, i32]
    lib.rga_check_gelu_tanh.restype = i32
    lib.rga_status_string.argtypes = [i32]
    lib.rga_status_string.restype = ctypes.c_char_p
    lib.rga_copy.argtypes = [p, p, i64, p]
    lib.rga_copy.restype = i32
    lib.rga_fill.argtypes = [p, i64, u32, p]
    lib.rga_fill.restype = i32
    lib.rga_read.argtypes = [p, i64, p, p]
    lib.rga_read.restype = i32
    pp = ctypes.POINTER(p)
    lib.rga_stream.argtypes = [pp, i32, p, i64, i32, p, p]
    lib.rga_stream.restype = i32
    lib.rga_check_stream.argtypes = [pp, i32, p, i64, i32, p]
    lib.rga_check_stream.restype = i32
    lib.rga_gate_add_variant.argtypes = [p, p, p, p, i64, i64, i64, i32, i32, p]
    lib.rga_gate_add_variant.restype = i32
    lib.rga_check_gate_add_variant.argtypes = [p, p, p, p, i64, i64, i64, i32, i32]
    lib.rga_check_gate_add_variant.restype = i32
    lib.rga_modulate_occupancy.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, i32, p]
    lib.rga_modulate_occupancy.restype = i32
    lib.rga_check_modulate_occupancy.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, i32]
    lib.rga_check_modulate_occupancy.restype = i32
    lib.rga_fused_occupancy.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64, i32, i32, i32, p]
    lib.rga_fused_occupancy.restype = i32
    lib.rga_check_fused_occupancy.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64, i32, i32,
                                              i32]
    lib.rga_check_fused_occupancy.restype = i32
    lib.rga_modulate_variant.argtypes = [p, p, p, f32, p, i64, i64, i64, i32, p]
    lib.rga_modulate_variant.restype = i32
    lib.rga_check_modulate_variant.argtypes = [p, p, p, f32, p, i64, i64, i64, i32]
    lib.rga_check_modulate_variant.restype = i32
    lib.rga_fused_variant.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64, i32, p]
    lib.rga_fused_variant.restype = i32
    lib.rga_check_fused_variant.argtypes = [p, p, p, p, p, f32, p, p, i64, i64, i64, i32]
    lib.rga_check_fused_variant.restype = i32
    return lib


_LIB = _load()


def library():
    return _LIB


def status_string(status: int) -> str:
    return _LIB.rga_status_string(int(status)).decode()


def check_residual_gate_add(x, u, g, out, B, L, D, gate_mode) -> int:
    """Host-only validation through the C ABI (addresses as integers)."""
    return _LIB.rga_check_residual_gate_add(x, u, g, out, B, L, D, gate_mode)


def check_rms_modulate(x, scale, shift, eps, out, B, L, D) -> int:
    return _LIB.rga_check_rms_modulate(x, scale, shift, eps, out, B, L, D)


def check_gate_add_rms_modulate(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                                gate_mode) -> int:
    return _LIB.rga_check_gate_add_rms_modulate(x, u, g, scale, shift, eps,
                                                x_out, y, B, L, D, gate_mode)


def check_residual_gate_add_ex(x, u, g, out, B, L, D, gate_mode, dtype) -> int:
    return _LIB.rga_check_residual_gate_add_ex(x, u, g, out, B, L, D, gate_mode, dtype)


def check_rms_modulate_ex(x, scale, shift, eps, out, B, L, D, mod_mode, dtype) -> int:
    return _LIB.rga_check_rms_modulate_ex(x, scale, shift, eps, out, B, L, D,
                                          mod_mode, dtype)


def check_gate_add_rms_modulate_ex(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                                   gate_mode, mod_mode, dtype) -> int:
    return _LIB.rga_check_gate_add_rms_modulate_ex(x, u, g, scale, shift, eps, x_out,
                                                   y, B, L, D, gate_mode, mod_mode,
                                                   dtype)


def check_gelu_tanh(x, bias, out, rows, F, dtype) -> int:
    return _LIB.rga_check_gelu_tanh(x, bias, out, rows, F, dtype)


def check_ln_modulate(x, scale, shift, eps, out, B, L, D, mod_mode, dtype) -> int:
    return _LIB.rga_check_ln_modulate(x, scale, shift, eps, out, B, L, D, mod_mode, dtype)


def pointer_array(ptrs):
    """A C array of device addresses (for rga_stream's source list)."""
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, a in enumerate(ptrs):
        arr[i] = a
    return arr


def check_stream(srcs, dst, nbytes, words_per_lane, sink) -> int:
    return _LIB.rga_check_stream(pointer_array(srcs) if srcs else None, len(srcs), dst,
                                 nbytes, words_per_lane, sink)


def check_gate_add_variant(x, u, g, out, B, L, D, rows_per_wave, store_policy) -> int:
    return _LIB.rga_check_gate_add_variant(x, u, g, out, B, L, D, rows_per_wave,
                                           store_policy)


def check_modulate_occupancy(x, scale, shift, eps, out, B, L, D, dtype, wg_per_cu) -> int:
    return _LIB.rga_check_modulate_occupancy(x, scale, shift, eps, out, B, L, D, dtype,
                                             wg_per_cu)


def check_fused_occupancy(x, u, g, scale, shift, eps, x_out, y, B, L, D, gate_mode, dtype,
                          wg_per_cu) -> int:
    return _LIB.rga_check_fused_occupancy(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                                          gate_mode, dtype, wg_per_cu)


def check_modulate_variant(x, scale, shift, eps, out, B, L, D, schedule) -> int:
    return _LIB.rga_check_modulate_variant(x, scale, shift, eps, out, B, L, D, schedule)


def check_fused_variant(x, u, g, scale, shift, eps, x_out, y, B, L, D, schedule) -> int:
    return _LIB.rga_check_fused_variant(x, u, g, scale, shift, eps, x_out, y, B, L, D,
                                        schedule)
