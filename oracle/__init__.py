"""CPU oracle: the gated residual add and the weightless-RMSNorm modulation,
written as plain binary32 loops with one final bf16 round-to-nearest-even.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package. The product path
never does, and this package never imports the product.

Arrays are numpy ``uint16`` holding bf16 bit patterns, row-major contiguous.
The arithmetic and its sources are documented in ``oracle.c``; this module
only marshals arguments through ctypes.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIBRARY, build_oracle

GATE_FULL = 0
GATE_BCAST = 1

BF16 = 0
F16 = 1
F32 = 2
MOD_ROW = 0
MOD_TOKEN = 1
_NP = {BF16: np.uint16, F16: np.uint16, F32: np.float32}

RMS_PINNED = 0
RMS_SEQUENTIAL = 1
RMS_F64 = 2

_LIB = None


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIBRARY):
        build_oracle()
    lib = ctypes.CDLL(LIBRARY)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_gate_add.argtypes = [p, p, p, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_gate_add.restype = None
    lib.oracle_rms_modulate.argtypes = [
        p, p, p, ctypes.c_float, p, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_rms_modulate.restype = ctypes.c_int
    lib.oracle_rms_norm.argtypes = [
        p, ctypes.c_float, p, i64, i64, i64, ctypes.c_int]
    lib.oracle_rms_norm.restype = ctypes.c_int
    lib.oracle_rms_factors.argtypes = [
        p, p, i64, i64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.oracle_rms_factors.restype = ctypes.c_int
    lib.oracle_bf16_from_f32.argtypes = [p, p, i64]
    lib.oracle_bf16_from_f32.restype = None
    lib.oracle_f32_from_bf16.argtypes = [p, p, i64]
    lib.oracle_f32_from_bf16.restype = None
    lib.oracle_gate_add_rms_modulate.argtypes = [
        p, p, p, p, p, ctypes.c_float, p, p, i64, i64, i64, ctypes.c_int,
        ctypes.c_int]
    lib.oracle_gate_add_rms_modulate.restype = ctypes.c_int
    lib.oracle_gate_add_ex.argtypes = [p, p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_gate_add_ex.restype = ctypes.c_int
    lib.oracle_rms_modulate_ex.argtypes = [
        p, p, p, ctypes.c_float, p, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_rms_modulate_ex.restype = ctypes.c_int
    lib.oracle_gate_add_rms_modulate_ex.argtypes = [
        p, p, p, p, p, ctypes.c_float, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int]
    lib.oracle_gate_add_rms_modulate_ex.restype = ctypes.c_int
    lib.oracle_f16_from_f32.argtypes = [p, p, i64]
    lib.oracle_f16_from_f32.restype = None
    lib.oracle_f32_from_f16.argtypes = [p, p, i64]
    lib.oracle_f32_from_f16.restype = None
    lib.oracle_ln_factors.argtypes = [p, p, p, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                      ctypes.c_int]
    lib.oracle_ln_factors.restype = ctypes.c_int
    lib.oracle_ln_modulate_ex.argtypes = [
        p, p, p, ctypes.c_float, p, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_ln_modulate_ex.restype = ctypes.c_int
    lib.oracle_gelu_tanh_f64.argtypes = [ctypes.c_double]
    lib.oracle_gelu_tanh_f64.restype = ctypes.c_double
    lib.oracle_gelu_tanh.argtypes = [p, p, p, i64, i64, ctypes.c_int]
    lib.oracle_gelu_tanh.restype = ctypes.c_int
    lib.oracle_contraction_probe.argtypes = []
    lib.oracle_contraction_probe.restype = ctypes.c_float
    _LIB = lib
    return lib


def _bits(a, name):
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected uint16 bf16 bit patterns, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name}: must be C-contiguous")
    return a


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def gate_add(x, u, g, gate_mode, out=None):
    """out = bf16_rne(x + u*g) (binary32 mul, then add). x, u: [B, L, D];
    g: [B, L, D] (GATE_FULL) or [B, 1, D] (GATE_BCAST). ``out`` may be ``x``."""
    x, u, g = _bits(x, "x"), _bits(u, "u"), _bits(g, "g")
    if x.ndim != 3 or u.shape != x.shape:
        raise ValueError("x and u must share one [B, L, D] shape")
    B, L, D = x.shape
    want = x.shape if gate_mode == GATE_FULL else (B, 1, D)
    if gate_mode not in (GATE_FULL, GATE_BCAST) or g.shape != want:
        raise ValueError(f"gate shape {g.shape} does not fit mode {gate_mode}")
    if out is None:
        out = np.empty_like(x)
    out = _bits(out, "out")
    if out.shape != x.shape:
        raise ValueError("out must be [B, L, D]")
    _load().oracle_gate_add(_ptr(x), _ptr(u), _ptr(g), _ptr(out), B, L, D,
                            gate_mode)
    return out


def rms_modulate(x, scale, shift, eps, out=None, variant=RMS_PINNED,
                 partials=64):
    """out = bf16_rne(rms_norm(x, eps) * (1 + scale) + shift), scale and shift
    [B, 1, D]. ``variant`` selects the sum of squares: the pinned P-partial
    order (default, P = ``partials``), a sequential binary32 sum, or binary64."""
    x = _bits(x, "x")
    scale, shift = _bits(scale, "scale"), _bits(shift, "shift")
    if x.ndim != 3:
        raise ValueError("x must be [B, L, D]")
    B, L, D = x.shape
    if scale.shape != (B, 1, D) or shift.shape != (B, 1, D):
        raise ValueError("scale and shift must be [B, 1, D]")
    if out is None:
        out = np.empty_like(x)
    out = _bits(out, "out")
    rc = _load().oracle_rms_modulate(_ptr(x), _ptr(scale), _ptr(shift),
                                     float(eps), _ptr(out), B, L, D, variant,
                                     partials)
    if rc:
        raise ValueError("oracle_rms_modulate: D must be a multiple of 8 and "
                         "partials a power of two <= 256")
    return out


def gate_add_rms_modulate(x, u, g, scale, shift, eps, gate_mode, x_out=None,
                          partials=64):
    """x_out = bf16(x + u*g) (as gate_add), then y = rms_modulate(x_out,
    scale, shift, eps). Returns (x_out, y). ``x_out`` may be ``x``."""
    x, u, g = _bits(x, "x"), _bits(u, "u"), _bits(g, "g")
    scale, shift = _bits(scale, "scale"), _bits(shift, "shift")
    B, L, D = x.shape
    if u.shape != x.shape:
        raise ValueError("x and u must share one [B, L, D] shape")
    want = x.shape if gate_mode == GATE_FULL else (B, 1, D)
    if gate_mode not in (GATE_FULL, GATE_BCAST) or g.shape != want:
        raise ValueError(f"gate shape {g.shape} does not fit mode {gate_mode}")
    if scale.shape != (B, 1, D) or shift.shape != (B, 1, D):
        raise ValueError("scale and shift must be [B, 1, D]")
    if x_out is None:
        x_out = np.empty_like(x)
    x_out = _bits(x_out, "x_out")
    y = np.empty_like(x)
    rc = _load().oracle_gate_add_rms_modulate(
        _ptr(x), _ptr(u), _ptr(g), _ptr(scale), _ptr(shift), float(eps),
        _ptr(x_out), _ptr(y), B, L, D, gate_mode, partials)
    if rc:
        raise ValueError("oracle_gate_add_rms_modulate: bad D or partials")
    return x_out, y


def rms_norm(x, eps, partials=64):
    """Weightless RMSNorm: bf16_rne(x * r) with the pinned factor r."""
    x = _bits(x, "x")
    B, L, D = x.shape
    out = np.empty_like(x)
    rc = _load().oracle_rms_norm(_ptr(x), float(eps), _ptr(out), B, L, D,
                                 partials)
    if rc:
        raise ValueError("oracle_rms_norm: bad D or partials")
    return out


def rms_factors(x, eps, variant=RMS_PINNED, partials=64):
    """Per-row binary32 factor r = 1/sqrt(mean(x^2) + eps), shape [B, L]."""
    x = _bits(x, "x")
    B, L, D = x.shape
    f = np.empty((B, L), dtype=np.float32)
    rc = _load().oracle_rms_factors(_ptr(x), _ptr(f), B, L, D, float(eps),
                                    variant, partials)
    if rc:
        raise ValueError("oracle_rms_factors: bad D or partials")
    return f


def bf16_from_f32(a):
    """The oracle's own binary32 -> bf16 round-to-nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_bf16_from_f32(_ptr(a), _ptr(out), a.size)
    return out


def f32_from_bf16(a):
    """The oracle's own bf16 -> binary32 widening."""
    a = _bits(np.ascontiguousarray(a), "a")
    out = np.empty(a.shape, dtype=np.float32)
    _load().oracle_f32_from_bf16(_ptr(a), _ptr(out), a.size)
    return out


def _typed(a, name, dtype):
    a = np.asarray(a)
    if a.dtype != _NP[dtype]:
        raise TypeError(f"{name}: expected {np.dtype(_NP[dtype])} storage for dtype {dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name}: must be C-contiguous")
    return a


def gate_add_ex(x, u, g, gate_mode, dtype, out=None):
    """out = x + u*g for storage dtype BF16/F16 (uint16 patterns) or F32
    (float32 arrays); binary32 arithmetic, one round-to-nearest-even."""
    x, u, g = _typed(x, "x", dtype), _typed(u, "u", dtype), _typed(g, "g", dtype)
    B, L, D = x.shape
    want = x.shape if gate_mode == GATE_FULL else (B, 1, D)
    if u.shape != x.shape or g.shape != want:
        raise ValueError("shape mismatch")
    if out is None:
        out = np.empty_like(x)
    rc = _load().oracle_gate_add_ex(_ptr(x), _ptr(u), _ptr(g), _ptr(out), B, L, D,
                                    gate_mode, dtype)
    if rc:
        raise ValueError("oracle_gate_add_ex: bad dtype")
    return out


def rms_modulate_ex(x, scale, shift, eps, mod_mode, dtype, out=None, partials=64):
    """rms_norm(x, eps) * (1 + scale) + shift for any D, storage dtype and
    modulation layout (MOD_ROW: [B,1,D], MOD_TOKEN: [B,L,D])."""
    x = _typed(x, "x", dtype)
    scale, shift = _typed(scale, "scale", dtype), _typed(shift, "shift", dtype)
    B, L, D = x.shape
    want = (B, 1, D) if mod_mode == MOD_ROW else (B, L, D)
    if scale.shape != want or shift.shape != want:
        raise ValueError("scale/shift shape does not fit the modulation layout")
    if out is None:
        out = np.empty_like(x)
    rc = _load().oracle_rms_modulate_ex(_ptr(x), _ptr(scale), _ptr(shift), float(eps),
                                        _ptr(out), B, L, D, mod_mode, dtype, partials)
    if rc:
        raise ValueError("oracle_rms_modulate_ex: bad dtype or partials")
    return out


def gate_add_rms_modulate_ex(x, u, g, scale, shift, eps, gate_mode, mod_mode, dtype,
                             x_out=None, partials=64):
    """(x + u*g, rms_modulate_ex(x + u*g, ...)) for any storage dtype."""
    x, u, g = _typed(x, "x", dtype), _typed(u, "u", dtype), _typed(g, "g", dtype)
    scale, shift = _typed(scale, "scale", dtype), _typed(shift, "shift", dtype)
    B, L, D = x.shape
    if x_out is None:
        x_out = np.empty_like(x)
    y = np.empty_like(x)
    rc = _load().oracle_gate_add_rms_modulate_ex(
        _ptr(x), _ptr(u), _ptr(g), _ptr(scale), _ptr(shift), float(eps), _ptr(x_out),
        _ptr(y), B, L, D, gate_mode, mod_mode, dtype, partials)
    if rc:
        raise ValueError("oracle_gate_add_rms_modulate_ex: bad dtype or partials")
    return x_out, y


def f16_from_f32(a):
    """The oracle's own binary32 -> binary16 round-to-nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f16_from_f32(_ptr(a), _ptr(out), a.size)
    return out


def f32_from_f16(a):
    """The oracle's own binary16 -> binary32 widening."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    _load().oracle_f32_from_f16(_ptr(a), _ptr(out), a.size)
    return out


def ln_modulate(x, scale, shift, eps, mod_mode, dtype, out=None, partials=64):
    """((x - mean) / sqrt(var + eps)) * (1 + scale) + shift per row (weightless
    LayerNorm, biased variance, both sums in the pinned order)."""
    x = _typed(x, "x", dtype)
    scale, shift = _typed(scale, "scale", dtype), _typed(shift, "shift", dtype)
    B, L, D = x.shape
    want = (B, 1, D) if mod_mode == MOD_ROW else (B, L, D)
    if scale.shape != want or shift.shape != want:
        raise ValueError("scale/shift shape does not fit the modulation layout")
    if out is None:
        out = np.empty_like(x)
    rc = _load().oracle_ln_modulate_ex(_ptr(x), _ptr(scale), _ptr(shift), float(eps),
                                       _ptr(out), B, L, D, mod_mode, dtype, partials)
    if rc:
        raise ValueError("oracle_ln_modulate_ex: bad dtype or partials")
    return out


def ln_factors(x, eps, dtype, partials=64):
    """(mean, 1/sqrt(var + eps)) per row as float32 arrays [B, L]."""
    x = _typed(x, "x", dtype)
    B, L, D = x.shape
    mean = np.empty((B, L), dtype=np.float32)
    rstd = np.empty((B, L), dtype=np.float32)
    rc = _load().oracle_ln_factors(_ptr(x), _ptr(mean), _ptr(rstd), B, L, D, float(eps),
                                   dtype, partials)
    if rc:
        raise ValueError("oracle_ln_factors: bad dtype or partials")
    return mean, rstd


def gelu_tanh_f64(h: float) -> float:
    """The oracle's binary64 tanh-GELU of one value (before any rounding)."""
    return float(_load().oracle_gelu_tanh_f64(float(h)))


def gelu_tanh(x, dtype, bias=None, out=None):
    """gelu(x (+ bias)) over [..., F], rounded once to the storage type."""
    x = _typed(x, "x", dtype)
    F = x.shape[-1] if x.ndim else 1
    rows = x.size // F if F else 0
    if bias is not None:
        bias = _typed(bias, "bias", dtype)
        if bias.shape != (F,):
            raise ValueError("bias must be [F]")
    if out is None:
        out = np.empty_like(x)
    rc = _load().oracle_gelu_tanh(_ptr(x), None if bias is None else _ptr(bias), _ptr(out),
                                  rows, F, dtype)
    if rc:
        raise ValueError("oracle_gelu_tanh: bad dtype")
    return out


def contraction_probe():
    """0.0 when the oracle build does not fuse multiply-add, 2**-24 if it does."""
    return float(_load().oracle_contraction_probe())
