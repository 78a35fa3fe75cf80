"""Tensor-level entry points: check dtype, device, contiguity and shapes,
then pass raw device addresses and the current HIP stream to the C ABI."""
from __future__ import annotations

import torch

from ._lib import (DTYPE_BF16, DTYPE_F16, DTYPE_F32, GATE_BCAST, GATE_FULL, MOD_ROW,
                   MOD_TOKEN, RGA_OK, SCHED_LIBRARY, STORE_NT, RGAError, library,
                   pointer_array)


# torch's raw accessor of the current stream (what its own compiled kernels
# use) costs ~0.1 us against ~2 us for building a torch.cuda.Stream object;
# builds without it take the public API
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device) -> int:
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


# storage types of the _ex calls
_DTYPES = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}


def _require(t: torch.Tensor, name: str, device=None, dtype=torch.bfloat16) -> None:
    # dtype by identity and device by index: building torch.device objects
    # for every check was a measurable part of a small call's host time
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype is not dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _x_shape(x: torch.Tensor, dtype) -> tuple:
    _require(x, "x", dtype=dtype)
    if x.dim() != 3:
        raise ValueError("x must be [B, L, D]")
    return tuple(x.shape)


def _storage(x) -> torch.dtype:
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.dtype not in _DTYPES:
        raise TypeError(f"x must be bfloat16, float16 or float32, got {x.dtype}")
    return x.dtype


def _gate(x, u, g, gate_mode, dtype, dev) -> int:
    B, L, D = x.shape
    _require(u, "u", dev, dtype)
    _require(g, "g", dev, dtype)
    if u.shape != x.shape:
        raise ValueError(f"u has shape {tuple(u.shape)}, expected {tuple(x.shape)}")
    if gate_mode is None:
        gate_mode = GATE_FULL if g.shape == x.shape else GATE_BCAST
    want = (B, L, D) if gate_mode == GATE_FULL else (B, 1, D)
    if gate_mode in (GATE_FULL, GATE_BCAST) and tuple(g.shape) != want:
        raise ValueError(f"g has shape {tuple(g.shape)}, expected {want}")
    return int(gate_mode)


def _modulation(x, scale, shift, mod_mode, dtype, dev) -> int:
    B, L, D = x.shape
    if mod_mode is None:
        mod_mode = MOD_TOKEN if (L != 1 and tuple(scale.shape) == (B, L, D)) else MOD_ROW
    want = (B, L, D) if mod_mode == MOD_TOKEN else (B, 1, D)
    for name, t in (("scale", scale), ("shift", shift)):
        _require(t, name, dev, dtype)
        if mod_mode in (MOD_ROW, MOD_TOKEN) and tuple(t.shape) != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")
    return int(mod_mode)


def _output(t, name, x, dev):
    if t is None:
        return torch.empty_like(x)
    _require(t, name, dev, x.dtype)
    if t.shape != x.shape:
        raise ValueError(f"{name} must have x's shape")
    return t


def rga_residual_gate_add(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                          out: torch.Tensor | None = None,
                          gate_mode: int | None = None) -> torch.Tensor:
    """out = x + u * g (binary32 multiply and add, one bf16 rounding).

    x, u: [B, L, D]; g: [B, L, D] (GATE_FULL) or [B, 1, D] (GATE_BCAST);
    gate_mode is inferred from g's shape when None. ``out`` may be x or u
    (in place), or g in full mode. Enqueued on the current stream."""
    B, L, D = _x_shape(x, torch.bfloat16)
    dev = x.device
    gate_mode = _gate(x, u, g, gate_mode, torch.bfloat16, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_residual_gate_add(
        x.data_ptr(), u.data_ptr(), g.data_ptr(), out.data_ptr(), B, L, D,
        gate_mode, _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_residual_gate_add")
    return out


def rga_residual_gate_add_ex(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                             out: torch.Tensor | None = None,
                             gate_mode: int | None = None) -> torch.Tensor:
    """rga_residual_gate_add for bf16, float16 or float32 tensors (all of one
    type), any D, and tensors that start at any element offset."""
    dt = _storage(x)
    B, L, D = _x_shape(x, dt)
    dev = x.device
    gate_mode = _gate(x, u, g, gate_mode, dt, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_residual_gate_add_ex(
        x.data_ptr(), u.data_ptr(), g.data_ptr(), out.data_ptr(), B, L, D,
        gate_mode, _DTYPES[dt], _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_residual_gate_add_ex")
    return out


def rms_modulate(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                 eps: float = 1e-6,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """out = rms_norm(x, eps) * (1 + scale) + shift with a weightless RMSNorm.

    x: [B, L, D]; scale, shift: [B, 1, D]; ``out`` may be x (in place).
    eps is passed as binary32. Enqueued on the current stream."""
    B, L, D = _x_shape(x, torch.bfloat16)
    dev = x.device
    _modulation(x, scale, shift, MOD_ROW, torch.bfloat16, dev)
    out = _output(out, "out", x, dev)
    st = library().rms_modulate(
        x.data_ptr(), scale.data_ptr(), shift.data_ptr(), float(eps),
        out.data_ptr(), B, L, D, _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rms_modulate")
    return out


def rga_rms_modulate_ex(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                        eps: float = 1e-6, out: torch.Tensor | None = None,
                        mod_mode: int | None = None) -> torch.Tensor:
    """rms_modulate for bf16, float16 or float32, any D, any element offset,
    and scale/shift per token ([B, L, D], MOD_TOKEN) or per batch row
    ([B, 1, D], MOD_ROW); mod_mode is inferred from scale's shape when None."""
    dt = _storage(x)
    B, L, D = _x_shape(x, dt)
    dev = x.device
    mod_mode = _modulation(x, scale, shift, mod_mode, dt, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_rms_modulate_ex(
        x.data_ptr(), scale.data_ptr(), shift.data_ptr(), float(eps),
        out.data_ptr(), B, L, D, mod_mode, _DTYPES[dt], _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_rms_modulate_ex")
    return out


def rga_ln_modulate(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                    eps: float = 1e-6, out: torch.Tensor | None = None,
                    mod_mode: int | None = None) -> torch.Tensor:
    """out = layer_norm(x, eps) * (1 + scale) + shift with a weightless
    LayerNorm (biased variance); bf16, float16 or float32, any D, scale/shift
    per batch row [B, 1, D] or per token [B, L, D]. ``out`` may be x."""
    dt = _storage(x)
    B, L, D = _x_shape(x, dt)
    dev = x.device
    mod_mode = _modulation(x, scale, shift, mod_mode, dt, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_ln_modulate(
        x.data_ptr(), scale.data_ptr(), shift.data_ptr(), float(eps),
        out.data_ptr(), B, L, D, mod_mode, _DTYPES[dt], _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_ln_modulate")
    return out


def rga_gate_add_rms_modulate(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                              scale: torch.Tensor, shift: torch.Tensor,
                              eps: float = 1e-6,
                              x_out: torch.Tensor | None = None,
                              y: torch.Tensor | None = None,
                              gate_mode: int | None = None):
    """x_out = x + u * g, then y = rms_norm(x_out, eps) * (1 + scale) + shift,
    in one pass. Returns (x_out, y). x_out and y may each be x or u."""
    B, L, D = _x_shape(x, torch.bfloat16)
    dev = x.device
    gate_mode = _gate(x, u, g, gate_mode, torch.bfloat16, dev)
    _modulation(x, scale, shift, MOD_ROW, torch.bfloat16, dev)
    x_out = _output(x_out, "x_out", x, dev)
    y = _output(y, "y", x, dev)
    st = library().rga_gate_add_rms_modulate(
        x.data_ptr(), u.data_ptr(), g.data_ptr(), scale.data_ptr(),
        shift.data_ptr(), float(eps), x_out.data_ptr(), y.data_ptr(), B, L, D,
        gate_mode, _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_gate_add_rms_modulate")
    return x_out, y


def rga_gate_add_rms_modulate_ex(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                                 scale: torch.Tensor, shift: torch.Tensor,
                                 eps: float = 1e-6,
                                 x_out: torch.Tensor | None = None,
                                 y: torch.Tensor | None = None,
                                 gate_mode: int | None = None,
                                 mod_mode: int | None = None):
    """rga_gate_add_rms_modulate for bf16, float16 or float32, any D, any
    element offset, and per-token or per-batch-row scale/shift."""
    dt = _storage(x)
    B, L, D = _x_shape(x, dt)
    dev = x.device
    gate_mode = _gate(x, u, g, gate_mode, dt, dev)
    mod_mode = _modulation(x, scale, shift, mod_mode, dt, dev)
    x_out = _output(x_out, "x_out", x, dev)
    y = _output(y, "y", x, dev)
    st = library().rga_gate_add_rms_modulate_ex(
        x.data_ptr(), u.data_ptr(), g.data_ptr(), scale.data_ptr(),
        shift.data_ptr(), float(eps), x_out.data_ptr(), y.data_ptr(), B, L, D,
        gate_mode, mod_mode, _DTYPES[dt], _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_gate_add_rms_modulate_ex")
    return x_out, y


def gelu_tanh(x: torch.Tensor, bias: torch.Tensor | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """out = gelu(x + bias) with the tanh approximation of GELU, over the last
    dimension F of x (any leading shape); bias is an optional [F] row of the
    same storage type (bf16, float16 or float32). ``out`` may be x."""
    dt = _storage(x)
    _require(x, "x", dtype=dt)
    if x.dim() < 1:
        raise ValueError("x needs at least one dimension")
    F = x.shape[-1]
    rows = x.numel() // F if F else 0
    dev = x.device
    if bias is not None:
        _require(bias, "bias", dev, dt)
        if tuple(bias.shape) != (F,):
            raise ValueError(f"bias has shape {tuple(bias.shape)}, expected {(F,)}")
    out = _output(out, "out", x, dev)
    st = library().rga_gelu_tanh(
        x.data_ptr(), None if bias is None else bias.data_ptr(), out.data_ptr(),
        rows, F, _DTYPES[dt], _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_gelu_tanh")
    return out


def copy_(dst: torch.Tensor, src: torch.Tensor) -> torch.Tensor:
    """Measurement helper: 128-bit device copy of src's bytes into dst."""
    if src.device.type != "cuda" or dst.device != src.device:
        raise ValueError("copy_ needs two tensors on one HIP device")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("copy_ needs contiguous tensors")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("copy_ needs equal byte sizes")
    st = library().rga_copy(src.data_ptr(), dst.data_ptr(), n,
                            _stream_handle(src.device))
    if st != RGA_OK:
        raise RGAError(st, "rga_copy")
    return dst


def fill_(dst: torch.Tensor, value: int = 0) -> torch.Tensor:
    """Measurement helper: writes every 32-bit word of dst with ``value``."""
    if dst.device.type != "cuda" or not dst.is_contiguous():
        raise ValueError("fill_ needs a contiguous tensor on a HIP device")
    st = library().rga_fill(dst.data_ptr(), dst.numel() * dst.element_size(),
                            int(value) & 0xFFFFFFFF, _stream_handle(dst.device))
    if st != RGA_OK:
        raise RGAError(st, "rga_fill")
    return dst


def read_(src: torch.Tensor, sink: torch.Tensor) -> torch.Tensor:
    """Measurement helper: reads all of src with cache-allocating loads and
    XORs its 16-byte words into sink (a 16-byte device tensor)."""
    if src.device.type != "cuda" or sink.device != src.device:
        raise ValueError("read_ needs two tensors on one HIP device")
    if not (src.is_contiguous() and sink.is_contiguous()):
        raise ValueError("read_ needs contiguous tensors")
    if sink.numel() * sink.element_size() < 16:
        raise ValueError("read_ needs a sink of at least 16 bytes")
    st = library().rga_read(src.data_ptr(), src.numel() * src.element_size(),
                            sink.data_ptr(), _stream_handle(src.device))
    if st != RGA_OK:
        raise RGAError(st, "rga_read")
    return sink


def stream_(srcs, dst: torch.Tensor | None = None, words_per_lane: int = 1,
            sink: torch.Tensor | None = None) -> None:
    """Measurement helper (rga_stream): reads every source tensor in full and,
    with ``dst``, writes dst = XOR of the sources (a read:write mix with no
    arithmetic). Sources and dst have one byte size; dst may be srcs[0] (in
    place). Without dst the stream is read-only and ``sink`` (16 bytes) is
    required."""
    srcs = list(srcs)
    ref = dst if dst is not None else srcs[0]
    n = ref.numel() * ref.element_size()
    for t in srcs + ([dst] if dst is not None else []) + ([sink] if sink is not None else []):
        if t.device.type != "cuda" or t.device != ref.device or not t.is_contiguous():
            raise ValueError("stream_ needs contiguous tensors on one HIP device")
    for t in srcs:
        if t.numel() * t.element_size() != n:
            raise ValueError("stream_ needs sources of the destination's byte size")
    st = library().rga_stream(pointer_array([t.data_ptr() for t in srcs]) if srcs else None,
                              len(srcs), dst.data_ptr() if dst is not None else None, n,
                              int(words_per_lane),
                              sink.data_ptr() if sink is not None else None,
                              _stream_handle(ref.device))
    if st != RGA_OK:
        raise RGAError(st, "rga_stream")


def gate_add_variant(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                     out: torch.Tensor | None = None, rows_per_wave: int = 1,
                     store_policy: int = STORE_NT) -> torch.Tensor:
    """Measurement helper (rga_gate_add_variant): the bf16 broadcast-gate add
    of rga_residual_gate_add in another kernel shape (rows per wave with the
    gate held, store cache policy); same result bit for bit."""
    B, L, D = _x_shape(x, torch.bfloat16)
    dev = x.device
    _gate(x, u, g, GATE_BCAST, torch.bfloat16, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_gate_add_variant(x.data_ptr(), u.data_ptr(), g.data_ptr(),
                                        out.data_ptr(), B, L, D, int(rows_per_wave),
                                        int(store_policy), _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_gate_add_variant")
    return out


def modulate_occupancy(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                       eps: float = 1e-6, out: torch.Tensor | None = None,
                       wg_per_cu: int = 0) -> torch.Tensor:
    """Measurement helper (rga_modulate_occupancy): rga_rms_modulate_ex with
    row modulation and a chosen number of workgroups per CU for the kernels
    that stage scale and shift in LDS (-1: no cap, 0: the library's rule)."""
    dt = _storage(x)
    B, L, D = _x_shape(x, dt)
    dev = x.device
    _modulation(x, scale, shift, MOD_ROW, dt, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_modulate_occupancy(x.data_ptr(), scale.data_ptr(), shift.data_ptr(),
                                          float(eps), out.data_ptr(), B, L, D, _DTYPES[dt],
                                          int(wg_per_cu), _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_modulate_occupancy")
    return out


def fused_occupancy(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor, scale: torch.Tensor,
                    shift: torch.Tensor, eps: float = 1e-6, x_out: torch.Tensor | None = None,
                    y: torch.Tensor | None = None, gate_mode: int | None = None,
                    wg_per_cu: int = 0):
    """Measurement helper (rga_fused_occupancy): rga_gate_add_rms_modulate_ex
    with row modulation and a chosen number of workgroups per CU."""
    dt = _storage(x)
    B, L, D = _x_shape(x, dt)
    dev = x.device
    gate_mode = _gate(x, u, g, gate_mode, dt, dev)
    _modulation(x, scale, shift, MOD_ROW, dt, dev)
    x_out = _output(x_out, "x_out", x, dev)
    y = _output(y, "y", x, dev)
    st = library().rga_fused_occupancy(x.data_ptr(), u.data_ptr(), g.data_ptr(),
                                       scale.data_ptr(), shift.data_ptr(), float(eps),
                                       x_out.data_ptr(), y.data_ptr(), B, L, D, gate_mode,
                                       _DTYPES[dt], int(wg_per_cu), _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_fused_occupancy")
    return x_out, y


def modulate_variant(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                     eps: float = 1e-6, out: torch.Tensor | None = None,
                     schedule: int = SCHED_LIBRARY) -> torch.Tensor:
    """Measurement helper (rga_modulate_variant): the bf16 rms_modulate of
    4096-element rows in a chosen schedule of the staged kernel (SCHED_*);
    same result bit for bit."""
    B, L, D = _x_shape(x, torch.bfloat16)
    dev = x.device
    _modulation(x, scale, shift, MOD_ROW, torch.bfloat16, dev)
    out = _output(out, "out", x, dev)
    st = library().rga_modulate_variant(x.data_ptr(), scale.data_ptr(), shift.data_ptr(),
                                        float(eps), out.data_ptr(), B, L, D, int(schedule),
                                        _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_modulate_variant")
    return out


def fused_variant(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor, scale: torch.Tensor,
                  shift: torch.Tensor, eps: float = 1e-6, x_out: torch.Tensor | None = None,
                  y: torch.Tensor | None = None, schedule: int = SCHED_LIBRARY):
    """Measurement helper (rga_fused_variant): the bf16 broadcast-gate
    rga_gate_add_rms_modulate of 4096-element rows in a chosen schedule of
    the staged kernel (SCHED_*); same results bit for bit."""
    B, L, D = _x_shape(x, torch.bfloat16)
    dev = x.device
    _gate(x, u, g, GATE_BCAST, torch.bfloat16, dev)
    _modulation(x, scale, shift, MOD_ROW, torch.bfloat16, dev)
    x_out = _output(x_out, "x_out", x, dev)
    y = _output(y, "y", x, dev)
    st = library().rga_fused_variant(x.data_ptr(), u.data_ptr(), g.data_ptr(),
                                     scale.data_ptr(), shift.data_ptr(), float(eps),
                                     x_out.data_ptr(), y.data_ptr(), B, L, D, int(schedule),
                                     _stream_handle(dev))
    if st != RGA_OK:
        raise RGAError(st, "rga_fused_variant")
    return x_out, y
