"""Tensor-level entry points: check dtype, device, contiguity and shapes,
then pass raw device addresses and the current HIP stream to the C ABI."""
from __future__ import annotations

import torch

from ._lib import GATE_BCAST, GATE_FULL, RGA_OK, RGAError, library


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def rga_residual_gate_add(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                          out: torch.Tensor | None = None,
                          gate_mode: int | None = None) -> torch.Tensor:
    """out = x + u * g (binary32 multiply and add, one bf16 rounding).

    x, u: [B, L, D]; g: [B, L, D] (GATE_FULL) or [B, 1, D] (GATE_BCAST);
    gate_mode is inferred from g's shape when None. ``out`` may be x or u
    (in place), or g in full mode. Enqueued on the current stream."""
    _require(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, L, D]")
    B, L, D = x.shape
    _require(u, "u", x.device)
    _require(g, "g", x.device)
    if u.shape != x.shape:
        raise ValueError(f"u has shape {tuple(u.shape)}, expected {tuple(x.shape)}")
    if gate_mode is None:
        gate_mode = GATE_FULL if g.shape == x.shape else GATE_BCAST
    want = (B, L, D) if gate_mode == GATE_FULL else (B, 1, D)
    if gate_mode in (GATE_FULL, GATE_BCAST) and tuple(g.shape) != want:
        raise ValueError(f"g has shape {tuple(g.shape)}, expected {want}")
    if out is None:
        out = torch.empty_like(x)
    else:
        _require(out, "out", x.device)
        if out.shape != x.shape:
            raise ValueError("out must have x's shape")
    st = library().rga_residual_gate_add(
        x.data_ptr(), u.data_ptr(), g.data_ptr(), out.data_ptr(), B, L, D,
        int(gate_mode), _stream_handle(x.device))
    if st != RGA_OK:
        raise RGAError(st, "rga_residual_gate_add")
    return out


def rms_modulate(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                 eps: float = 1e-6,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """out = rms_norm(x, eps) * (1 + scale) + shift with a weightless RMSNorm.

    x: [B, L, D]; scale, shift: [B, 1, D]; ``out`` may be x (in place).
    eps is passed as binary32. Enqueued on the current stream."""
    _require(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, L, D]")
    B, L, D = x.shape
    for name, t in (("scale", scale), ("shift", shift)):
        _require(t, name, x.device)
        if tuple(t.shape) != (B, 1, D):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, 1, D)}")
    if out is None:
        out = torch.empty_like(x)
    else:
        _require(out, "out", x.device)
        if out.shape != x.shape:
            raise ValueError("out must have x's shape")
    st = library().rms_modulate(
        x.data_ptr(), scale.data_ptr(), shift.data_ptr(), float(eps),
        out.data_ptr(), B, L, D, _stream_handle(x.device))
    if st != RGA_OK:
        raise RGAError(st, "rms_modulate")
    return out


def rga_gate_add_rms_modulate(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                              scale: torch.Tensor, shift: torch.Tensor,
                              eps: float = 1e-6,
                              x_out: torch.Tensor | None = None,
                              y: torch.Tensor | None = None,
                              gate_mode: int | None = None):
    """x_out = x + u * g, then y = rms_norm(x_out, eps) * (1 + scale) + shift,
    in one pass. Returns (x_out, y). x_out and y may each be x or u."""
    _require(x, "x")
    if x.dim() != 3:
        raise ValueError("x must be [B, L, D]")
    B, L, D = x.shape
    _require(u, "u", x.device)
    _require(g, "g", x.device)
    if u.shape != x.shape:
        raise ValueError(f"u has shape {tuple(u.shape)}, expected {tuple(x.shape)}")
    if gate_mode is None:
        gate_mode = GATE_FULL if g.shape == x.shape else GATE_BCAST
    want = (B, L, D) if gate_mode == GATE_FULL else (B, 1, D)
    if gate_mode in (GATE_FULL, GATE_BCAST) and tuple(g.shape) != want:
        raise ValueError(f"g has shape {tuple(g.shape)}, expected {want}")
    for name, t in (("scale", scale), ("shift", shift)):
        _require(t, name, x.device)
        if tuple(t.shape) != (B, 1, D):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, 1, D)}")
    if x_out is None:
        x_out = torch.empty_like(x)
    if y is None:
        y = torch.empty_like(x)
    for name, t in (("x_out", x_out), ("y", y)):
        _require(t, name, x.device)
        if t.shape != x.shape:
            raise ValueError(f"{name} must have x's shape")
    st = library().rga_gate_add_rms_modulate(
        x.data_ptr(), u.data_ptr(), g.data_ptr(), scale.data_ptr(),
        shift.data_ptr(), float(eps), x_out.data_ptr(), y.data_ptr(), B, L, D,
        int(gate_mode), _stream_handle(x.device))
    if st != RGA_OK:
        raise RGAError(st, "rga_gate_add_rms_modulate")
    return x_out, y


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
