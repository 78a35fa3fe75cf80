"""torch integration: custom ops for torch.compile and a first-use check.

Custom ops. The entry points are registered as torch custom ops
(``rga::residual_gate_add``, ``rga::rms_modulate``,
``rga::gate_add_rms_modulate``, their ``_ex`` forms, ``rga::ln_modulate`` and
``rga::gelu_tanh``), functional (they allocate their outputs), each with a
fake implementation that only describes the output shapes. A
``torch.compile(fullgraph=True)`` trace then sees one opaque op instead of
tracing into ctypes ("[KDA-Pilot] Add diffusion residual-gate CUDA fast path
for LTX2", "Modifications": an eager custom op with a fake impl so direct
torch.compile tracing sees an opaque op).

First-use check. ``FirstUseGuard`` wraps a functional call and, the first time
it sees a runtime key (op, shapes, dtype, device, extra arguments), also runs
a reference the caller supplies -- the model's own math -- and compares the
two ("[Kernel] Enable LTX DiffVAE fusions on SM100 and SM103", "Purpose":
each runtime key checked bit for bit on first use). The library has no
second implementation of its own: on a mismatch or a launch error the guard
raises, unless the caller asked for ``fallback=True``, in which case that key
is served by the caller's reference from then on.
"""
from __future__ import annotations

import threading
import warnings
from typing import Callable, Optional

import torch

from . import ops
from ._lib import RGAError

# ---- custom ops ---------------------------------------------------------


@torch.library.custom_op("rga::residual_gate_add", mutates_args=())
def residual_gate_add(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """out = x + u * g; g is [B, L, D] (full) or [B, 1, D] (broadcast)."""
    return ops.rga_residual_gate_add(x, u, g)


@residual_gate_add.register_fake
def _residual_gate_add_fake(x, u, g):
    return torch.empty_like(x)


@torch.library.custom_op("rga::rms_modulate", mutates_args=())
def rms_modulate(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                 eps: float) -> torch.Tensor:
    """out = rms_norm(x, eps) * (1 + scale) + shift (weightless RMSNorm)."""
    return ops.rms_modulate(x, scale, shift, eps)


@rms_modulate.register_fake
def _rms_modulate_fake(x, scale, shift, eps):
    return torch.empty_like(x)


@torch.library.custom_op("rga::gate_add_rms_modulate", mutates_args=())
def gate_add_rms_modulate(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                          scale: torch.Tensor, shift: torch.Tensor,
                          eps: float) -> tuple[torch.Tensor, torch.Tensor]:
    """(x + u * g, rms_norm(x + u * g, eps) * (1 + scale) + shift)."""
    return ops.rga_gate_add_rms_modulate(x, u, g, scale, shift, eps)


@gate_add_rms_modulate.register_fake
def _gate_add_rms_modulate_fake(x, u, g, scale, shift, eps):
    return torch.empty_like(x), torch.empty_like(x)


@torch.library.custom_op("rga::residual_gate_add_ex", mutates_args=())
def residual_gate_add_ex(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """residual_gate_add for bf16, float16 or float32, any D, any offset."""
    return ops.rga_residual_gate_add_ex(x, u, g)


@residual_gate_add_ex.register_fake
def _residual_gate_add_ex_fake(x, u, g):
    return torch.empty_like(x)


@torch.library.custom_op("rga::rms_modulate_ex", mutates_args=())
def rms_modulate_ex(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                    eps: float) -> torch.Tensor:
    """rms_modulate for any storage type; scale/shift [B, 1, D] or [B, L, D]."""
    return ops.rga_rms_modulate_ex(x, scale, shift, eps)


@rms_modulate_ex.register_fake
def _rms_modulate_ex_fake(x, scale, shift, eps):
    return torch.empty_like(x)


@torch.library.custom_op("rga::gate_add_rms_modulate_ex", mutates_args=())
def gate_add_rms_modulate_ex(x: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
                             scale: torch.Tensor, shift: torch.Tensor,
                             eps: float) -> tuple[torch.Tensor, torch.Tensor]:
    """gate_add_rms_modulate for any storage type and modulation layout."""
    return ops.rga_gate_add_rms_modulate_ex(x, u, g, scale, shift, eps)


@gate_add_rms_modulate_ex.register_fake
def _gate_add_rms_modulate_ex_fake(x, u, g, scale, shift, eps):
    return torch.empty_like(x), torch.empty_like(x)


@torch.library.custom_op("rga::ln_modulate", mutates_args=())
def ln_modulate(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                eps: float) -> torch.Tensor:
    """layer_norm(x, eps) * (1 + scale) + shift (weightless LayerNorm)."""
    return ops.rga_ln_modulate(x, scale, shift, eps)


@ln_modulate.register_fake
def _ln_modulate_fake(x, scale, shift, eps):
    return torch.empty_like(x)


@torch.library.custom_op("rga::gelu_tanh", mutates_args=())
def gelu_tanh(x: torch.Tensor, bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gelu(x + bias), tanh approximation, over the last dimension."""
    return ops.gelu_tanh(x, bias)


@gelu_tanh.register_fake
def _gelu_tanh_fake(x, bias=None):
    return torch.empty_like(x)


# ---- first-use check ------------------------------------------------------


def bitwise_equal(a, b) -> bool:
    """True when every output tensor matches bit for bit."""
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    if len(a) != len(b):
        return False
    for p, q in zip(a, b):
        if p.shape != q.shape or p.dtype != q.dtype:
            return False
        if p.element_size() == 2:
            if not torch.equal(p.view(torch.int16), q.view(torch.int16)):
                return False
        elif not torch.equal(p, q):
            return False
    return True


def allclose(atol: float, rtol: float) -> Callable:
    """Tolerance check (e.g. the RMSNorm+modulate page's unit test uses
    atol=3e-2, rtol=1e-2 against eager)."""
    def check(a, b) -> bool:
        a = a if isinstance(a, (tuple, list)) else (a,)
        b = b if isinstance(b, (tuple, list)) else (b,)
        return len(a) == len(b) and all(
            p.shape == q.shape and torch.allclose(p.float(), q.float(), atol=atol, rtol=rtol)
            for p, q in zip(a, b))
    return check


def _default_key(args, kwargs):
    def part(v):
        if isinstance(v, torch.Tensor):
            return ("T", tuple(v.shape), str(v.dtype), str(v.device))
        return ("V", repr(v))
    return tuple(part(a) for a in args) + tuple(sorted((k, part(v)) for k, v in kwargs.items()))


class GuardMismatch(RuntimeError):
    pass


class FirstUseGuard:
    """Checks ``fn`` against the caller's ``reference`` once per runtime key.

    fn, reference : functional callables with the same signature (no
                    in-place outputs: both run on the same inputs)
    check         : (fn_result, reference_result) -> bool; default bit for bit
    fallback      : False (default) raises GuardMismatch / RGAError on the
                    first bad key; True warns and serves that key with
                    ``reference`` from then on
    """

    def __init__(self, fn: Callable, reference: Callable,
                 check: Callable = bitwise_equal, fallback: bool = False,
                 key: Callable = _default_key):
        self.fn = fn
        self.reference = reference
        self.check = check
        self.fallback = fallback
        self.key = key
        self._state: dict = {}
        self._lock = threading.Lock()

    def state(self, *args, **kwargs):
        """None (unseen), True (checked, kernel path) or False (failed)."""
        return self._state.get(self.key(args, kwargs))

    def __call__(self, *args, **kwargs):
        k = self.key(args, kwargs)
        ok = self._state.get(k)
        if ok is True:
            return self.fn(*args, **kwargs)
        if ok is False:
            return self.reference(*args, **kwargs)
        with self._lock:
            return self._first_use(k, args, kwargs)

    def _first_use(self, k, args, kwargs):
        try:
            out = self.fn(*args, **kwargs)
        except RGAError as e:
            if not self.fallback:
                raise
            warnings.warn(f"rga: launch failed for {k}: {e}; using the reference")
            self._state[k] = False
            return self.reference(*args, **kwargs)
        ref = self.reference(*args, **kwargs)
        if self.check(out, ref):
            self._state[k] = True
            return out
        if not self.fallback:
            raise GuardMismatch(f"rga: result differs from the reference for {k}")
        warnings.warn(f"rga: result differs from the reference for {k}; using the reference")
        self._state[k] = False
        return ref
