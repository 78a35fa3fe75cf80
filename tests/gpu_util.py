"""Helpers for the GPU parity tests: host <-> device transfer of bf16 bit
patterns and the bf16 ULP metric. No arithmetic of the method lives here."""
import numpy as np
import torch

from tests.exact_round import is_nan, is_nan_typed, ulp_diff, ulp_diff_typed  # noqa: F401


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize(t.device)
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bitwise equal except that any NaN matches any NaN."""
    na, nb = is_nan(a), is_nan(b)
    return bool(np.array_equal(na, nb) and np.all((a == b) | na))


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    bad = np.nonzero(~((a == b) | (is_nan(a) & is_nan(b))))
    if not len(bad[0]):
        return "none"
    i = tuple(int(v[0]) for v in bad)
    return f"{len(bad[0])} mismatches, first at {i}: got {a[i]:#06x} want {b[i]:#06x}"


def say(msg: str) -> None:
    print(msg, flush=True)


_TORCH = {0: torch.bfloat16, 1: torch.float16, 2: torch.float32}


def to_dev_typed(a: np.ndarray, dtype: int, offset: int = 0) -> torch.Tensor:
    """Host array (uint16 patterns for bf16/f16, float32 for f32) -> device
    tensor of that storage type. offset > 0 places the tensor that many
    elements into a larger allocation, so its address is only element
    aligned."""
    a = np.ascontiguousarray(a)
    if dtype == 2:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    else:
        t = torch.from_numpy(a.astype(np.uint16, copy=False).view(np.int16)).view(_TORCH[dtype])
    if offset == 0:
        return t.to(dev())
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=dev())
    view = flat[offset:].view(t.shape)
    view.copy_(t.to(dev()))
    return view


def to_host_typed(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize(t.device)
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def same_bits_typed(a: np.ndarray, b: np.ndarray, dtype: int) -> bool:
    """Bitwise equal except that any NaN matches any NaN."""
    na, nb = is_nan_typed(a, dtype), is_nan_typed(b, dtype)
    ab = a.view(np.uint32) if dtype == 2 else a
    bb = b.view(np.uint32) if dtype == 2 else b
    return bool(np.array_equal(na, nb) and np.all((ab == bb) | na))


def first_mismatch_typed(a: np.ndarray, b: np.ndarray, dtype: int) -> str:
    ab = a.view(np.uint32) if dtype == 2 else a
    bb = b.view(np.uint32) if dtype == 2 else b
    bad = np.nonzero(~((ab == bb) | (is_nan_typed(a, dtype) & is_nan_typed(b, dtype))))
    if not len(bad[0]):
        return "none"
    i = tuple(int(v[0]) for v in bad)
    return f"{len(bad[0])} mismatches, first at {i}: got {int(ab[i]):#x} want {int(bb[i]):#x}"
