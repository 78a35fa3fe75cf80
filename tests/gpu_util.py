"""Helpers for the GPU parity tests: host <-> device transfer of bf16 bit
patterns and the bf16 ULP metric. No arithmetic of the method lives here."""
import numpy as np
import torch

from tests.exact_round import is_nan, ulp_diff  # noqa: F401


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
