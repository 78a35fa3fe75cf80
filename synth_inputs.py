"""Seeded synthetic inputs for the gated residual add and the adaLN modulation.

This module serves both the oracle side and the HIP side and therefore holds
none of the method's arithmetic: it draws binary32 samples with numpy's PCG64
and narrows them to bf16 with torch's CPU conversion (a library routine), so
the same host bytes reach the oracle and, by copy, the GPU.

The workloads are the traced shapes of the residual-gate page ("[KDA-Pilot]
Add diffusion residual-gate CUDA fast path for LTX2", B200/H100 kernel
benchmark tables: ltx2_bcast_s32640_c4096, ltx2_full_s8160_c4096,
flux2_bcast_s{512,4096,4608}_c3072, ltx2_full_s126_c2048) and the video and
audio hidden sizes 4096 / 2048 of the RMSNorm+modulate page's unit test. No
page measures on a dataset; these seeded tensors are the whole workload.

Draw order inside one case: x, u, g, scale, shift (those present), each as
``standard_normal(shape) * std`` or ``uniform(-1, 1, shape)`` in binary32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

GATE_FULL = 0
GATE_BCAST = 1

# storage types (the library's and the oracle's numbering)
BF16 = 0
F16 = 1
F32 = 2


@dataclass(frozen=True)
class Dist:
    kind: str  # "normal" or "uniform"
    std: float = 1.0  # standard deviation for "normal"

    def draw(self, rng: np.random.Generator, shape) -> np.ndarray:
        if self.kind == "normal":
            a = rng.standard_normal(shape, dtype=np.float32)
            if self.std != 1.0:
                a *= np.float32(self.std)
            return a
        if self.kind == "uniform":
            return rng.uniform(-1.0, 1.0, shape).astype(np.float32)
        raise ValueError(self.kind)


N01 = Dist("normal", 1.0)
N02 = Dist("normal", 2.0)  # "N(0,2)" read as standard deviation 2
N001 = Dist("normal", 0.1)
U11 = Dist("uniform")


@dataclass(frozen=True)
class Case:
    """One seeded input case. ``gate`` is GATE_FULL / GATE_BCAST / None;
    ``rms`` adds scale/shift rows [B, 1, D] for the modulation."""
    name: str
    B: int
    L: int
    D: int
    seed: int
    gate: int | None
    x: Dist = N01
    u: Dist | None = N01
    g: Dist | None = U11
    rms: bool = False
    scale: Dist = N001
    shift: Dist = N001
    eps: float = 1e-6
    inplace: bool = False
    tags: tuple = field(default=())

    @property
    def elems(self) -> int:
        return self.B * self.L * self.D

    @property
    def rows(self) -> int:
        return self.B * self.L


# The five workload configurations (shapes, distributions, seeds).
CASES = {
    # full gate [1,126,2048] + modulation on the same x (audio hidden 2048)
    "c1": Case("c1_full_s126_c2048", 1, 126, 2048, 101, GATE_FULL, rms=True),
    # broadcast gate [1,L,3072], L in {512, 4096, 4608}
    "c2a": Case("c2_bcast_s512_c3072", 1, 512, 3072, 102, GATE_BCAST),
    "c2b": Case("c2_bcast_s4096_c3072", 1, 4096, 3072, 103, GATE_BCAST),
    "c2c": Case("c2_bcast_s4608_c3072", 1, 4608, 3072, 104, GATE_BCAST),
    # full gate at DiT scale
    "c3": Case("c3_full_s8160_c4096", 1, 8160, 4096, 105, GATE_FULL),
    # broadcast gate at the large video-token count, in place on x
    "c4": Case("c4_bcast_s32640_c4096", 1, 32640, 4096, 106, GATE_BCAST,
               inplace=True),
    # modulation then broadcast gated residual (in place on x), B = 2
    "c5": Case("c5_rmsmod_bcast_b2_s32640_c4096", 2, 32640, 4096, 107,
               GATE_BCAST, x=N02, u=N01, g=N001, rms=True, inplace=True),
}

# Other shapes from the residual-gate page's benchmark table, outside the
# five configurations: parity cases and extra bench lines.
EXTRA_CASES = {
    "ideogram4": Case("ideogram4_bcast_s4096_c4608", 1, 4096, 4608, 108, GATE_BCAST),
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns via torch's CPU conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw_bits(rng, dist: Dist, shape, chunk_rows: int = 2048) -> np.ndarray:
    """Draw in row chunks so a large tensor never holds a full binary32 copy.
    numpy's float32 ziggurat normals and its uniform doubles consume the
    PCG64 stream element by element, so the chunked draw yields the same
    values as one draw of the whole shape (checked by a test)."""
    B, L, D = shape
    rows = B * L
    out = np.empty(rows * D, dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0 * D:r1 * D] = to_bf16_bits(dist.draw(rng, ((r1 - r0) * D,)))
    return out.reshape(shape)


def make_inputs(case: Case) -> dict:
    """Returns {"x", "u", "g", "scale", "shift"} (those the case has) as
    uint16 bf16 bit arrays, drawn in that order from PCG64(seed)."""
    rng = np.random.default_rng(case.seed)
    shape = (case.B, case.L, case.D)
    row = (case.B, 1, case.D)
    out = {"x": _draw_bits(rng, case.x, shape)}
    if case.gate is not None:
        out["u"] = _draw_bits(rng, case.u, shape)
        gshape = shape if case.gate == GATE_FULL else row
        out["g"] = _draw_bits(rng, case.g, gshape)
    if case.rms:
        out["scale"] = _draw_bits(rng, case.scale, row)
        out["shift"] = _draw_bits(rng, case.shift, row)
    return out


def random_bits(seed: int, shape, dist: Dist = N01) -> np.ndarray:
    """Small ad-hoc tensors for edge-case tests."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(dist.draw(rng, shape)).reshape(shape)


def random_typed(seed: int, shape, dist: Dist = N01, dtype: int = BF16) -> np.ndarray:
    """random_bits for any storage type: uint16 bf16 or binary16 patterns,
    or a float32 array. The binary32 draw is the same for every type; the
    2-byte types round it to nearest even (torch for bf16, numpy for f16)."""
    rng = np.random.default_rng(seed)
    a = dist.draw(rng, shape).reshape(shape)
    if dtype == BF16:
        return to_bf16_bits(a).reshape(shape)
    if dtype == F16:
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown storage type {dtype}")
