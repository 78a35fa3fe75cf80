"""Seeded random layouts: every call on shapes and element offsets drawn at
random, against the oracle.

The element paths branch on each operand's byte offset inside a 16-byte
word, pick a register slot count from a ladder, and size the LDS-staged
workgroups to the row; hand-picked cases reach only some of those
combinations. Each case here draws a storage type, D (weighted toward the
ladder and wave-count switch points), B, L, an element offset for every
operand and output, and the gate and modulation modes, then checks the gated
add, both modulations, the fused call and the GELU (with and without a bias)
to their usual bars: bit-exact, identical, and within one ULP for the GELU.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, F16, F32, GATE_BCAST, GATE_FULL, N001, N01, N02, U11, random_typed
from tests.gpu_util import say, to_dev_typed, to_host_typed, ulp_diff_typed
from tests.test_gpu_gelu import _check as gelu_check, _values as gelu_values

pytestmark = pytest.mark.gpu

MOD_ROW, MOD_TOKEN = oracle.MOD_ROW, oracle.MOD_TOKEN
NAMES = {BF16: "bf16", F16: "f16", F32: "f32"}
# D near the slot ladder's ends (512 times 1, 2, 4, 6, 8, 9, 12, 16 elements)
# and the LDS wave-count switches (12288 and 24576 bytes of row)
EDGES = [1, 7, 8, 9, 511, 512, 513, 1024, 1025, 2048, 2049, 3072, 3073, 4096, 4097, 4608,
         4609, 6144, 6145, 8192, 8193, 12288, 12289]
CASES = 120


def _draw(rng):
    dtype = [BF16, F16, F32][rng.integers(3)]
    if rng.random() < 0.5:
        D = int(rng.choice(EDGES)) + int(rng.integers(-2, 3))
    else:
        D = int(rng.integers(1, 13000))
    D = max(1, D)
    if dtype == F32:
        D = min(D, 12000)  # rows up to 48 KB: LDS-staged
    B, L = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    offs = [int(v) for v in rng.integers(0, 8, size=10)]
    return dtype, B, L, D, offs


def _empty_at(shape, like, offset):
    n = int(np.prod(shape))
    return torch.empty(n + offset, dtype=like.dtype, device=like.device)[offset:].view(shape)


def _same(got, want, label):
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), label


def _zero_ulp(got, want, dtype, label):
    d = ulp_diff_typed(got, want, dtype)
    assert d.max() == 0, f"{label}: max ULP {int(d.max())}"


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


@pytest.mark.parametrize("case", range(CASES))
def test_random_layout(dte, case):
    rng = np.random.default_rng(9100 + case)
    dtype, B, L, D, o = _draw(rng)
    say(f"[random layout {case}] {NAMES[dtype]} B={B} L={L} D={D} offsets={o}")
    seed = 9200 + 16 * case
    x = random_typed(seed, (B, L, D), N02, dtype)
    u = random_typed(seed + 1, (B, L, D), N01, dtype)
    gb = random_typed(seed + 2, (B, 1, D), U11, dtype)
    gf = random_typed(seed + 3, (B, L, D), U11, dtype)
    s = random_typed(seed + 4, (B, 1, D), N001, dtype)
    t = random_typed(seed + 5, (B, 1, D), N001, dtype)
    ts = random_typed(seed + 6, (B, L, D), N001, dtype)
    tt = random_typed(seed + 7, (B, L, D), N001, dtype)
    bias = random_typed(seed + 8, (D,), N01, dtype)
    dx, du, dgb, dgf, ds, dt, dts, dtt, dbias = (
        to_dev_typed(a, dtype, off) for a, off in zip((x, u, gb, gf, s, t, ts, tt, bias), o[:9]))
    out = _empty_at((B, L, D), dx, o[9])
    yo = _empty_at((B, L, D), dx, (o[9] + 3) % 8)

    dte.rga_residual_gate_add_ex(dx, du, dgb, out=out)
    _same(to_host_typed(out), oracle.gate_add_ex(x, u, gb, GATE_BCAST, dtype), "gate bcast")
    dte.rga_residual_gate_add_ex(dx, du, dgf, out=out, gate_mode=GATE_FULL)
    _same(to_host_typed(out), oracle.gate_add_ex(x, u, gf, GATE_FULL, dtype), "gate full")

    dte.rga_rms_modulate_ex(dx, ds, dt, 1e-6, out=out)
    _zero_ulp(to_host_typed(out), oracle.rms_modulate_ex(x, s, t, 1e-6, MOD_ROW, dtype), dtype,
              "rms row")
    dte.rga_rms_modulate_ex(dx, dts, dtt, 1e-6, out=out, mod_mode=MOD_TOKEN)
    _zero_ulp(to_host_typed(out), oracle.rms_modulate_ex(x, ts, tt, 1e-6, MOD_TOKEN, dtype),
              dtype, "rms token")
    dte.rga_ln_modulate(dx, ds, dt, 1e-6, out=out)
    _zero_ulp(to_host_typed(out), oracle.ln_modulate(x, s, t, 1e-6, MOD_ROW, dtype), dtype,
              "ln row")
    dte.rga_ln_modulate(dx, dts, dtt, 1e-6, out=out, mod_mode=MOD_TOKEN)
    _zero_ulp(to_host_typed(out), oracle.ln_modulate(x, ts, tt, 1e-6, MOD_TOKEN, dtype), dtype,
              "ln token")

    dte.rga_gate_add_rms_modulate_ex(dx, du, dgb, ds, dt, 1e-6, x_out=out, y=yo)
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, gb, s, t, 1e-6, GATE_BCAST, MOD_ROW, dtype)
    _same(to_host_typed(out), wx, "fused bcast x_out")
    _zero_ulp(to_host_typed(yo), wy, dtype, "fused bcast y")
    dte.rga_gate_add_rms_modulate_ex(dx, du, dgf, dts, dtt, 1e-6, x_out=out, y=yo,
                                     gate_mode=GATE_FULL, mod_mode=MOD_TOKEN)
    wx, wy = oracle.gate_add_rms_modulate_ex(x, u, gf, ts, tt, 1e-6, GATE_FULL, MOD_TOKEN, dtype)
    _same(to_host_typed(out), wx, "fused full x_out")
    _zero_ulp(to_host_typed(yo), wy, dtype, "fused full y")

    x2 = x.reshape(B * L, D)
    dte.gelu_tanh(dx.view(B * L, D), out=out.view(B * L, D))
    gelu_check(to_host_typed(out).reshape(B * L, D), oracle.gelu_tanh(x2, dtype),
               gelu_values(x2, dtype), dtype, "gelu")
    dte.gelu_tanh(dx.view(B * L, D), dbias, out=out.view(B * L, D))
    h = (gelu_values(x2, dtype).astype(np.float32)
         + gelu_values(bias, dtype).astype(np.float32)).astype(np.float64)
    gelu_check(to_host_typed(out).reshape(B * L, D), oracle.gelu_tanh(x2, dtype, bias=bias), h,
               dtype, "gelu bias")
