"""Parity of the LayerNorm modulation (rga_ln_modulate) with the oracle.

Bar: within one ULP of the storage type (the bound the modulation page
allows its fused kernel); the library and the oracle fix the same binary32
order for both sums, so the tests also check that the results are identical.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, F16, F32, N001, N02, random_typed
from tests.gpu_util import say, to_dev_typed, to_host_typed, ulp_diff_typed

pytestmark = pytest.mark.gpu
ROW, TOKEN = oracle.MOD_ROW, oracle.MOD_TOKEN
NAMES = {BF16: "bf16", F16: "f16", F32: "f32"}


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def _inputs(seed, B, L, D, mod, dtype):
    shape = (B, L, D) if mod == TOKEN else (B, 1, D)
    return (random_typed(seed, (B, L, D), N02, dtype), random_typed(seed + 1, shape, N001, dtype),
            random_typed(seed + 2, shape, N001, dtype))


def _identical(got, want, dtype, label):
    d = ulp_diff_typed(got, want, dtype)
    hist = np.bincount(np.minimum(d.ravel(), 3), minlength=4)
    say(f"[{label}] ULP histogram 0:{hist[0]} 1:{hist[1]} 2:{hist[2]} >2:{hist[3]}")
    assert d.max() <= 1, f"{label}: max {d.max()} ULP"
    assert d.max() == 0, f"{label}: pinned order, expected identical results"


SHAPES = [(1, 1, 8), (2, 5, 24), (3, 7, 520), (1, 126, 2048), (2, 33, 4096), (1, 9, 8192),
          (1, 3, 1), (2, 5, 7), (3, 7, 13), (2, 9, 1001), (1, 17, 4100), (2, 3, 8200),
          (1, 2, 16384), (1, 19, 4608), (2, 9, 4104), (2, 19, 1009), (1, 7, 3071),
          (2, 5, 4607)]


@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=NAMES.get)
@pytest.mark.parametrize("mod", [ROW, TOKEN])
@pytest.mark.parametrize("B,L,D", SHAPES)
def test_ln_modulate(dte, B, L, D, mod, dtype):
    say(f"[ln] {NAMES[dtype]} B={B} L={L} D={D} mod={mod}")
    x, s, t = _inputs(11000 + 3 * B + L + D, B, L, D, mod, dtype)
    want = oracle.ln_modulate(x, s, t, 1e-6, mod, dtype)
    got = dte.rga_ln_modulate(to_dev_typed(x, dtype), to_dev_typed(s, dtype),
                              to_dev_typed(t, dtype), 1e-6, mod_mode=mod)
    _identical(to_host_typed(got), want, dtype, f"ln {NAMES[dtype]} {B}x{L}x{D} mod={mod}")


@pytest.mark.parametrize("dtype", [BF16, F32], ids=NAMES.get)
def test_offsets_and_in_place(dte, dtype):
    B, L, D = 2, 21, 1000
    say(f"[ln offsets] {NAMES[dtype]}")
    x, s, t = _inputs(11500, B, L, D, ROW, dtype)
    want = oracle.ln_modulate(x, s, t, 1e-6, ROW, dtype)
    dx, ds, dt = (to_dev_typed(a, dtype, offset=1) for a in (x, s, t))
    assert dx.data_ptr() % 16 != 0
    _identical(to_host_typed(dte.rga_ln_modulate(dx, ds, dt, 1e-6)), want, dtype, "offset")
    dx = to_dev_typed(x, dtype)
    dte.rga_ln_modulate(dx, to_dev_typed(s, dtype), to_dev_typed(t, dtype), 1e-6, out=dx)
    _identical(to_host_typed(dx), want, dtype, "in place")


def test_special_rows(dte):
    # constant rows (zero variance: the output is the shift), a row whose
    # mean is exactly 0, large offsets, and NaN / inf rows
    B, L, D = 1, 6, 4096
    x = np.zeros((B, L, D), dtype=np.float32)
    x[0, 0] = 3.0
    x[0, 1] = np.where(np.arange(D) % 2 == 0, 5.0, -5.0)
    x[0, 2] = 1000.0 + np.random.default_rng(1).standard_normal(D)
    x[0, 3, 17] = np.nan
    x[0, 4, 5] = np.inf
    x[0, 5] = np.random.default_rng(2).standard_normal(D) * 1e-20
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    s = random_typed(12, (B, 1, D), N001, BF16)
    t = random_typed(13, (B, 1, D), N001, BF16)
    say("[ln special rows]")
    want = oracle.ln_modulate(xb, s, t, 1e-6, ROW, BF16)
    got = to_host_typed(dte.rga_ln_modulate(to_dev_typed(xb, BF16), to_dev_typed(s, BF16),
                                            to_dev_typed(t, BF16), 1e-6))
    _identical(got, want, BF16, "special rows")


def test_video_scale_sampled_rows(dte):
    # the c5 shape [2, 32640, 4096] bf16 through the kernel, 128 rows checked
    B, L, D = 2, 32640, 4096
    say(f"[ln video] [{B}, {L}, {D}]")
    gen = torch.Generator(device="cuda").manual_seed(41)
    x = (torch.randn(B, L, D, generator=gen, device="cuda") * 2).to(torch.bfloat16)
    s = (torch.randn(B, 1, D, generator=gen, device="cuda") * 0.1).to(torch.bfloat16)
    t = (torch.randn(B, 1, D, generator=gen, device="cuda") * 0.1).to(torch.bfloat16)
    y = dte.rga_ln_modulate(x, s, t, 1e-6)
    rows = np.linspace(0, L - 1, 64).astype(np.int64)
    for b in range(B):
        xs = to_host_typed(x[b:b + 1, rows])
        want = oracle.ln_modulate(xs, to_host_typed(s[b:b + 1]), to_host_typed(t[b:b + 1]),
                                  1e-6, ROW, BF16)
        _identical(to_host_typed(y[b:b + 1, rows]), want, BF16, f"video batch {b}")


@pytest.mark.parametrize("D", [4096, 1003])
def test_eps_zero_degenerate_rows(dte, D):
    # eps = 0: an all-zero row has r = 1/sqrt(0) = inf and 0 * inf = NaN; a
    # constant row (LayerNorm) the same. Both sides take IEEE's answer: NaN
    # outputs match by class, everything else bit for bit. D = 1003 runs the
    # element path, 4096 the pack path.
    B, L = 1, 4
    x = random_typed(13000 + D, (B, L, D), N02, BF16)
    x[0, 0] = 0                                   # zero row
    x[0, 1] = 0x3F80                              # constant 1.0 row
    x[0, 2] = 0x8000                              # -0 row
    s = random_typed(13001, (B, 1, D), N001, BF16)
    t = random_typed(13002, (B, 1, D), N001, BF16)
    say(f"[eps 0] D={D}")
    for name, fn, ref in (
            ("rms", dte.rga_rms_modulate_ex, lambda: oracle.rms_modulate_ex(x, s, t, 0.0, ROW, BF16)),
            ("ln", dte.rga_ln_modulate, lambda: oracle.ln_modulate(x, s, t, 0.0, ROW, BF16))):
        got = to_host_typed(fn(to_dev_typed(x, BF16), to_dev_typed(s, BF16), to_dev_typed(t, BF16),
                               0.0))
        _identical(got, ref(), BF16, f"eps 0 {name} D={D}")
