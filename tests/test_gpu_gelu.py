"""Parity of the tanh-GELU kernels (rga_gelu_tanh) with the oracle.

Bar: for bf16 and binary16 storage, within one ULP of the oracle's correctly
rounded value (the kernel's binary32 evaluation has a relative error of a few
times 2^-24 (1 + |t|), t = 2 sqrt(2/pi) (h + 0.044715 h^3), so only values
within that distance of a rounding boundary can land on the neighbour); NaN
for NaN. For binary32 storage, |y - y_oracle| <= (8 + 6|t|) 2^-24 |y_oracle|
+ (2 + |h|) 2^-149, the same error budget without the final rounding to a
narrower format. Inputs stand in for an FFN intermediate: normal draws with
standard deviation 2, plus every 2-byte bit pattern.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, F16, F32, N01, N02, random_typed
from tests.gpu_util import say, to_dev_typed, to_host_typed, ulp_diff_typed

pytestmark = pytest.mark.gpu
NAMES = {BF16: "bf16", F16: "f16", F32: "f32"}


@pytest.fixture(scope="module")
def dte():
    import diffusion_transformer_elementwise_amd as m
    return m


def _values(a, dtype):
    if dtype == F32:
        return a.astype(np.float64)
    if dtype == F16:
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check(got, want, h, dtype, label):
    """h: the binary32 inputs of the GELU (after any bias add), as float64."""
    if dtype == F32:
        t = np.abs(2 * np.sqrt(2 / np.pi) * (h + 0.044715 * h ** 3))
        g, w = got.astype(np.float64), want.astype(np.float64)
        both_nan = np.isnan(g) & np.isnan(w)
        with np.errstate(invalid="ignore", over="ignore"):
            bound = (8 + 6 * t) * 2.0 ** -24 * np.abs(w) + (2 + np.abs(h)) * 2.0 ** -149
            ok = both_nan | (g == w) | (np.abs(g - w) <= bound)
        bad = np.flatnonzero(~ok)
        say(f"[{label}] binary32: {int((g != w).sum() - both_nan.sum())} inexact of {g.size}, "
            f"{bad.size} outside the bound")
        assert bad.size == 0, [(float(h.ravel()[i]), float(g.ravel()[i]), float(w.ravel()[i]))
                               for i in bad[:5]]
        return
    d = ulp_diff_typed(got, want, dtype)
    hist = np.bincount(np.minimum(d.ravel(), 3), minlength=4)
    say(f"[{label}] ULP histogram 0:{hist[0]} 1:{hist[1]} 2:{hist[2]} >2:{hist[3]}")
    assert d.max() <= 1, f"{label}: max {d.max()} ULP"


@pytest.mark.parametrize("dtype", [BF16, F16], ids=NAMES.get)
def test_every_2_byte_pattern(dte, dtype):
    x = np.arange(1 << 16, dtype=np.uint16).reshape(256, 256)
    say(f"[gelu patterns] {NAMES[dtype]}")
    want = oracle.gelu_tanh(x, dtype)
    got = to_host_typed(dte.gelu_tanh(to_dev_typed(x, dtype)))
    _check(got, want, _values(x, dtype), dtype, f"patterns {NAMES[dtype]}")


def test_binary32_spread_patterns(dte):
    rng = np.random.default_rng(404)
    w = rng.integers(0, 1 << 32, size=1 << 16, dtype=np.uint64).astype(np.uint32)
    x = w.view(np.float32).reshape(64, 1024)
    say("[gelu patterns] f32")
    want = oracle.gelu_tanh(x, F32)
    got = to_host_typed(dte.gelu_tanh(to_dev_typed(x, F32)))
    _check(got, want, x.astype(np.float64), F32, "patterns f32")


SHAPES = [(1, 8), (3, 24), (5, 1000), (7, 4104), (2, 16384), (1, 1), (3, 13), (4, 515),
          (2, 4100), (333, 520)]


@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=NAMES.get)
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("rows,F", SHAPES)
def test_shapes(dte, rows, F, with_bias, dtype):
    say(f"[gelu] {NAMES[dtype]} rows={rows} F={F} bias={with_bias}")
    seed = 9000 + rows + 7 * F + with_bias
    x = random_typed(seed, (1, rows, F), N02, dtype).reshape(rows, F)
    b = random_typed(seed + 1, (1, 1, F), N01, dtype).reshape(F) if with_bias else None
    want = oracle.gelu_tanh(x, dtype, bias=b)
    got = to_host_typed(dte.gelu_tanh(to_dev_typed(x, dtype),
                                      None if b is None else to_dev_typed(b, dtype)))
    h = _values(x, dtype)
    if b is not None:
        h = (h.astype(np.float32) + _values(b, dtype).astype(np.float32)).astype(np.float64)
    _check(got, want, h, dtype, f"{NAMES[dtype]} {rows}x{F} bias={with_bias}")


@pytest.mark.parametrize("dtype", [BF16, F32], ids=NAMES.get)
def test_offsets_and_in_place(dte, dtype):
    rows, F = 9, 1000
    say(f"[gelu offsets] {NAMES[dtype]}")
    x = random_typed(9500, (1, rows, F), N02, dtype).reshape(rows, F)
    b = random_typed(9501, (1, 1, F), N01, dtype).reshape(F)
    want = oracle.gelu_tanh(x, dtype, bias=b)
    h = (_values(x, dtype).astype(np.float32) + _values(b, dtype).astype(np.float32)).astype(np.float64)
    dx, db = to_dev_typed(x, dtype, offset=1), to_dev_typed(b, dtype, offset=1)
    assert dx.data_ptr() % 16 != 0
    _check(to_host_typed(dte.gelu_tanh(dx, db)), want, h, dtype, "offset")
    dx = to_dev_typed(x, dtype)
    dte.gelu_tanh(dx, to_dev_typed(b, dtype), out=dx)
    _check(to_host_typed(dx), want, h, dtype, "in place")


def test_ffn_scale_sampled_rows(dte):
    # the bench's FFN intermediate [1, 32640, 16384] bf16 (video tokens x 4
    # hidden): the whole tensor through the kernel, 96 rows checked
    L, F = 32640, 16384
    say(f"[gelu ffn] [1, {L}, {F}] bf16")
    gen = torch.Generator(device="cuda").manual_seed(31)
    x = (torch.randn(1, L, F, generator=gen, device="cuda") * 2).to(torch.bfloat16)
    y = dte.gelu_tanh(x)
    rows = np.linspace(0, L - 1, 96).astype(np.int64)
    xs = to_host_typed(x[0, rows])
    ys = to_host_typed(y[0, rows])
    want = oracle.gelu_tanh(xs, BF16)
    _check(ys, want, _values(xs, BF16), BF16, "ffn sampled rows")


def test_gelu_rejections(dte):
    x = torch.zeros(2, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        dte.gelu_tanh(x, torch.zeros(7, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):
        dte.gelu_tanh(x, torch.zeros(8, dtype=torch.float16, device="cuda"))
    # out overlapping x other than exactly: rejected by the library
    buf = torch.zeros(32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dte.RGAError) as e:
        dte.gelu_tanh(buf[:16].view(2, 8), out=buf[8:24].view(2, 8))
    assert e.value.status == dte.RGA_ERR_ALIAS
    e0 = dte.gelu_tanh(torch.zeros(0, 8, dtype=torch.float32, device="cuda"))
    assert e0.shape == (0, 8)
    torch.cuda.synchronize()
