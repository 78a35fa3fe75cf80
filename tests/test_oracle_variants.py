"""Pins of the oracle's storage-type, per-token and any-D variants
(oracle_*_ex) against numpy/torch conversions and binary64 arithmetic.

The residual-gate page's test covers "dtype coverage" and "tail shapes"
("[KDA-Pilot] Add diffusion residual-gate CUDA fast path for LTX2",
"Modifications"); the reading is binary32 arithmetic with one
round-to-nearest-even narrowing to the storage type.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import N001, N01, N02, U11, random_bits
from tests.exact_round import bf16_bits_to_f32, f32_to_bf16_bits, ulp_diff

EPS = np.float32(1e-6)
U32 = 2.0 ** -24
BF16, F16, F32 = oracle.BF16, oracle.F16, oracle.F32


# ---- conversions through libraries (independent of the oracle) -------------

def to_f32(a, dtype):
    if dtype == BF16:
        return bf16_bits_to_f32(a)
    if dtype == F16:
        return a.view(np.float16).astype(np.float32)
    return a.astype(np.float32)


def from_f32(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    if dtype == F16:
        with np.errstate(over="ignore"):
            return a.astype(np.float16).view(np.uint16)
    return a


def rand(seed, shape, dist, dtype):
    rng = np.random.default_rng(seed)
    return from_f32(dist.draw(rng, (int(np.prod(shape)),)).reshape(shape), dtype)


def is_nan16(bits, dtype):
    if dtype == BF16:
        return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
    return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x03FF) != 0)


def same(a, b, dtype):
    if dtype == F32:
        na, nb = np.isnan(a), np.isnan(b)
        return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))
    na, nb = is_nan16(a, dtype), is_nan16(b, dtype)
    return bool(np.array_equal(na, nb) and np.all((a == b) | na))


# ---- binary16 conversions ---------------------------------------------------

def test_f16_widening_all_patterns():
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f32_from_f16(a)
    want = a.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


F16_TABLE = [
    (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (70000.0, 0x7C00),
    (-65520.0, 0xFC00), (1.0, 0x3C00), (1.0 + 2.0 ** -11, 0x3C00),    # tie to even
    (1.0 + 3 * 2.0 ** -11, 0x3C02), (2.0 ** -14, 0x0400), (2.0 ** -24, 0x0001),
    (2.0 ** -25, 0x0000), (3 * 2.0 ** -25, 0x0002), (2.0 ** -14 - 2.0 ** -25, 0x0400),
    (-0.0, 0x8000), (float("inf"), 0x7C00),
]


def test_f16_narrowing_table():
    src = np.array([v for v, _ in F16_TABLE], dtype=np.float32)
    want = np.array([b for _, b in F16_TABLE], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.f16_from_f32(src), want)


def test_f16_narrowing_matches_numpy():
    rng = np.random.default_rng(5)
    pats = rng.integers(0, 2 ** 32, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    # concentrate on the binary16 range and its rounding boundaries
    near = (rng.integers(0x33000000, 0x47900000, size=2_000_000, dtype=np.uint64)).astype(np.uint32)
    ties = (near & ~np.uint32(0x1FFF)) | np.uint32(0x1000)
    f = np.concatenate([pats, near, ties]).view(np.float32)
    got = oracle.f16_from_f32(f)
    with np.errstate(over="ignore", invalid="ignore"):
        want = f.astype(np.float16).view(np.uint16)
    assert same(got, want, F16)


# ---- gate-add variants --------------------------------------------------------

@pytest.mark.parametrize("mode", [oracle.GATE_FULL, oracle.GATE_BCAST])
def test_ex_bf16_equals_the_original(mode):
    shape = (2, 33, 520)
    x, u = random_bits(1, shape), random_bits(2, shape)
    g = random_bits(3, shape if mode == oracle.GATE_FULL else (2, 1, 520), U11)
    assert np.array_equal(oracle.gate_add_ex(x, u, g, mode, BF16), oracle.gate_add(x, u, g, mode))


def test_f16_gate_add_against_binary64_and_library_rounding():
    shape = (2, 40, 1000)
    x, u, g = rand(10, shape, N01, F16), rand(11, shape, N01, F16), rand(12, shape, U11, F16)
    got = oracle.gate_add_ex(x, u, g, oracle.GATE_FULL, F16)
    x64, u64, g64 = (to_f32(a, F16).astype(np.float64) for a in (x, u, g))
    p32 = (u64 * g64).astype(np.float32)          # exact: 11 x 11 significand bits
    s64 = x64 + p32.astype(np.float64)
    bb = s64 - x64
    assert np.all((x64 - (s64 - bb)) + (p32 - bb) == 0)  # two-sum: the sum is exact
    want = from_f32(s64.astype(np.float32), F16)
    assert same(got, want, F16)
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.float16)
    tw = (t(x).float() + t(u).float() * t(g).float()).half().view(torch.int16).numpy().view(np.uint16)
    assert same(got, tw, F16)


def test_f16_every_x_pattern():
    xs = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1, 1, -1)
    for uf, gf in [(1.5, 0.75), (3.0e-3, -250.0), (2.0 ** -12, 2.0 ** -13), (100.0, 700.0)]:
        u = np.full(xs.shape, from_f32(np.float32(uf), F16), dtype=np.uint16)
        g = np.full(xs.shape, from_f32(np.float32(gf), F16), dtype=np.uint16)
        got = oracle.gate_add_ex(xs, u, g, oracle.GATE_FULL, F16)
        with np.errstate(all="ignore"):
            p = (to_f32(u, F16) * to_f32(g, F16)).astype(np.float32)
            s = (to_f32(xs, F16).astype(np.float64) + p.astype(np.float64)).astype(np.float32)
        assert same(got, from_f32(s, F16), F16), (uf, gf)


def test_f32_gate_add_is_numpy_float32_arithmetic():
    shape = (3, 17, 264)
    x, u, g = rand(20, shape, N01, F32), rand(21, shape, N01, F32), rand(22, (3, 1, 264), U11, F32)
    got = oracle.gate_add_ex(x, u, g, oracle.GATE_BCAST, F32)
    want = x + u * g  # numpy float32: multiply rounded, then add rounded
    assert same(got, want.astype(np.float32), F32)


# ---- modulation variants ------------------------------------------------------

def _half_ulp(y, dtype):
    e = np.frexp(np.abs(y))[1]
    if dtype == BF16:
        return np.ldexp(1.0, e - 9)
    if dtype == F16:
        return np.maximum(np.ldexp(1.0, e - 12), 2.0 ** -25)
    return np.zeros_like(y)


def _check_bound(out, x, s, t, eps, dtype, mod_mode):
    B, L, D = x.shape
    x64 = to_f32(x, dtype).astype(np.float64)
    s64 = to_f32(s, dtype).astype(np.float64)
    t64 = to_f32(t, dtype).astype(np.float64)
    r64 = 1.0 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + float(eps))
    na = x64 * r64 * (1.0 + s64)
    y64 = na + t64
    groups = -(-D // 8)
    chain = -(-groups // 64) * 8 - 1 + 6
    bound = (chain / 2 + 8) * U32 * np.abs(na) + U32 * np.abs(y64)
    got = to_f32(out, dtype).astype(np.float64)
    assert np.all(np.abs(got - y64) <= _half_ulp(y64, dtype) * (1 + 2.0 ** -7) + bound)
    if dtype != F32:
        well = bound < 2.0 ** -14 * np.abs(y64)
        want = from_f32(y64.astype(np.float32), dtype)
        assert ulp_diff(out[well], want[well]).max() <= 1
        assert well.mean() > 0.98


@pytest.mark.parametrize("D", [8, 12, 520, 1001, 2048, 4100])
@pytest.mark.parametrize("dtype", [BF16, F16, F32])
@pytest.mark.parametrize("mod_mode", [oracle.MOD_ROW, oracle.MOD_TOKEN])
def test_modulation_variants_within_binary64_bound(D, dtype, mod_mode):
    B, L = 2, 9
    x = rand(30 + D, (B, L, D), N02, dtype)
    mshape = (B, 1, D) if mod_mode == oracle.MOD_ROW else (B, L, D)
    s = rand(31 + D, mshape, N001, dtype)
    t = rand(32 + D, mshape, N001, dtype)
    out = oracle.rms_modulate_ex(x, s, t, EPS, mod_mode, dtype)
    _check_bound(out, x, s, t, EPS, dtype, mod_mode)


def test_ex_rms_bf16_row_equals_the_original():
    x = random_bits(40, (2, 21, 1032), N02)
    s, t = random_bits(41, (2, 1, 1032), N001), random_bits(42, (2, 1, 1032), N001)
    assert np.array_equal(oracle.rms_modulate_ex(x, s, t, EPS, oracle.MOD_ROW, BF16),
                          oracle.rms_modulate(x, s, t, EPS))


@pytest.mark.parametrize("dtype", [BF16, F16, F32])
def test_token_modulation_with_repeated_rows_equals_row_modulation(dtype):
    B, L, D = 2, 7, 520
    x = rand(50, (B, L, D), N02, dtype)
    s, t = rand(51, (B, 1, D), N001, dtype), rand(52, (B, 1, D), N001, dtype)
    st = np.ascontiguousarray(np.broadcast_to(s, (B, L, D)))
    tt = np.ascontiguousarray(np.broadcast_to(t, (B, L, D)))
    a = oracle.rms_modulate_ex(x, s, t, EPS, oracle.MOD_ROW, dtype)
    b = oracle.rms_modulate_ex(x, st, tt, EPS, oracle.MOD_TOKEN, dtype)
    assert same(a, b, dtype)


def test_any_d_with_one_partial_is_sequential():
    # P = 1 puts every group, partial last group included, in one partial in
    # element order: the plain sequential sum
    x = random_bits(60, (1, 5, 1001), N01)
    s = np.zeros((1, 1, 1001), dtype=np.uint16)
    t = np.full((1, 1, 1001), 0x8000, dtype=np.uint16)
    a = oracle.rms_modulate_ex(x, s, t, EPS, oracle.MOD_ROW, BF16, partials=1)
    xf = bf16_bits_to_f32(x)
    for row in range(5):
        ss = np.float32(0)
        for v in xf[0, row]:
            ss = np.float32(ss + np.float32(v * v))
        r = np.float32(np.float32(1) / np.sqrt(np.float32(np.float32(ss / np.float32(1001)) + EPS)))
        want = f32_to_bf16_bits((xf[0, row] * r).astype(np.float32))
        assert np.array_equal(a[0, row], want), row


@pytest.mark.parametrize("dtype", [BF16, F16, F32])
def test_fused_ex_is_the_composition(dtype):
    B, L, D = 2, 6, 1001
    x, u = rand(70, (B, L, D), N02, dtype), rand(71, (B, L, D), N01, dtype)
    g = rand(72, (B, 1, D), N001, dtype)
    s, t = rand(73, (B, L, D), N001, dtype), rand(74, (B, L, D), N001, dtype)
    xo, y = oracle.gate_add_rms_modulate_ex(x, u, g, s, t, EPS, oracle.GATE_BCAST,
                                            oracle.MOD_TOKEN, dtype)
    wx = oracle.gate_add_ex(x, u, g, oracle.GATE_BCAST, dtype)
    assert same(xo, wx, dtype)
    assert same(y, oracle.rms_modulate_ex(wx, s, t, EPS, oracle.MOD_TOKEN, dtype), dtype)
