"""Pins of the oracle's gated residual add against facts fixed outside it:
exact rational arithmetic, binary64 arithmetic rounded by library routines,
torch CPU, broadcasting semantics and IEEE special-value rules.

The operation is the residual-gate update of "[KDA-Pilot] Add diffusion
residual-gate CUDA fast path for LTX2" ("Motivation"): hidden + update * gate
over [B, L, D] with a full or [B, 1, D] gate, read as binary32 multiply,
binary32 add, one bf16 round-to-nearest-even.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import N01, U11, random_bits
from tests.exact_round import (
    bf16_bits_to_f32, exact_gate_add_bits, f32_to_bf16_bits, is_nan)

FULL, BCAST = oracle.GATE_FULL, oracle.GATE_BCAST


def _bits(values):
    return f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


def _same(a, b):
    """Bitwise equal, with any NaN equal to any NaN (compared by class)."""
    na, nb = is_nan(a), is_nan(b)
    return bool(np.all(na == nb) and np.all((a == b) | na))


def _library_reference(x, u, g):
    """bf16(fl32(x + fl32(u*g))) from binary64 arithmetic and library casts:
    the binary64 product of two bf16 values is exact, numpy's cast rounds it
    to binary32, the binary64 sum of two binary32 values is checked exact by
    the two-sum error term, numpy rounds it to binary32 and torch to bf16.
    Returns (bits, exact_mask)."""
    x64 = bf16_bits_to_f32(x).astype(np.float64)
    u64 = bf16_bits_to_f32(u).astype(np.float64)
    g64 = bf16_bits_to_f32(g).astype(np.float64)
    with np.errstate(all="ignore"):
        p32 = (u64 * g64).astype(np.float32)
        p64 = p32.astype(np.float64)
        s64 = x64 + p64
        bb = s64 - x64
        err = (x64 - (s64 - bb)) + (p64 - bb)
        exact = ~np.isfinite(s64) | (err == 0)
        s32 = s64.astype(np.float32)
    return f32_to_bf16_bits(s32), exact


def test_contraction_probe_is_zero():
    # a*b + c with a = b = 1 + 2^-12, c = -(1 + 2^-11): 0 with two roundings,
    # 2^-24 if the build fused the multiply-add.
    assert oracle.contraction_probe() == 0.0


RNE_TABLE = [
    # (binary32 pattern, bf16 pattern) from the IEEE round-to-nearest-even rule
    (0x3F800000, 0x3F80),  # 1.0 exact
    (0x3F808000, 0x3F80),  # halfway, kept part even -> down
    (0x3F818000, 0x3F82),  # halfway, kept part odd -> up
    (0x3F808001, 0x3F81),  # above half -> up
    (0x3F807FFF, 0x3F80),  # below half -> down
    (0xBF818000, 0xBF82),  # sign symmetric
    (0x7F7F7FFF, 0x7F7F),  # largest below the overflow tie
    (0x7F7F8000, 0x7F80),  # overflow tie rounds to infinity (odd kept part)
    (0x7F7FFFFF, 0x7F80),  # max binary32 -> infinity
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00008000, 0x0000),  # subnormal halfway to even zero
    (0x00018000, 0x0002),  # subnormal halfway up to even
    (0x00000001, 0x0000),  # smallest subnormal -> 0
    (0x007FFFFF, 0x0080),  # largest subnormal rounds up to min normal
    (0x80008001, 0x8001),  # negative subnormal above half
]


def test_rne_table():
    src = np.array([p for p, _ in RNE_TABLE], dtype=np.uint32).view(np.float32)
    want = np.array([b for _, b in RNE_TABLE], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.bf16_from_f32(src), want)


def test_rne_nan_stays_nan():
    pats = np.array([0x7F800001, 0x7FC00000, 0xFFFFFFFF, 0x7F80FFFF,
                     0xFF800001, 0x7FFFFFFF], dtype=np.uint32)
    out = oracle.bf16_from_f32(pats.view(np.float32))
    assert is_nan(out).all()
    # sign survives
    assert ((out >> 15) == (pats >> 31)).all()


def test_rne_matches_torch_on_random_patterns():
    rng = np.random.default_rng(1)
    pats = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # plus every tie and near-tie around a spread of exponents
    hi = rng.integers(0, 2**16, size=200_000, dtype=np.uint64).astype(np.uint32) << 16
    extra = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    f = np.concatenate([pats, extra]).view(np.float32)
    got = oracle.bf16_from_f32(f)
    want = f32_to_bf16_bits(f)
    assert _same(got, want)


def test_widening_matches_torch():
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f32_from_bf16(allp)
    want = bf16_bits_to_f32(allp)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("shape", [(1, 126, 2048), (2, 33, 520), (3, 5, 8)])
def test_gate_add_full_vs_binary64(shape):
    x = random_bits(11, shape, N01)
    u = random_bits(12, shape, N01)
    g = random_bits(13, shape, U11)
    want, exact = _library_reference(x, u, g)
    assert exact.all()
    assert _same(oracle.gate_add(x, u, g, FULL), want)


def test_gate_add_vs_torch_cpu_fp32():
    shape = (2, 64, 1024)
    x = random_bits(21, shape, N01)
    u = random_bits(22, shape, N01)
    g = random_bits(23, shape, U11)
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    ref = (t(x).float() + t(u).float() * t(g).float()).bfloat16()
    want = ref.view(torch.int16).numpy().view(np.uint16)
    assert _same(oracle.gate_add(x, u, g, FULL), want)


@pytest.mark.parametrize("B", [1, 2, 3])
def test_bcast_equals_full_with_repeated_row(B):
    # broadcasting a [B,1,D] gate over L equals the full gate with row b
    # repeated L times
    L, D = 37, 264
    x = random_bits(31 + B, (B, L, D))
    u = random_bits(41 + B, (B, L, D))
    grow = random_bits(51 + B, (B, 1, D), U11)
    gfull = np.ascontiguousarray(np.broadcast_to(grow, (B, L, D)))
    a = oracle.gate_add(x, u, grow, BCAST)
    b = oracle.gate_add(x, u, gfull, FULL)
    assert np.array_equal(a, b)
    # and batch b really used row b
    for bi in range(B):
        one = oracle.gate_add(x[bi:bi + 1].copy(), u[bi:bi + 1].copy(),
                              grow[bi:bi + 1].copy(), BCAST)
        assert np.array_equal(a[bi], one[0])


def test_all_ones_gate_is_torch_bf16_add():
    shape = (1, 200, 512)
    x = random_bits(61, shape)
    u = random_bits(62, shape)
    ones = _bits(np.ones((1, 1, 512)))
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    want = (t(x) + t(u)).view(torch.int16).numpy().view(np.uint16)
    assert _same(oracle.gate_add(x, u, ones, BCAST), want)


def test_zero_gate_is_identity():
    shape = (2, 50, 256)
    x = random_bits(71, shape)
    x[x == 0x8000] = 0  # -0 + +0 = +0 is the one exception
    u = random_bits(72, shape)
    zeros = np.zeros((2, 1, 256), dtype=np.uint16)
    assert np.array_equal(oracle.gate_add(x, u, zeros, BCAST), x)


def test_in_place_equals_out_of_place():
    shape = (2, 17, 136)
    x = random_bits(81, shape)
    u = random_bits(82, shape)
    g = random_bits(83, (2, 1, 136), U11)
    want = oracle.gate_add(x, u, g, BCAST)
    xx = x.copy()
    oracle.gate_add(xx, u, g, BCAST, out=xx)
    assert np.array_equal(xx, want)
    gf = random_bits(84, shape, U11)
    want = oracle.gate_add(x, u, gf, FULL)
    uu = u.copy()
    oracle.gate_add(x, uu, gf, FULL, out=uu)
    assert np.array_equal(uu, want)


# (u, g) pairs covering normal, subnormal-product, overflowing, zero, signed
# zero, infinite and NaN products
PAIRS = [
    (1.5, 0.75), (-0.3125, 0.8125), (3.0e-3, -2.5e2),
    (1.0078125 * 2.0 ** -70, 1.9921875 * 2.0 ** -62),   # product subnormal, inexact
    (-1.5 * 2.0 ** -75, 1.25 * 2.0 ** -60),             # subnormal, exact
    (2.0 ** -100, 2.0 ** -60),                           # underflows to 0
    (1.5 * 2.0 ** 100, 1.75 * 2.0 ** 30),                # overflows to inf
    (0.0, 5.0), (-0.0, 5.0), (0.0, -0.0),
    (float("inf"), 0.5), (float("inf"), 0.0), (float("nan"), 1.0),
]


def test_all_x_patterns_against_exact_arithmetic():
    xs = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n = xs.size
    for uf, gf in PAIRS:
        ub, gb = _bits([uf])[0], _bits([gf])[0]
        x = xs.reshape(1, 1, n)
        u = np.full((1, 1, n), ub, dtype=np.uint16)
        g = np.full((1, 1, n), gb, dtype=np.uint16)
        got = oracle.gate_add(x, u, g, FULL)
        want, exact = _library_reference(x, u, g)
        # the binary64 route is exact where the two-sum error vanishes;
        # everywhere else use exact rationals
        idx = np.nonzero(~exact.ravel())[0]
        want = want.ravel().copy()
        for i in idx:
            want[i] = exact_gate_add_bits(int(xs[i]), int(ub), int(gb))
        assert _same(got.ravel(), want), (uf, gf)
        # a sample of exact-route elements also checked by rationals
        for i in range(0, n, 4099):
            e = exact_gate_add_bits(int(xs[i]), int(ub), int(gb))
            assert _same(np.array([got.ravel()[i]]), np.array([e], dtype=np.uint16)), (uf, gf, i)


@pytest.mark.parametrize("B,L,D", [
    (b, l, d) for b, l, d in itertools.product([1, 2, 3], [1, 2, 5], [8, 16, 24])]
    + [(1, 126, 8), (2, 1, 520)])
@pytest.mark.parametrize("mode", [FULL, BCAST])
def test_tiny_shapes_against_exact_rationals(B, L, D, mode):
    seed = 1000 + 97 * B + 13 * L + D + 7 * mode
    x = random_bits(seed, (B, L, D))
    u = random_bits(seed + 1, (B, L, D))
    gshape = (B, L, D) if mode == FULL else (B, 1, D)
    g = random_bits(seed + 2, gshape, U11)
    got = oracle.gate_add(x, u, g, mode)
    for b in range(B):
        for l in range(L):
            for d in range(D):
                gi = g[b, l, d] if mode == FULL else g[b, 0, d]
                want = exact_gate_add_bits(int(x[b, l, d]), int(u[b, l, d]), int(gi))
                assert got[b, l, d] == want, (b, l, d)


def test_special_value_table():
    inf, nan = float("inf"), float("nan")
    big = 1.5 * 2.0 ** 127
    rows = [
        # x, u, g, expected (None = NaN)
        (0.0, 0.0, 0.0, 0x0000),
        (-0.0, -0.0, 1.0, 0x8000),     # -0 + -0 = -0
        (-0.0, 0.0, 1.0, 0x0000),      # -0 + +0 = +0
        (1.0, -1.0, 1.0, 0x0000),      # exact cancellation gives +0
        (inf, 1.0, 1.0, 0x7F80),
        (-inf, 1.0, 1.0, 0xFF80),
        (inf, -inf, 1.0, None),        # inf - inf
        (1.0, inf, 0.0, None),         # inf * 0
        (nan, 1.0, 1.0, None),
        (1.0, nan, 1.0, None),
        (big, big, 1.0, 0x7F80),       # sum overflows binary32
        (-big, big, -1.0, 0xFF80),
        (1.0, 2.0 ** 100, 2.0 ** 100, 0x7F80),  # product overflows
        (2.0 ** -133, 0.0, 0.0, 0x0001),        # bf16 subnormal passes through
    ]
    x = _bits([r[0] for r in rows]).reshape(1, 1, -1)
    u = _bits([r[1] for r in rows]).reshape(1, 1, -1)
    g = _bits([r[2] for r in rows]).reshape(1, 1, -1)
    got = oracle.gate_add(x, u, g, FULL).ravel()
    for i, r in enumerate(rows):
        if r[3] is None:
            assert is_nan(got[i:i + 1])[0], r
        else:
            assert got[i] == r[3], (r, hex(got[i]))


def test_subnormal_product_rounds_before_the_add():
    # u*g = -2^-132 * (1 + a/128)(1 + b/128) is subnormal in binary32 (exact
    # there: its lowest bit, 2^-147, is above the subnormal quantum 2^-149)
    # and x = 2^-126 puts the sum on the normal/subnormal boundary, where
    # bf16 keeps bits of the product down to 2^-133: a product flushed to
    # zero, or a sum on the wrong grid, shows. Checked against exact
    # rationals element by element. (A fused multiply-add cannot show at a
    # bf16 output: a product of two bf16 values has at most 16 significant
    # bits, so only subnormal products round in binary32, and the bf16
    # rounding of the sum never sees those bits; the build's probe pins the
    # contraction instead.)
    vals = []
    for a in range(1, 128, 9):
        for b in range(1, 128, 11):
            vals.append((2.0 ** -126, (1 + a / 128) * 2.0 ** -70, -(1 + b / 128) * 2.0 ** -62))
    x = _bits([v[0] for v in vals]).reshape(1, 1, -1)
    u = _bits([v[1] for v in vals]).reshape(1, 1, -1)
    g = _bits([v[2] for v in vals]).reshape(1, 1, -1)
    got = oracle.gate_add(x, u, g, FULL).ravel()
    for i in range(len(vals)):
        assert got[i] == exact_gate_add_bits(int(x.ravel()[i]), int(u.ravel()[i]), int(g.ravel()[i]))
