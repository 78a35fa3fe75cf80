"""Pins of the oracle's weightless-LayerNorm modulation.

Operation (reading of the LN+modulate fusion the RMSNorm+modulate page lists
beside its own, prhub summary of sglang PR #34172, "实现拆解" items 2 and 4):
y = ((x - mean) / sqrt(var + eps)) * (1 + scale) + shift, mean and biased
variance over the row, both sums in the library's pinned order.

Pinned against: binary64 with an error bound, closed forms (constant rows,
two-value rows), exact shift invariance, identity with the RMS modulation on
rows whose sum is exactly zero, an emulation of the documented order, and
torch's CPU layer_norm.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import BF16, F16, F32, N001, N01, N02, random_typed
from tests.exact_round import bf16_bits_to_f32, f32_to_bf16_bits, ulp_diff, ulp_diff_typed

EPS = np.float32(1e-6)
U32 = 2.0 ** -24
ROW, TOKEN = oracle.MOD_ROW, oracle.MOD_TOKEN


def _rows(seed, B, L, D, xdist=N02, mod=ROW, dtype=BF16):
    x = random_typed(seed, (B, L, D), xdist, dtype)
    shape = (B, L, D) if mod == TOKEN else (B, 1, D)
    return x, random_typed(seed + 1, shape, N001, dtype), random_typed(seed + 2, shape, N001, dtype)


def _f64(x, s, t, eps):
    x64 = bf16_bits_to_f32(x).astype(np.float64)
    s64 = bf16_bits_to_f32(s).astype(np.float64)
    t64 = bf16_bits_to_f32(t).astype(np.float64)
    mu = x64.mean(axis=-1, keepdims=True)
    var = ((x64 - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + float(eps))
    na = (x64 - mu) * r * (1.0 + s64)
    mean_abs = np.abs(x64).mean(axis=-1, keepdims=True)
    return na + t64, np.abs(na), r * mean_abs * np.abs(1.0 + s64)


@pytest.mark.parametrize("B,L,D", [(1, 126, 2048), (2, 40, 4096), (3, 7, 520), (1, 9, 13),
                                   (2, 5, 4100)])
def test_within_error_bound_of_binary64(B, L, D):
    x, s, t = _rows(300 + D + B, B, L, D)
    out = oracle.ln_modulate(x, s, t, EPS, ROW, BF16)
    y64, na, mterm = _f64(x, s, t, EPS)
    got = bf16_bits_to_f32(out).astype(np.float64)
    # binary32 error of the pinned sums (chain of at most ceil(D/512)*8 - 1
    # lane additions plus 6 tree levels), the mean's error carried into every
    # deviation, the division, eps add, sqrt and reciprocal, two products
    # and the final add
    chain = -(-D // 512) * 8 - 1 + 6
    bound = (chain / 2 + 10) * U32 * na + (chain + 4) * U32 * mterm + U32 * np.abs(y64)
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(y64))[1] - 9)
    assert np.all(np.abs(got - y64) <= half_ulp * (1 + 2.0 ** -7) + bound)
    well = bound < 2.0 ** -12 * np.abs(y64)
    want = f32_to_bf16_bits(y64.astype(np.float32))
    assert ulp_diff(out[well], want[well]).max() <= 1
    assert well.mean() > 0.98


@pytest.mark.parametrize("c", [1.0, -3.5, 2.0 ** -10, 100.0])
def test_constant_rows_return_the_shift(c):
    # x_d = c: the sum D c is exact, the mean is c, every deviation 0, so
    # y = (0 * r) * (1 + s) + t = t for any t other than -0
    B, L, D = 2, 3, 1024
    x = f32_to_bf16_bits(np.full((B, L, D), c, dtype=np.float32))
    s = random_typed(11, (B, 1, D), N001, BF16)
    t = random_typed(12, (B, 1, D), N001, BF16)
    t[t == 0x8000] = 0
    y = oracle.ln_modulate(x, s, t, EPS, ROW, BF16)
    assert np.array_equal(y, np.broadcast_to(t, (B, L, D)))
    mean, rstd = oracle.ln_factors(x, EPS, BF16)
    assert np.all(mean == np.float32(c))
    assert np.all(rstd == np.float32(1) / np.sqrt(EPS))


@pytest.mark.parametrize("delta", [2.0 ** -11, 2.0 ** -4, 1.0, 8.0])
def test_two_value_rows_closed_form(delta):
    # x alternates c + delta, c - delta (c = 4 delta: both exact in bf16):
    # mean c and variance delta^2 exactly, so
    # y = +-delta / sqrt(delta^2 + eps) * (1 + s) + t
    B, L, D, c = 1, 2, 2048, 4 * delta
    v = np.where(np.arange(D) % 2 == 0, c + delta, c - delta).astype(np.float32)
    xf = np.broadcast_to(v, (B, L, D)).copy()
    x = f32_to_bf16_bits(xf)
    assert np.array_equal(bf16_bits_to_f32(x), xf)
    s = random_typed(13, (B, 1, D), N001, BF16)
    t = random_typed(14, (B, 1, D), N001, BF16)
    y = oracle.ln_modulate(x, s, t, EPS, ROW, BF16)
    r64 = 1.0 / np.sqrt(delta * delta + float(EPS))
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    y64 = sign * delta * r64 * (1.0 + bf16_bits_to_f32(s).astype(np.float64)) \
        + bf16_bits_to_f32(t).astype(np.float64)
    want = f32_to_bf16_bits(np.broadcast_to(y64, (B, L, D)).astype(np.float32))
    assert ulp_diff(y, want).max() <= 1


def test_exact_shift_invariance():
    # multiples of 1/8 in [-8, 8) and the same values plus 16 are exact in
    # bf16, every partial and the mean are exact in binary32 (D a power of
    # two), so x + 16 and x give the same deviations: identical outputs
    B, L, D = 2, 5, 1024
    rng = np.random.default_rng(15)
    q = rng.integers(-64, 64, size=(B, L, D)).astype(np.float32) / 8
    x0, x1 = f32_to_bf16_bits(q), f32_to_bf16_bits(q + 16)
    assert np.array_equal(bf16_bits_to_f32(x1), q + 16)
    s = random_typed(16, (B, 1, D), N001, BF16)
    t = random_typed(17, (B, 1, D), N001, BF16)
    a = oracle.ln_modulate(x0, s, t, EPS, ROW, BF16)
    b = oracle.ln_modulate(x1, s, t, EPS, ROW, BF16)
    assert np.array_equal(a, b)


def test_zero_sum_rows_equal_the_rms_modulation():
    # small integers in +-pairs inside every group: every partial sum is
    # exact, the mean is exactly 0, the deviations are x itself, so the
    # LayerNorm modulation is the RMS modulation bit for bit
    B, L, D = 2, 4, 4096
    rng = np.random.default_rng(18)
    half = rng.integers(-20, 21, size=(B, L, D // 2)).astype(np.float32)
    xf = np.empty((B, L, D), dtype=np.float32)
    xf[..., 0::2], xf[..., 1::2] = half, -half
    x = f32_to_bf16_bits(xf)
    s = random_typed(19, (B, 1, D), N001, BF16)
    t = random_typed(20, (B, 1, D), N001, BF16)
    mean, _ = oracle.ln_factors(x, EPS, BF16)
    assert np.all(mean == 0)
    assert np.array_equal(oracle.ln_modulate(x, s, t, EPS, ROW, BF16),
                          oracle.rms_modulate(x, s, t, EPS))


def test_factors_follow_the_documented_order():
    # numpy binary32 scalars: groups of 8 (last one shorter), group k ->
    # partial k mod P, xor-distance tree; mean first, then the deviations
    D = 1037
    x = random_typed(21, (1, 2, D), N01, BF16)
    xf = bf16_bits_to_f32(x)
    for P in (64, 4):
        mean, rstd = oracle.ln_factors(x, EPS, BF16, partials=P)
        for row in range(2):
            def tree(vals):
                part = [np.float32(0)] * P
                for k in range((D + 7) // 8):
                    for d in range(8 * k, min(8 * k + 8, D)):
                        part[k % P] = np.float32(part[k % P] + vals(d))
                m = 1
                while m < P:
                    part = [np.float32(part[j] + part[j ^ m]) for j in range(P)]
                    m <<= 1
                return part[0]
            mu = np.float32(tree(lambda d: xf[0, row, d]) / np.float32(D))
            ss = tree(lambda d: np.float32(np.float32(xf[0, row, d] - mu) ** 2))
            var = np.float32(ss / np.float32(D))
            r = np.float32(np.float32(1) / np.sqrt(np.float32(var + EPS)))
            assert mu.view(np.uint32) == mean[0, row].view(np.uint32), (P, row)
            assert r.view(np.uint32) == rstd[0, row].view(np.uint32), (P, row)


@pytest.mark.parametrize("D", [2048, 4096])
def test_unmodulated_path_matches_torch_layer_norm(D):
    # scale = +0, shift = -0 leave the normalized value unchanged bit for bit.
    # torch sums in another order; the two differ by more than one ULP only
    # where x - mean cancels, i.e. by no more than the mean's rounding error
    # carried through r
    x = random_typed(22 + D, (2, 33, D), N02, BF16)
    s = np.zeros((2, 1, D), dtype=np.uint16)
    t = np.full((2, 1, D), 0x8000, dtype=np.uint16)
    y = oracle.ln_modulate(x, s, t, EPS, ROW, BF16)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(bf16_bits_to_f32(x)), [D],
                                         eps=float(EPS)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    d = ulp_diff(y, ref)
    yf, rf = bf16_bits_to_f32(y).astype(np.float64), bf16_bits_to_f32(ref).astype(np.float64)
    assert d[np.abs(rf) >= 2.0 ** -8].max() <= 1
    xf = bf16_bits_to_f32(x).astype(np.float64)
    _, rstd = oracle.ln_factors(x, EPS, BF16)
    mean_err = 64 * U32 * np.abs(xf).mean(axis=-1) * rstd
    small = np.abs(rf) < 2.0 ** -8
    assert np.all(np.abs(yf - rf)[small] <= (mean_err[..., None] + 2.0 ** -16)
                  .repeat(D, axis=-1)[small])
    assert (d > 0).mean() < 1e-3


def test_token_layout_and_storage_types():
    # per-token rows equal to the broadcast row give the row result; binary16
    # and binary32 storage follow the same steps with their own rounding
    B, L, D = 2, 6, 520
    x, s, t = _rows(23, B, L, D)
    a = oracle.ln_modulate(x, s, t, EPS, ROW, BF16)
    b = oracle.ln_modulate(x, np.broadcast_to(s, (B, L, D)).copy(),
                           np.broadcast_to(t, (B, L, D)).copy(), EPS, TOKEN, BF16)
    assert np.array_equal(a, b)
    xf = bf16_bits_to_f32(x)
    sf, tf = bf16_bits_to_f32(s), bf16_bits_to_f32(t)
    y32 = oracle.ln_modulate(xf, sf, tf, EPS, ROW, F32)
    # bf16 result = the binary32 result rounded once
    assert np.array_equal(f32_to_bf16_bits(y32), a)
    x16 = xf.astype(np.float16).view(np.uint16)
    s16, t16 = sf.astype(np.float16).view(np.uint16), tf.astype(np.float16).view(np.uint16)
    y16 = oracle.ln_modulate(x16, s16, t16, EPS, ROW, F16)
    y32b = oracle.ln_modulate(x16.view(np.float16).astype(np.float32),
                              s16.view(np.float16).astype(np.float32),
                              t16.view(np.float16).astype(np.float32), EPS, ROW, F32)
    assert ulp_diff_typed(y16, y32b.astype(np.float16).view(np.uint16), F16).max() <= 0
