"""Pins of the oracle's weightless-RMSNorm modulation against facts fixed
outside it: the binary64 definition with a rigorous binary32 error bound,
closed forms (constant and zero rows), torch's CPU rms_norm, the identity
composition of the unmodulated path, scale invariance and the pages' own
test tolerance.

Operation: rms_norm(x, eps) * (1 + scale) + shift with a weightless RMSNorm
(prhub summary of sglang PR #34172, "关键源码片段"; RMSNormNoWeight and eps
1e-6 from its unit test), one bf16 rounding at the end.
"""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import N001, N01, N02, random_bits
from tests.exact_round import bf16_bits_to_f32, f32_to_bf16_bits, ulp_diff

EPS = np.float32(1e-6)
U32 = 2.0 ** -24


def _rows(seed, B, L, D, xdist=N01):
    x = random_bits(seed, (B, L, D), xdist)
    s = random_bits(seed + 1, (B, 1, D), N001)
    t = random_bits(seed + 2, (B, 1, D), N001)
    return x, s, t


def _f64_reference(x, s, t, eps):
    """y = x * r * (1 + s) + t in binary64 with r = 1/sqrt(mean(x^2) + eps),
    plus |x r (1+s)| for the error bound."""
    x64 = bf16_bits_to_f32(x).astype(np.float64)
    s64 = bf16_bits_to_f32(s).astype(np.float64)
    t64 = bf16_bits_to_f32(t).astype(np.float64)
    r64 = 1.0 / np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + float(eps))
    na = x64 * r64 * (1.0 + s64)
    return na + t64, np.abs(na), r64


def _bound(D, na_abs, y64):
    """Rigorous bound on |fl32 result - exact| for the pinned order: every
    square passes through at most ceil(D/512)*8 - 1 lane additions plus 6
    tree levels; the division by D, the eps add, sqrt and reciprocal add a
    few roundings (sqrt halves the incoming relative error); the products by
    r and (1 + s) two more; the final add one relative to |y|."""
    chain = -(-D // 512) * 8 - 1 + 6
    k = chain / 2 + 8
    return k * U32 * na_abs + U32 * np.abs(y64)


def _check_against_f64(out, x, s, t, eps):
    D = x.shape[-1]
    y64, na, _ = _f64_reference(x, s, t, eps)
    got = bf16_bits_to_f32(out).astype(np.float64)
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(y64))[1] - 9)  # half bf16 ulp of |y|
    err = np.abs(got - y64)
    assert np.all(err <= half_ulp * (1 + 2.0 ** -7) + _bound(D, na, y64))
    # Away from cancellation (the binary32 error far below one bf16 ulp of
    # y) the rounded result is within one bf16 ulp of the exact value.
    well = _bound(D, na, y64) < 2.0 ** -12 * np.abs(y64)
    want = f32_to_bf16_bits(y64.astype(np.float32))
    assert ulp_diff(out[well], want[well]).max() <= 1
    return well.mean()


@pytest.mark.parametrize("B,L,D", [(1, 126, 2048), (2, 40, 4096), (1, 64, 3072),
                                   (3, 7, 520), (1, 5, 8)])
def test_modulate_within_rigorous_bound_of_binary64(B, L, D):
    x, s, t = _rows(100 + D + B, B, L, D, N02 if D == 4096 else N01)
    out = oracle.rms_modulate(x, s, t, EPS)
    frac_well = _check_against_f64(out, x, s, t, EPS)
    assert frac_well > 0.99


@pytest.mark.parametrize("c", [2.0 ** -12, -(2.0 ** -10), 2.0 ** -10, 2.0 ** -8, 1.0, -8.0])
@pytest.mark.parametrize("D", [64, 2048, 4096])
def test_constant_rows_closed_form(c, D):
    # x_d = c: sum of squares D*c^2 is exact, r = 1/sqrt(c^2 + eps); for
    # |c| near 2^-10 the eps term is of the same size as c^2, so its place
    # inside the square root decides the result.
    B, L = 2, 3
    x = f32_to_bf16_bits(np.full((B, L, D), c, dtype=np.float32))
    s = random_bits(7, (B, 1, D), N001)
    t = np.zeros((B, 1, D), dtype=np.uint16)
    out = oracle.rms_modulate(x, s, t, EPS)
    r64 = 1.0 / np.sqrt(c * c + float(EPS))
    y64 = c * r64 * (1.0 + bf16_bits_to_f32(s).astype(np.float64))
    y64 = np.broadcast_to(y64, (B, L, D))
    want = f32_to_bf16_bits(y64.astype(np.float32))
    assert ulp_diff(out, want).max() <= 1
    fac = oracle.rms_factors(x, EPS)
    assert np.all(np.abs(fac.astype(np.float64) / r64 - 1) < 4 * U32)


def test_zero_rows_return_shift():
    B, L, D = 2, 4, 1024
    x = np.zeros((B, L, D), dtype=np.uint16)
    s = random_bits(9, (B, 1, D), N001)
    t = random_bits(10, (B, 1, D), N001)
    t[t == 0x8000] = 0  # keep +0 + -0 aside
    out = oracle.rms_modulate(x, s, t, EPS)
    assert np.array_equal(out, np.broadcast_to(t, (B, L, D)))


@pytest.mark.parametrize("D", [2048, 4096, 520])
def test_unmodulated_path_is_the_norm(D):
    # scale = +0 and shift = -0 make (n * 1) + (-0) == n exactly for every n,
    # so the modulation reduces to the weightless norm bit for bit
    x = random_bits(200 + D, (2, 33, D), N02)
    s = np.zeros((2, 1, D), dtype=np.uint16)
    t = np.full((2, 1, D), 0x8000, dtype=np.uint16)
    y = oracle.rms_modulate(x, s, t, EPS)
    assert np.array_equal(y, oracle.rms_norm(x, EPS))
    # and the norm is within one bf16 ulp of torch's CPU rms_norm in fp32
    xt = torch.from_numpy(bf16_bits_to_f32(x))
    ref = torch.nn.functional.rms_norm(xt, [D], eps=float(EPS)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    assert ulp_diff(y, ref).max() <= 1


def test_scale_invariance_without_eps():
    # with eps = 0, x -> 2^k x scales ss by 4^k, sqrt by 2^k and r by 2^-k,
    # all exactly, so the output is unchanged bit for bit
    x, s, t = _rows(300, 2, 16, 2048)
    base = oracle.rms_modulate(x, s, t, 0.0)
    xf = bf16_bits_to_f32(x)
    for k in (-6, -1, 3, 9):
        xk = f32_to_bf16_bits(xf * np.float32(2.0 ** k))
        assert np.array_equal(oracle.rms_modulate(xk, s, t, 0.0), base), k


def test_batches_use_their_own_rows():
    x, s, t = _rows(400, 3, 9, 256)
    all_b = oracle.rms_modulate(x, s, t, EPS)
    for b in range(3):
        one = oracle.rms_modulate(x[b:b + 1].copy(), s[b:b + 1].copy(),
                                  t[b:b + 1].copy(), EPS)
        assert np.array_equal(all_b[b], one[0])


def test_pages_test_tolerance_against_fp32_eager():
    # the pages' mounted-path check: allclose(atol=3e-2, rtol=1e-2) against
    # the eager expression
    for hidden in (4096, 2048):
        x, s, t = _rows(500 + hidden, 1, 64, hidden)
        f = lambda a: torch.from_numpy(bf16_bits_to_f32(a))
        ref = torch.nn.functional.rms_norm(f(x), [hidden], eps=1e-6) * (1 + f(s)) + f(t)
        got = torch.from_numpy(bf16_bits_to_f32(oracle.rms_modulate(x, s, t, EPS)))
        assert torch.allclose(got, ref, atol=3e-2, rtol=1e-2)


def test_one_partial_is_the_sequential_sum():
    # with P = 1 every group lands in one partial in element order, which is
    # the plain sequential sum (a separate code path in the oracle)
    x, s, t = _rows(600, 2, 20, 1032)
    a = oracle.rms_factors(x, EPS, variant=oracle.RMS_PINNED, partials=1)
    b = oracle.rms_factors(x, EPS, variant=oracle.RMS_SEQUENTIAL)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_pinned_partials_follow_group_order():
    # Emulate the documented order with numpy binary32 scalars on a few rows:
    # groups of 8, group k -> partial k mod P, then the xor-distance tree.
    D = 1040
    x = random_bits(700, (1, 3, D), N01)
    xf = bf16_bits_to_f32(x)
    for P in (64, 256, 4):
        fac = oracle.rms_factors(x, EPS, partials=P)
        for row in range(3):
            part = [np.float32(0)] * P
            for k in range(D // 8):
                for e in range(8):
                    v = xf[0, row, 8 * k + e]
                    part[k % P] = np.float32(part[k % P] + np.float32(v * v))
            m = 1
            while m < P:
                part = [np.float32(part[j] + part[j ^ m]) for j in range(P)]
                m <<= 1
            ms = np.float32(part[0] / np.float32(D))
            r = np.float32(np.float32(1) / np.sqrt(np.float32(ms + EPS)))
            assert r.view(np.uint32) == fac[0, row].view(np.uint32), (P, row)


def test_order_variants_differ_only_at_cancellation():
    # The pinned, sequential and binary64 sums give outputs that differ by
    # more than one bf16 ulp only where |y| is small against |x r (1+s)|.
    B, L, D = 2, 256, 4096
    x, s, t = _rows(800, B, L, D, N02)
    y64, na, _ = _f64_reference(x, s, t, EPS)
    pinned = oracle.rms_modulate(x, s, t, EPS)
    cancel = np.abs(y64) < 2.0 ** -6 * na
    for v in (oracle.RMS_SEQUENTIAL, oracle.RMS_F64):
        other = oracle.rms_modulate(x, s, t, EPS, variant=v)
        d = ulp_diff(pinned, other)
        assert d[~cancel].max() <= 1
        assert (d > 0).mean() < 0.01


def test_in_place_modulation():
    x, s, t = _rows(900, 2, 11, 512)
    want = oracle.rms_modulate(x, s, t, EPS)
    xx = x.copy()
    oracle.rms_modulate(xx, s, t, EPS, out=xx)
    assert np.array_equal(xx, want)


def test_rejects_d_not_multiple_of_8():
    x = np.zeros((1, 2, 12), dtype=np.uint16)
    s = np.zeros((1, 1, 12), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.rms_modulate(x, s, s, EPS)


@pytest.mark.parametrize("mode", [oracle.GATE_FULL, oracle.GATE_BCAST])
def test_fused_residual_then_modulation_is_the_composition(mode):
    # the fused step is defined as the two operations in sequence, the
    # modulation reading the bf16-rounded updated residual
    B, L, D = 2, 17, 1032
    x = random_bits(1100, (B, L, D), N02)
    u = random_bits(1101, (B, L, D), N01)
    g = random_bits(1102, (B, L, D) if mode == oracle.GATE_FULL else (B, 1, D), N001)
    s = random_bits(1103, (B, 1, D), N001)
    t = random_bits(1104, (B, 1, D), N001)
    xo, y = oracle.gate_add_rms_modulate(x, u, g, s, t, EPS, mode)
    want_x = oracle.gate_add(x, u, g, mode)
    assert np.array_equal(xo, want_x)
    assert np.array_equal(y, oracle.rms_modulate(want_x, s, t, EPS))
    # in place on x gives the same two outputs
    xx = x.copy()
    xo2, y2 = oracle.gate_add_rms_modulate(xx, u, g, s, t, EPS, mode, x_out=xx)
    assert np.array_equal(xx, want_x) and np.array_equal(y2, y)
    # and the modulation is within the binary64 bound of the updated residual
    _check_against_f64(y, want_x, s, t, EPS)
