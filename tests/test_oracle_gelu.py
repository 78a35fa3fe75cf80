"""Pins of the oracle's tanh-GELU against what the mathematics fixes.

The oracle evaluates gelu(h) = 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3)))
in binary64 through h / (1 + exp(-2a)) and rounds once to the storage type.
Independent routes used here: the tanh form itself at 200 significant digits
(mpmath), exact rational rounding of those values (Fraction), torch's own
float64 gelu(approximate="tanh") where that evaluation is accurate, the
identity gelu(h) - gelu(-h) = h, and the limits.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
from tests.exact_round import round_rne

BF16, F16, F32 = oracle.BF16, oracle.F16, oracle.F32


def gelu_tanh_form(h, dps=200):
    """0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))) as printed, at dps digits."""
    with mpmath.workdps(dps):
        h = mpmath.mpf(h)
        a = mpmath.sqrt(2 / mpmath.pi) * (h + mpmath.mpf("0.044715") * h ** 3)
        return mpmath.mpf("0.5") * h * (1 + mpmath.tanh(a))


def _fraction(v) -> Fraction:
    """The exact value of an mpmath number (a signed integer times 2^exp)."""
    v = mpmath.mpf(v)
    sign, man, exp, _ = v._mpf_
    q = Fraction(int(man)) * (Fraction(2) ** int(exp))
    return -q if sign else q


def _exact_bits(h: float, dtype: int) -> int:
    """Correct rounding of gelu(h) to the storage type, from the tanh form
    evaluated with enough digits that no cancellation survives."""
    if np.isnan(h):
        return -1
    if np.isinf(h):
        if dtype == F32:
            return int(np.float32(h if h > 0 else -0.0).view(np.uint32))
        if dtype == BF16:
            return 0x7F80 if h > 0 else 0x8000
        return 0x7C00 if h > 0 else 0x8000
    a = abs(float(np.sqrt(2 / np.pi) * (h + 0.044715 * h ** 3)))
    if h >= 0:
        q = _fraction(gelu_tanh_form(h, dps=60))
    elif a > 4000:  # |gelu(h)| < |h| exp(-8000): far below every subnormal
        q = Fraction(0)
    else:
        # 1 + tanh(-a) is about 2 exp(-2a): keep 60 digits beyond it
        q = _fraction(gelu_tanh_form(h, dps=int(70 + 2 * a / 2.302585)))
    mant, emin, emax = {BF16: (8, -126, 127), F16: (11, -14, 15), F32: (24, -126, 127)}[dtype]
    r = round_rne(q, mant, emin, emax)
    neg = h < 0 or (h == 0 and np.signbit(h))
    if isinstance(r, float):  # infinity
        v = r
    else:
        v = float(r)
        if v == 0.0 and neg:
            v = -0.0
    if dtype == F32:
        return int(np.float32(v).view(np.uint32))
    if dtype == F16:
        return int(np.float16(v).view(np.uint16))
    return int(np.float32(v).view(np.uint32) >> 16)


def _bits(a: np.ndarray, dtype: int) -> np.ndarray:
    return a.view(np.uint32) if dtype == F32 else a


# ---- binary64 evaluation ----------------------------------------------------

def test_f64_matches_the_tanh_form_to_the_binary64_error_bound():
    xs = np.concatenate([np.linspace(-12, 12, 2401), [1e-30, -1e-30, 1e-5, -1e-5, 1e5, -40.0]])
    for h in xs:
        want = gelu_tanh_form(float(h))
        got = oracle.gelu_tanh_f64(float(h))
        a = abs(np.sqrt(2 / np.pi) * (h + 0.044715 * h ** 3))
        # each binary64 step rounds once; exp amplifies the relative error of
        # its argument 2a by |2a|
        bound = (8 + 8 * 2 * a) * 2.0 ** -53
        if want == 0:
            assert got == 0
            continue
        rel = abs((mpmath.mpf(got) - want) / want)
        assert rel <= bound, (h, got, want, rel, bound)


def test_f64_agrees_with_torch_where_its_tanh_form_is_accurate():
    # torch evaluates 0.5 h (1 + tanh(a)) directly; for h >= -3 the term
    # 1 + tanh(a) is >= 2e-3 and loses at most ~1e-13 relative
    x = torch.linspace(-3, 10, 4001, dtype=torch.float64)
    ref = torch.nn.functional.gelu(x, approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh_f64(float(v)) for v in x])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)


def test_odd_part_identity_and_limits():
    # gelu(h) - gelu(-h) = h (the logistic factors sum to one)
    for h in np.linspace(0.01, 9, 300):
        d = oracle.gelu_tanh_f64(h) - oracle.gelu_tanh_f64(-h)
        assert abs(d - h) <= 4 * 2.0 ** -52 * h, h
    assert oracle.gelu_tanh_f64(0.0) == 0.0
    assert np.signbit(oracle.gelu_tanh_f64(-0.0))
    assert oracle.gelu_tanh_f64(float("inf")) == float("inf")
    m = oracle.gelu_tanh_f64(float("-inf"))
    assert m == 0.0 and np.signbit(m)
    assert np.isnan(oracle.gelu_tanh_f64(float("nan")))
    # far right the factor is 1 to binary64 precision, far left the value
    # underflows to -0
    assert oracle.gelu_tanh_f64(50.0) == 50.0
    v = oracle.gelu_tanh_f64(-30.0)
    assert v == 0.0 and np.signbit(v)
    # the worked values of the approximation at +-1 (from the tanh form)
    assert abs(oracle.gelu_tanh_f64(1.0) - 0.8411919906082768) < 1e-15
    assert abs(oracle.gelu_tanh_f64(-1.0) + 0.15880800939172324) < 1e-15


# ---- rounding to the storage types -------------------------------------------

@pytest.mark.parametrize("dtype", [BF16, F16])
def test_every_2_byte_pattern_is_correctly_rounded(dtype):
    pats = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.gelu_tanh(pats, dtype)
    vals = (pats.astype(np.uint32) << 16).view(np.float32) if dtype == BF16 \
        else pats.view(np.float16).astype(np.float32)
    wrong = []
    for i in range(1 << 16):
        h = float(vals[i])
        want = _exact_bits(h, dtype)
        if want == -1:
            nan = (got[i] & 0x7F80) == 0x7F80 and (got[i] & 0x7F) if dtype == BF16 \
                else (got[i] & 0x7C00) == 0x7C00 and (got[i] & 0x3FF)
            if not nan:
                wrong.append((i, h, int(got[i]), "nan"))
        elif int(got[i]) != want:
            wrong.append((i, h, int(got[i]), want))
    assert not wrong, wrong[:10]


def test_binary32_outputs_are_correctly_rounded():
    rng = np.random.default_rng(77)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 3,
                        np.float32([-9.5, -7.25, 0.0, -0.0, 1e-38, -1e-40, 3e38])])
    got = _bits(oracle.gelu_tanh(x, F32), F32)
    for i, h in enumerate(x):
        assert int(got[i]) == _exact_bits(float(h), F32), (i, float(h))


def test_bias_is_added_in_binary32_first():
    # h = fl32(x + b): pairs whose sum is inexact in binary32 must use the
    # rounded sum, not the exact one
    x = np.float32([1.0, 3.0, -2.0, 0.5])
    b = np.float32([2.0 ** -24 + 2.0 ** -30, 1e-7, -2.0 ** -22, 0.25])
    got = oracle.gelu_tanh(x.reshape(1, 4), F32, bias=b)[0]
    for i in range(4):
        h = np.float32(x[i] + b[i])
        assert got[i].view(np.uint32) == _exact_bits(float(h), F32)
    # rows share the bias row
    xs = np.stack([x, -x, 2 * x]).astype(np.float32)
    got = oracle.gelu_tanh(xs, F32, bias=b)
    for r in range(3):
        for i in range(4):
            h = np.float32(xs[r, i] + b[i])
            assert got[r, i].view(np.uint32) == _exact_bits(float(h), F32)


def test_exhaustive_cases_include_double_rounding_traps():
    # inputs whose binary64 gelu, rounded to nearest binary32, lands exactly
    # on a midpoint of the 2-byte format although the binary64 value is not
    # that midpoint: rounding to nearest twice errs exactly there, so the
    # exhaustive tests above pin the oracle's round-to-odd step
    pats = np.arange(1 << 16, dtype=np.uint16)
    traps = {}
    for dtype in (BF16, F16):
        vals = (pats.astype(np.uint32) << 16).view(np.float32) if dtype == BF16 \
            else pats.view(np.float16).astype(np.float32)
        n = 0
        for h in vals:
            if not np.isfinite(h):
                continue
            y = oracle.gelu_tanh_f64(float(h))
            f = np.float32(y)
            if float(f) == y or not np.isfinite(f):
                continue
            w = int(f.view(np.uint32))
            if dtype == BF16 and (w & 0xFFFF) == 0x8000:
                n += 1
            if dtype == F16 and abs(float(f)) >= 2.0 ** -14 and (w & 0x1FFF) == 0x1000:
                n += 1
        traps[dtype] = n
    assert traps[F16] >= 1, traps


def _near_midpoint(y: np.ndarray, dtype: int, ulps: int = 2) -> np.ndarray:
    """Mask of binary64 results whose nearest binary32 lies within `ulps`
    binary32 ulps of a midpoint between two neighbours of the 2-byte format
    (where a wrong last rounding step shows)."""
    with np.errstate(over="ignore", invalid="ignore"):
        f = y.astype(np.float32)
        return _near_midpoint_bits(f, dtype, ulps)


def _near_midpoint_bits(f: np.ndarray, dtype: int, ulps: int) -> np.ndarray:
    w = f.view(np.uint32).astype(np.int64)
    finite = np.isfinite(f)
    if dtype == BF16:  # bf16 rounds binary32 at bit 16 at every magnitude
        return finite & (np.abs((w & 0xFFFF) - 0x8000) <= ulps)
    a = np.abs(f.astype(np.float64))
    normal = finite & (a >= 2.0 ** -14) & (np.abs((w & 0x1FFF) - 0x1000) <= ulps)
    # binary16 subnormals: midpoints are the odd multiples of 2^-25
    r = a * 2.0 ** 25
    k = np.rint(r)
    ulp = np.spacing(np.abs(f)).astype(np.float64) * 2.0 ** 25
    sub = finite & (a < 2.0 ** -14) & (k % 2 == 1) & (np.abs(r - k) <= ulps * ulp)
    return normal | sub


@pytest.mark.parametrize("dtype", [BF16, F16])
def test_results_near_midpoints_are_correctly_rounded(dtype):
    # the inputs of the 2-byte format whose gelu lies next to a rounding
    # midpoint of that format, chosen with numpy's float64 evaluation of the
    # logistic form; the expected bits come from the tanh form at high
    # precision
    pats = np.arange(1 << 16, dtype=np.uint16)
    vals = (pats.astype(np.uint32) << 16).view(np.float32) if dtype == BF16 \
        else pats.view(np.float16).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        h = vals.astype(np.float64)
        a = np.sqrt(2 / np.pi) * (h + 0.044715 * h ** 3)
        y = h / (1.0 + np.exp(-2.0 * a))
    pick = np.flatnonzero(_near_midpoint(y, dtype) & np.isfinite(h))
    assert len(pick) >= (100 if dtype == BF16 else 20), len(pick)
    got = oracle.gelu_tanh(pats[pick], dtype)
    for j, i in enumerate(pick):
        assert int(got[j]) == _exact_bits(float(vals[i]), dtype), (int(i), float(vals[i]))
