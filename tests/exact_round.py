"""Exact reference arithmetic for the oracle's pins: IEEE round-to-nearest-even
done on rationals (``fractions.Fraction``), and helpers for bf16 bit patterns.

Nothing here calls the oracle; it is an independent route to the same
results (exact rational arithmetic and library conversions instead of the
oracle's bit manipulation).
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import torch

INF = float("inf")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 patterns with torch (library conversion)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Narrow binary32 with torch's round-to-nearest-even (library)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 patterns -> integers whose difference counts representable values
    between two finite bf16 numbers (+0 and -0 both map to 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan(bits: np.ndarray) -> np.ndarray:
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ordered(a) - ordered(b)|; NaN vs NaN counts 0, NaN vs non-NaN a huge
    number. Infinities are the ends of the ordered range."""
    d = np.abs(ordered(a) - ordered(b))
    na, nb = is_nan(a), is_nan(b)
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, 1 << 20, d)


# Storage-type aware forms: uint16 patterns for bf16 (0) and binary16 (1),
# float32 arrays (compared through their uint32 patterns) for binary32 (2).
_LAYOUT = {0: (0x8000, 0x7F80, 0x007F), 1: (0x8000, 0x7C00, 0x03FF),
           2: (0x80000000, 0x7F800000, 0x007FFFFF)}


def _as_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if dtype == 2:
        return a.astype(np.float32, copy=False).view(np.uint32).astype(np.int64)
    return a.astype(np.uint16, copy=False).astype(np.int64)


def is_nan_typed(a: np.ndarray, dtype: int) -> np.ndarray:
    sign, exp, frac = _LAYOUT[dtype]
    b = _as_bits(a, dtype)
    return ((b & exp) == exp) & ((b & frac) != 0)


def ulp_diff_typed(a: np.ndarray, b: np.ndarray, dtype: int) -> np.ndarray:
    """ulp_diff for any storage type: the count of representable values
    between a and b (+0 and -0 both 0; NaN vs NaN 0; NaN vs other huge)."""
    sign = _LAYOUT[dtype][0]
    def order(v):
        bits = _as_bits(v, dtype)
        mag = bits & (sign - 1)
        return np.where(bits & sign, -mag, mag)
    d = np.abs(order(a) - order(b))
    na, nb = is_nan_typed(a, dtype), is_nan_typed(b, dtype)
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, 1 << 40, d)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if a < Fraction(2) ** e:
        e -= 1
    return e


def round_rne(q: Fraction, mant_bits: int, emin: int = -126, emax: int = 127):
    """Round the exact rational q to a binary format with ``mant_bits``
    significand bits (hidden bit included), normal exponents [emin, emax] and
    gradual underflow; ties to even; overflow to +-inf. Returns a Fraction or
    +-inf (zero results are returned as Fraction(0); the caller decides the
    sign of zero)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * INF
    return sign * r


def f32_value(f: float) -> Fraction:
    return Fraction(float(np.float32(f)))


def fraction_to_f32(q) -> np.float32:
    if isinstance(q, float):
        return np.float32(q)
    return np.float32(float(q))  # q is already on the binary32 grid


def exact_gate_add_bits(xb: int, ub: int, gb: int) -> int:
    """One element of out = bf16(fl32(x + fl32(u*g))) by exact rationals,
    specials by the IEEE rules. Returns the bf16 pattern (NaN as 0x7FC0)."""
    x = float(bf16_bits_to_f32(np.array([xb], dtype=np.uint16))[0])
    u = float(bf16_bits_to_f32(np.array([ub], dtype=np.uint16))[0])
    g = float(bf16_bits_to_f32(np.array([gb], dtype=np.uint16))[0])
    # binary32 product
    if any(v != v for v in (x, u, g)):
        return 0x7FC0
    if (u in (INF, -INF) and g == 0) or (g in (INF, -INF) and u == 0):
        return 0x7FC0
    if u in (INF, -INF) or g in (INF, -INF):
        p = INF if (u > 0) == (g > 0) else -INF
        p_negzero = False
    else:
        pq = round_rne(Fraction(u) * Fraction(g), 24)
        if pq == 0:
            p = 0.0
            p_negzero = (struct.pack(">f", u)[0] >> 7) ^ (struct.pack(">f", g)[0] >> 7)
        else:
            p = pq if isinstance(pq, float) else pq
            p_negzero = False
    # binary32 sum
    if isinstance(p, float) and p in (INF, -INF):
        if x in (INF, -INF) and x != p:
            return 0x7FC0
        s = p
    elif x in (INF, -INF):
        s = x
    else:
        pv = Fraction(0) if (isinstance(p, float) and p == 0.0) else p
        sq = round_rne(Fraction(x) + pv, 24)
        if isinstance(sq, float):
            s = sq
        elif sq == 0:
            x_neg = struct.pack(">f", x)[0] >> 7
            s = -0.0 if (x == 0 and x_neg and (pv == 0 and p_negzero)) else 0.0
        else:
            s = sq
    # bf16 rounding of the binary32 sum
    if isinstance(s, float):
        if s in (INF, -INF):
            return 0xFF80 if s < 0 else 0x7F80
        return 0x8000 if struct.pack(">f", s)[0] >> 7 else 0x0000
    bq = round_rne(s, 8)
    if isinstance(bq, float):
        return 0xFF80 if bq < 0 else 0x7F80
    if bq == 0:
        return 0x8000 if s < 0 else 0x0000
    return int(f32_to_bf16_bits(np.array([float(bq)], dtype=np.float32))[0])
