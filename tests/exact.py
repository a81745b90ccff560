"""Exact rational arithmetic for pinning the oracle's floating point.

Independent of NumPy's float64: values are Fractions, rounding to binary32 is
written out from IEEE 754's definition (nearest, ties to even, gradual
underflow, overflow to infinity), and the E4M3 value set is enumerated from
the OCP field definitions as Fractions.
"""
from __future__ import annotations

import struct
from fractions import Fraction

F32_MIN_EXP = -149          # exponent of the smallest subnormal quantum
F32_MANT = 23


def frac(x: float) -> Fraction:
    return Fraction(float(x))


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix to floor
    if a >= Fraction(2) ** e:
        return e
    return e - 1


def round_f32(q: Fraction, negative_zero: bool = False) -> float:
    """Round an exact rational to the nearest binary32 value, ties to even."""
    if q == 0:
        return -0.0 if negative_zero else 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = _floor_log2(a)
    qexp = max(e - F32_MANT, F32_MIN_EXP)
    m = a / (Fraction(2) ** qexp)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * (Fraction(2) ** qexp)
    if val >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(val)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def e4m3_table():
    """(code, exact value) of every finite non-negative E4M3 code, from the OCP fields."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            v = Fraction(m, 8) * Fraction(1, 64)
        else:
            v = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
        out.append((code, v))
    return out


_E4M3 = e4m3_table()


def e4m3_nearest(y: float) -> int:
    """Saturating nearest-even E4M3 code of a finite fp32 value, by exhaustive comparison."""
    a = abs(Fraction(y))
    sign = 0x80 if (y < 0 or (y == 0 and str(y).startswith("-"))) else 0
    if a >= 448:
        return 0x7E | sign
    best = None
    for code, v in _E4M3:
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | sign


def int_nearest(y: float, lo: int, hi: int) -> int:
    """Round half to even by exact comparison, then clamp."""
    a = Fraction(y)
    fl = a.numerator // a.denominator
    rem = a - fl
    r = fl + 1 if (rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1)) else fl
    return max(lo, min(hi, r))


def sqrt_f32(x: float) -> float:
    """Correctly rounded binary32 square root of a non-negative binary32 value, by exact
    comparison of squares (nearest, ties to even)."""
    a = Fraction(x)
    if a == 0:
        return x
    import math
    import numpy as _np
    y0 = _np.float32(math.sqrt(float(a)))
    cands = [y0]
    for _ in range(3):
        cands.append(_np.nextafter(cands[-1], _np.float32(_np.inf)))
        cands.insert(0, _np.nextafter(cands[0], _np.float32(0)))
    cands = [Fraction(float(c)) for c in cands]
    for lo, hi in zip(cands, cands[1:]):
        if lo * lo <= a <= hi * hi:
            mid = (lo + hi) / 2
            if a < mid * mid:
                return float(lo)
            if a > mid * mid:
                return float(hi)
            lo_bits = f32_bits(float(lo))
            return float(lo) if lo_bits % 2 == 0 else float(hi)
    raise AssertionError("sqrt bracket not found")
