"""Exact-arithmetic helpers for the oracle's pins (tests only).

They re-derive rounding decisions from rational arithmetic (Python
``fractions.Fraction`` and integers), independently of the oracle's numpy
code, so that a pin never re-types the formula it checks.
"""

import math
import struct
from fractions import Fraction


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def f32_value(b):
    """Exact rational value of a finite float32 bit pattern."""
    return Fraction(f32_from_bits(b))


def rn_f32(fr):
    """Round a rational to the nearest float32 (ties to even), returned as
    bit pattern of the magnitude with the sign applied.  Finite results only.

    Works on the integer significand directly: for |fr| in [2^e, 2^(e+1))
    the float32 grid spacing is 2^(max(e, -126) - 23).
    """
    if fr == 0:
        return 0
    sign = 0x80000000 if fr < 0 else 0
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix possible off-by-one from the float log2
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, -126) - 23                       # grid exponent
    scaled = a / (Fraction(2) ** q)             # significand in grid units
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    # n * 2^q -> float32 bits
    val = Fraction(n) * (Fraction(2) ** q)
    if val == 0:
        return sign
    return sign | f32_bits(float(val))


def e4m3_value(code):
    """Exact value of an e4m3fn code from the OCP closed form (NaN -> None)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        return s * Fraction(m, 512)
    return s * Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))


def e4m3_brute(fr):
    """Nearest finite e4m3fn code to a rational by scanning every code
    (ties to even mantissa, saturate at 448, sign kept, ``fr`` may be -0.0
    passed as the float)."""
    neg = (fr < 0) or (isinstance(fr, float) and math.copysign(1.0, fr) < 0)
    a = abs(Fraction(fr))
    best, best_d = None, None
    for c in range(127):
        d = abs(a - e4m3_value(c))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    if a >= 448:
        best = 126
    return best | (0x80 if neg else 0)


def rn_bf16_from_f32_bits(b):
    """bf16 bit pattern nearest (ties to even) to the float32 with bits ``b``;
    magnitudes that round past the largest bf16 give infinity."""
    sign = (b >> 16) & 0x8000
    mag = b & 0x7FFFFFFF
    if mag == 0x7F800000:
        return sign | 0x7F80
    v = f32_value(mag)
    if v == 0:
        return sign
    e = math.floor(math.log2(v.numerator) - math.log2(v.denominator))
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    q = max(e, -126) - 7                        # bf16 grid: 8 significant bits
    scaled = v / (Fraction(2) ** q)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * (Fraction(2) ** q)
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    return sign | (f32_bits(float(val)) >> 16)
