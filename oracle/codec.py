"""Number codecs used by the oracle: FP8 e4m3fn, E8M0 and bf16.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the element type ``float8_e4m3fn`` and the scale type
``uint8`` E8M0 ([prequant] "Quick start"; the 1x32 E8M0 row of "Formats")
but print neither bit layout.  The layouts below are those of the public OCP
8-bit floating point specification (e4m3fn: 1 sign, 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest finite
448) and of the OCP Microscaling specification (E8M0: unsigned exponent,
bias 127, no sign, no zero, 0xFF = NaN).

Rounding readings (none is printed on the pages):
  * fp32 -> e4m3fn: round to nearest, ties to the code with an even
    mantissa; magnitudes >= 448 saturate to 448 (0x7E); the sign bit is kept,
    so -0 and negative values that round to zero give 0x80.
  * fp32 -> bf16: IEEE round to nearest, ties to even.
Inputs to the FP8 encoder must be finite; the bf16 rounding follows IEEE
overflow (values past the largest bf16 round to infinity).
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each e4m3fn code (float64; NaN for 0x7F / 0xFF).

    Closed form of the OCP layout: e = bits 6..3, m = bits 2..0;
    e == 0 -> m * 2^-9 (subnormal), otherwise (1 + m/8) * 2^(e-7);
    e == 15 and m == 7 is NaN.  Bit 7 is the sign.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_nonneg_table():
    """The 127 finite non-negative e4m3fn values, indexed by code 0..126.

    Codes 0..126 are ordered by value (the format is sign-magnitude with the
    exponent above the mantissa), which the encoder relies on; a test checks
    the ordering.
    """
    return e4m3_decode(np.arange(127))


_TABLE = e4m3_nonneg_table()


def e4m3_encode(v):
    """Encode finite values to e4m3fn codes (uint8): RNE, saturating at 448.

    ``v`` is taken exactly as given (float32 or float64 values); the caller
    performs any earlier rounding the method prescribes.
      1. sign = sign bit of v (so -0.0 keeps its sign);
      2. a = |v|; if a >= 448 the magnitude code is 126 (0x7E);
      3. otherwise the nearest table value is chosen by comparing a with the
         midpoint of its two neighbouring codes (midpoints of e4m3 values
         are exact in float64, so the comparison is exact); a tie goes to
         the even code;
      4. the sign bit is OR-ed back in.
    """
    v = np.asarray(v)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: inputs must be finite")
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8)
    lo = np.searchsorted(_TABLE, a, side="right") - 1  # _TABLE[lo] <= a
    lo = np.clip(lo, 0, 125)
    hi = lo + 1
    mid = (_TABLE[lo] + _TABLE[hi]) * 0.5
    pick_hi = (a > mid) | ((a == mid) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= E4M3_MAX, 126, mag)
    return (mag.astype(np.uint8) | (sign << 7)).astype(np.uint8)


def e8m0_decode(codes):
    """Value 2^(E-127) of E8M0 codes (float64); 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16(x):
    """float32 values -> bf16 bit patterns (uint16), round to nearest even.

    Plain form: the magnitude's two bf16 neighbours are the truncation t
    (drop the low 16 bits) and t + 1 ulp; the nearer one wins and a tie
    goes to the one with an even last bit.  Both distances are exact in
    float64.  Above the largest finite bf16 the upper neighbour is 2^128,
    i.e. infinity, as in IEEE overflow under round-to-nearest; +-inf maps to
    +-inf.  NaN is rejected.
    """
    x = np.asarray(x, dtype=np.float32)
    if np.any(np.isnan(x)):
        raise ValueError("f32_to_bf16: NaN input")
    bits = x.view(np.uint32)
    sign = (bits >> np.uint32(31)).astype(np.uint32)
    mag_bits = bits & np.uint32(0x7FFFFFFF)
    is_inf = mag_bits == np.uint32(0x7F800000)
    mag_bits = np.where(is_inf, np.uint32(0), mag_bits)
    t = mag_bits >> np.uint32(16)                 # truncated bf16 magnitude
    lo = (t << np.uint32(16)).view(np.float32).astype(np.float64)
    up = ((t + np.uint32(1)) << np.uint32(16)).view(np.float32).astype(np.float64)
    up = np.where(t + np.uint32(1) == np.uint32(0x7F80), 2.0 ** 128, up)
    a = mag_bits.view(np.float32).astype(np.float64)
    d_lo = a - lo
    d_up = up - a
    take_up = (d_up < d_lo) | ((d_up == d_lo) & ((t & np.uint32(1)) == 1))
    r = np.where(take_up, t + np.uint32(1), t)
    r = np.where(is_inf, np.uint32(0x7F80), r)
    return (r | (sign << np.uint32(15))).astype(np.uint16)
