"""NVFP4 prequantization (oracle): packed FP4 values with FP8 block scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page ([prequant] "Formats") names the format ``nvfp4`` as packed FP4
values with FP8 block scales, served at FP4, and says no more.  Readings:
  * FP4 element: E2M1 of the public OCP Microscaling specification -- sign,
    2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5,
    2, 3, 4, 6; no Inf or NaN.  Two codes per byte: element 2j of a row in
    the low nibble of byte j, element 2j + 1 in the high nibble.
  * block: 16 consecutive elements of a row (the block length of the
    NVFP4 format the name refers to); its scale is an e4m3fn code (the
    "FP8" of the table).
  * a second, per-tensor fp32 scale g lets the e4m3 block scales cover the
    tensor's range: g = RN32(A / 2688), A = max |x| over the tensor,
    2688 = 448 * 6 (largest e4m3 times largest E2M1).
  * block scale S = e4m3(RN32(a / RN32(6 * g))) with a the block's amax
    (round to nearest even, saturating at 448, as for the FP8 codes);
    S = 0 when g = 0 (an all-zero tensor).
  * block multiplier m = RN32(e4m3(S) * g); element code
    c = e2m1(RN32(x / m)): nearest E2M1 magnitude, a tie to the code with an
    even mantissa bit, magnitudes above 6 saturate to 6, the sign bit of x
    is kept; a block with m = 0 gets the sign bit alone (value +-0).
  * dequantized value RN_bf16(RN32(e2m1(c) * m)).
A batch of tensors stacked along the rows (rows_per_tensor rows each) has
one A and one g per tensor.
"""

import numpy as np

from .codec import bf16_to_f32, e4m3_decode, e4m3_encode, f32_to_bf16

BLOCK = 16
E2M1_MAX = 6.0
GLOBAL_DIVISOR = 448.0 * 6.0

# E2M1 magnitudes by code 0..7 from the layout: e = bits 2..1, m = bit 0;
# e == 0 -> m * 0.5 (subnormal), otherwise (1 + m/2) * 2^(e-1).
_E2M1_MAG = np.array([(m * 0.5) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
                      for e in range(4) for m in range(2)], dtype=np.float64)


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code 0..15 (float64); bit 3 is the sign."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where((c >> 3) & 1, -1.0, 1.0) * _E2M1_MAG[c & 7]


def e2m1_encode(v):
    """Encode finite values to E2M1 codes (uint8 0..15): nearest magnitude,
    ties to the even code, saturating at 6, sign bit kept.

    The magnitude is compared with the midpoint of its two neighbouring
    codes (exact in float64); codes are ordered by value."""
    v = np.asarray(v)
    if not np.all(np.isfinite(v)):
        raise ValueError("e2m1_encode: inputs must be finite")
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.uint8)
    lo = np.clip(np.searchsorted(_E2M1_MAG, a, side="right") - 1, 0, 6)
    hi = lo + 1
    mid = (_E2M1_MAG[lo] + _E2M1_MAG[hi]) * 0.5
    pick_hi = (a > mid) | ((a == mid) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= E2M1_MAX, 7, mag)
    return (mag.astype(np.uint8) | (sign << 3)).astype(np.uint8)


def pack(codes):
    """[R, C] codes 0..15 -> [R, C/2] bytes, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    """[R, C/2] bytes -> [R, C] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def _check(rows, cols, rows_per_tensor):
    if cols % BLOCK or rows_per_tensor < 1 or rows % rows_per_tensor:
        raise ValueError("nvfp4: cols % 16 == 0 and rows % rows_per_tensor == 0 required")


def tensor_amax(x_bits, rows_per_tensor):
    """A = max |x| of each tensor of the stack, float32 [T] (exact)."""
    xf = bf16_to_f32(np.ascontiguousarray(x_bits, dtype=np.uint16))
    rows, cols = xf.shape
    _check(rows, cols, rows_per_tensor)
    t = rows // rows_per_tensor
    if xf.size == 0:
        return np.zeros(t, dtype=np.float32)
    return np.abs(xf.reshape(t, -1)).max(axis=1).astype(np.float32)


def global_scale(amax):
    """g = RN32(A / 2688): one IEEE float32 division."""
    return (np.asarray(amax, dtype=np.float32) / np.float32(GLOBAL_DIVISOR)).astype(np.float32)


def quantize(x_bits, rows_per_tensor=None, amax=None):
    """Quantize a bf16 matrix (uint16 bits [R, C]) to NVFP4.

    rows_per_tensor: rows of each stacked tensor (default: all rows, one
    tensor).  amax: optional per-tensor A to use instead of the measured one.
    Returns (packed uint8 [R, C/2], block_scale uint8 e4m3 codes [R, C/16],
    g float32 [T], A float32 [T], xdq bf16 bits [R, C])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    rpt = rows if rows_per_tensor is None else rows_per_tensor
    if rows == 0:
        rpt = max(rpt, 1)
    _check(rows, cols, rpt)
    A = tensor_amax(x_bits, rpt) if amax is None else np.asarray(amax, dtype=np.float32)
    g = global_scale(A)
    xf = bf16_to_f32(x_bits)
    xb = xf.reshape(rows, cols // BLOCK, BLOCK)
    a = np.abs(xb).max(axis=-1) if xb.size else np.zeros((rows, cols // BLOCK), np.float32)
    g_rows = np.repeat(g, rpt)[:, None]                               # g of each row's tensor
    t = (np.float32(6.0) * g_rows).astype(np.float32)                 # RN32(6 g)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (a / t).astype(np.float32)                            # RN32(a / t)
    ratio = np.where(t == 0, np.float32(0.0), ratio)
    S = e4m3_encode(ratio)
    m = (e4m3_decode(S).astype(np.float32) * g_rows).astype(np.float32)   # RN32(e4m3(S) g)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (xb / m[..., None]).astype(np.float32)                  # RN32(x / m)
    quot = np.where(np.broadcast_to((m == 0)[..., None], xb.shape), xb * np.float32(0.0), quot)
    codes = e2m1_encode(quot).reshape(rows, cols)
    packed = pack(codes) if rows else np.zeros((0, cols // 2), np.uint8)
    return packed, S.astype(np.uint8), g, A, dequantize(packed, S, g, rpt)


def dequantize_f32(packed, block_scale, g, rows_per_tensor):
    """RN32(e2m1(c) * m) as float32 [R, C], m = RN32(e4m3(S) * g)."""
    codes = unpack(packed)
    rows, cols = codes.shape
    g_rows = np.repeat(np.asarray(g, dtype=np.float32), rows_per_tensor)[:, None]
    m = (e4m3_decode(block_scale).astype(np.float32) * g_rows).astype(np.float32)
    mm = np.repeat(m, BLOCK, axis=1)
    return (e2m1_decode(codes).astype(np.float32) * mm).astype(np.float32)


def dequantize(packed, block_scale, g, rows_per_tensor):
    """RN_bf16(RN32(e2m1(c) * m)) as bf16 bits [R, C]."""
    return f32_to_bf16(dequantize_f32(packed, block_scale, g, rows_per_tensor))
