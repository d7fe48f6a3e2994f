"""Fine-grained block-wise FP8 quantization (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * weights and activations are split into sub-matrices, each with its own
    scaling factor, so an outlier only affects its own block
    ([DSV3-Blog5] "The Solution: Block-Wise Quantization");
  * weights use 128x128 blocks with an fp32 "scale inverse" used for
    dequantization; activations are quantized online per token in groups
    of 128 channels ([FP8-DSV3-ru] "Как FP8 встроен в DeepSeek V3",
    "Почему обычное округление не подходит", "Почему FP8 требует scale
    factors");
  * MXFP8 is 1x32 block FP8 with E8M0 scales, stored as a float8_e4m3fn
    weight plus a uint8 ``weight_scale_inv`` ([prequant] "Quick start",
    "Formats").

Readings taken where the pages are silent:
  * the scale comes from the block's largest magnitude (amax);
  * fp32 kinds store the dequantization multiplier s = RN32(amax / 448) and
    each element is encoded as e4m3(RN32(x / s)) -- an fp32 quotient, then
    the FP8 rounding; an all-zero block has s = 0 and its codes are +-0 by
    the sign of x;
  * E8M0 "ceil" (default): the smallest power of two 2^X, X in [-127, 127],
    with amax <= 448 * 2^X, so the block maximum never saturates; E8M0
    "floor": the OCP MX rule X = floor(log2 amax) - 8, clamped to
    [-127, 127] (elements above 448 * 2^X saturate); amax == 0 gives
    X = -127 under both rules; elements are encoded as e4m3(x * 2^-X),
    an exact scaling;
  * blocks run along the last (contiguous) dimension; 128x128 blocks are
    aligned at (0, 0); scale arrays are row-major:
      "1x32"    uint8 codes E = X + 127, shape [R, C/32]
      "1x128"   float32 s, shape [R, C/128]
      "128x128" float32 s, shape [R/128, C/128]
  * the fake-quant (dequantized) output is RN_bf16(RN32(decode(q) * scale)).
"""

import numpy as np

from .codec import (E4M3_MAX, bf16_to_f32, e4m3_decode, e4m3_encode,
                    e8m0_decode, f32_to_bf16)

KINDS = ("1x32", "1x128", "128x128")
BLOCK_SHAPE = {"1x32": (1, 32), "1x128": (1, 128), "128x128": (128, 128)}


def _check_shape(rows, cols, kind):
    br, bc = BLOCK_SHAPE[kind]
    if rows % br or cols % bc:
        raise ValueError(f"shape {rows}x{cols} is not a multiple of the {kind} block")


def block_view(x, kind):
    """[R, C] -> [R/br, C/bc, br*bc]: one row per block, block elements last."""
    br, bc = BLOCK_SHAPE[kind]
    r, c = x.shape
    return (x.reshape(r // br, br, c // bc, bc)
             .transpose(0, 2, 1, 3)
             .reshape(r // br, c // bc, br * bc))


def unblock(xb, rows, cols, kind):
    """Inverse of ``block_view``."""
    br, bc = BLOCK_SHAPE[kind]
    return (xb.reshape(rows // br, cols // bc, br, bc)
              .transpose(0, 2, 1, 3)
              .reshape(rows, cols))


def block_amax(xf, kind):
    """Largest magnitude of each block, shape [R/br, C/bc] (float32, exact)."""
    return np.abs(block_view(xf, kind)).max(axis=-1)


def fp32_scale(amax):
    """s = RN32(amax / 448): one IEEE float32 division (numpy float32 '/')."""
    return (np.asarray(amax, dtype=np.float32) / np.float32(E4M3_MAX)).astype(np.float32)


_POW2_THRESH = E4M3_MAX * np.exp2(np.arange(-127, 128, dtype=np.float64))  # 448*2^X, exact


def e8m0_exponent(amax, rule="ceil"):
    """Block exponent X (int64) of the E8M0 scale 2^X.

    ceil : smallest X in [-127, 127] with amax <= 448 * 2^X (exact float64
           comparisons against the 255 thresholds 448 * 2^X); a block too large
           for X = 127 would clamp to 127 (no bf16 value reaches it).
    floor: X = floor(log2 amax) - 8 (8 = exponent of the largest e4m3 binade),
           from frexp, which is exact; clamped to [-127, 127]; amax == 0 -> -127.
    """
    a = np.asarray(amax, dtype=np.float64)
    if rule == "ceil":
        idx = np.searchsorted(_POW2_THRESH, a, side="left")  # first threshold >= a
        return np.minimum(idx, 254).astype(np.int64) - 127
    if rule == "floor":
        _, e = np.frexp(a)                 # a = m * 2^e, m in [0.5, 1)
        x = (e.astype(np.int64) - 1) - 8   # floor(log2 a) = e - 1
        x = np.where(a == 0, -127, x)
        return np.clip(x, -127, 127)
    raise ValueError(f"unknown E8M0 rule {rule!r}")


def quantize(x_bits, kind, rule="ceil"):
    """Quantize a bf16 matrix (uint16 bits, [R, C]) block-wise to e4m3fn.

    Returns (q uint8 [R, C], scale, xdq uint16 [R, C]) where ``scale`` is
    uint8 E8M0 codes for "1x32" and float32 s for the fp32 kinds, and ``xdq``
    is the fake-quant output (see ``dequantize``).
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    _check_shape(rows, cols, kind)
    xf = bf16_to_f32(x_bits)
    xb = block_view(xf, kind)
    amax = np.abs(xb).max(axis=-1)
    if kind == "1x32":
        X = e8m0_exponent(amax, rule)
        v = xb.astype(np.float64) * np.exp2(-X.astype(np.float64))[..., None]  # exact
        qb = e4m3_encode(v)
        scale = (X + 127).astype(np.uint8)
    else:
        s = fp32_scale(amax)
        with np.errstate(divide="ignore", invalid="ignore"):
            quot = (xb / s[..., None]).astype(np.float32)      # RN32(x / s)
        zero_blk = np.broadcast_to((s == 0)[..., None], xb.shape)
        quot = np.where(zero_blk, xb, quot)   # s == 0: the block is all +-0
        qb = e4m3_encode(quot)
        scale = s
    q = unblock(qb, rows, cols, kind)
    return q, scale, dequantize(q, scale, kind)


def scale_multiplier(scale, kind, rows, cols):
    """Per-element float32 scale value broadcast to [R, C]."""
    br, bc = BLOCK_SHAPE[kind]
    if kind == "1x32":
        sv = e8m0_decode(scale).astype(np.float32)   # 2^X, exact in float32
    else:
        sv = np.asarray(scale, dtype=np.float32)
    return np.repeat(np.repeat(sv, br, axis=0), bc, axis=1)[:rows, :cols]


def dequantize_f32(q, scale, kind):
    """RN32(decode(q) * scale) as float32 [R, C] (the dequantized operand).

    IEEE float32 multiply: a product beyond the largest float rounds to
    +-inf (possible only for E8M0 blocks whose amax is within one e4m3 step
    of the bf16 maximum)."""
    rows, cols = q.shape
    dq = e4m3_decode(q).astype(np.float32)           # exact
    with np.errstate(over="ignore"):
        return (dq * scale_multiplier(scale, kind, rows, cols)).astype(np.float32)


def dequantize(q, scale, kind):
    """Fake-quant output RN_bf16(RN32(decode(q) * scale)) as bf16 bits."""
    return f32_to_bf16(dequantize_f32(q, scale, kind))
