"""Pins of oracle.merge (QAT forward: W + B.A in bf16, then 128x128 fake-quant).

The special cases reduce the merge to plain quantization or to a single hand
computable element; an exact-rational re-derivation of the sequential fp32
sum checks the vectorised float64 formulation; a float64 bound checks the
merge against the exact W + B.A.
"""

from fractions import Fraction

import numpy as np

from oracle import codec, merge, quant
from tests import exact


def _bf(x):
    return codec.f32_to_bf16(np.asarray(x, dtype=np.float32))


def _inputs(n, k, r, seed):
    rng = np.random.default_rng(seed)
    w = _bf(rng.standard_normal((n, k)) * 0.02)
    b = _bf(rng.standard_normal((n, r)) * 0.01)
    a = _bf(rng.standard_normal((r, k)) * 0.01)
    return w, b, a


def test_zero_lora_reduces_to_quantize():
    w, b, a = _inputs(256, 384, 16, 0)
    zb = np.zeros_like(b)
    q, s, wdq = merge.fake_quant_merge(w, zb, a)
    q2, s2, wdq2 = quant.quantize(w, "128x128")
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(wdq, wdq2)
    za = np.zeros_like(a)
    q3, s3, _ = merge.fake_quant_merge(w, b, za)
    assert np.array_equal(q3, q2) and np.array_equal(s3, s2)


def test_single_nonzero_by_hand():
    w, _, _ = _inputs(128, 128, 4, 1)
    b = np.zeros((128, 4), np.uint16)
    a = np.zeros((4, 128), np.uint16)
    b[7, 2] = _bf(np.float32(0.375))          # 3/8
    a[2, 9] = _bf(np.float32(-0.0625))        # -1/16  -> product -3/128, exact in bf16
    wp = merge.merge_weights(w, b, a)
    expect = w.copy()
    expect[7, 9] = _bf(codec.bf16_to_f32(w[7, 9]) + np.float32(-3.0 / 128))
    assert np.array_equal(wp, expect)


def _exact_merge_element(wv, brow, acol):
    """Sequential fp32 accumulation re-derived with rationals."""
    acc = Fraction(0)
    for bv, av in zip(brow, acol):
        acc = exact.f32_value(exact.rn_f32(acc + Fraction(float(bv)) * Fraction(float(av))))
    delta = codec.bf16_to_f32(codec.f32_to_bf16(np.float32(float(acc))))    # acc is a float32 value
    s = exact.f32_value(exact.rn_f32(Fraction(float(wv)) + Fraction(float(delta))))
    return int(codec.f32_to_bf16(np.float32(float(s))))


def test_sequential_sum_matches_exact_rationals():
    rng = np.random.default_rng(2)
    n, k, r = 6, 10, 16
    # wide magnitude spread (incl. products far below fp32's normal range)
    b = _bf(rng.standard_normal((n, r)) * np.exp2(rng.integers(-70, 10, (n, r))))
    a = _bf(rng.standard_normal((r, k)) * np.exp2(rng.integers(-70, 10, (r, k))))
    w = _bf(rng.standard_normal((n, k)) * np.exp2(rng.integers(-30, 5, (n, k))))
    wp = merge.merge_weights(w, b, a)
    bf, af, wf = codec.bf16_to_f32(b), codec.bf16_to_f32(a), codec.bf16_to_f32(w)
    for i in range(n):
        for j in range(k):
            assert int(wp[i, j]) == _exact_merge_element(wf[i, j], bf[i], af[:, j]), (i, j)


def test_merge_close_to_exact_product():
    w, b, a = _inputs(64, 256, 16, 3)
    wp = codec.bf16_to_f32(merge.merge_weights(w, b, a)).astype(np.float64)
    exact_sum = (codec.bf16_to_f32(w).astype(np.float64)
                 + codec.bf16_to_f32(b).astype(np.float64) @ codec.bf16_to_f32(a).astype(np.float64))
    bf16_u = 2.0 ** -8
    babs = np.abs(codec.bf16_to_f32(b).astype(np.float64)) @ np.abs(codec.bf16_to_f32(a).astype(np.float64))
    # delta: 16 fp32 roundings + one bf16 rounding; add: one fp32 + one bf16 rounding
    bound = bf16_u * (np.abs(exact_sum) + babs) * 1.01 + 16 * 2.0 ** -24 * babs
    assert np.all(np.abs(wp - exact_sum) <= bound)


def test_order_matters_reading():
    """The reading fixes r = 0..R-1.  With products spread over many binades
    the fp32 partial sums round, and a reversed order changes some bits, so
    the exact-rational pin above does constrain the order.  (For LoRA factors
    of similar magnitude the 16 products usually sum exactly in fp32.)"""
    rng = np.random.default_rng(4)
    b = _bf(rng.standard_normal((128, 16)) * np.exp2(rng.integers(-12, 12, (128, 16))))
    a = _bf(rng.standard_normal((16, 512)) * np.exp2(rng.integers(-12, 12, (16, 512))))
    d1 = merge.lora_delta(b, a)
    d2 = merge.lora_delta(b[:, ::-1].copy(), a[::-1].copy())
    assert not np.array_equal(d1, d2)
