"""Pins of the QAT-backward oracle (oracle/lora_grad.py), CPU only.

The gradients are checked against central finite differences of the loss
L(B, A) = sum(dY * Y), Y = X . (W + B.A)^T (the fake-quant passed straight
through), which is linear in B and in A, so the differences are exact up to
float64 rounding; against the special cases B = 0 (dA = 0) and dY = 0; and
the column-sampled variant against the full one.
"""

import numpy as np

from oracle import lora_grad
from oracle.codec import bf16_to_f32, f32_to_bf16


def _bf16(rng, shape, scale=1.0):
    return f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def _loss(dy, x, w, b, a):
    y = x @ (w + b @ a).T
    return float(np.sum(dy * y))


def test_finite_differences():
    rng = np.random.default_rng(0)
    m, n, k, r = 5, 6, 7, 3
    dyb, xb, wb, bb, ab = (_bf16(rng, s) for s in ((m, n), (m, k), (n, k), (n, r), (r, k)))
    dy, x, w, b, a = (bf16_to_f32(t).astype(np.float64) for t in (dyb, xb, wb, bb, ab))
    gb, ga = lora_grad.lora_grads(dyb, xb, bb, ab)
    h = 0.5
    for (i, j) in [(0, 0), (3, 1), (5, 2)]:
        bp, bm = b.copy(), b.copy()
        bp[i, j] += h
        bm[i, j] -= h
        fd = (_loss(dy, x, w, bp, a) - _loss(dy, x, w, bm, a)) / (2 * h)
        assert abs(fd - gb[i, j]) <= 1e-12 * (1 + abs(fd))
    for (i, j) in [(0, 0), (1, 4), (2, 6)]:
        ap, am = a.copy(), a.copy()
        ap[i, j] += h
        am[i, j] -= h
        fd = (_loss(dy, x, w, b, ap) - _loss(dy, x, w, b, am)) / (2 * h)
        assert abs(fd - ga[i, j]) <= 1e-12 * (1 + abs(fd))


def test_special_cases():
    rng = np.random.default_rng(1)
    m, n, k, r = 8, 16, 24, 4
    dyb, xb, bb, ab = (_bf16(rng, s) for s in ((m, n), (m, k), (n, r), (r, k)))
    gb, ga = lora_grad.lora_grads(dyb, xb, np.zeros_like(bb), ab)
    assert np.all(ga == 0) and np.any(gb != 0)
    gb, ga = lora_grad.lora_grads(np.zeros_like(dyb), xb, bb, ab)
    assert np.all(gb == 0) and np.all(ga == 0)


def test_columns_match_full():
    rng = np.random.default_rng(2)
    m, n, k, r = 32, 40, 48, 5
    dyb, xb, bb, ab = (_bf16(rng, s) for s in ((m, n), (m, k), (n, r), (r, k)))
    gb, ga = lora_grad.lora_grads(dyb, xb, bb, ab)
    rows, cols = np.array([0, 7, 39]), np.array([1, 30, 47])
    sb, sa = lora_grad.lora_grads_columns(dyb, xb, bb, ab, rows, cols)
    assert np.allclose(sb, gb[rows], rtol=1e-12, atol=0)
    assert np.allclose(sa, ga[:, cols], rtol=1e-12, atol=0)
