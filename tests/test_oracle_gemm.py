"""Pins of oracle.gemm (block-scaled GEMM, grouped GEMM, error metric).

Exact rational brute force on tiny shapes, integer-valued products that
fp32 sums exactly, an identity operand, scale changes confined to one block
(they catch scale indexing and transposition slips), and the grouped GEMM
against separately built per-group problems.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, gemm, quant


def _bf(x):
    return codec.f32_to_bf16(np.asarray(x, dtype=np.float32))


def _quantized(rows, cols, kind, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = _bf(rng.standard_normal((rows, cols)) * scale)
    q, s, _ = quant.quantize(x, kind)
    return q, s


def test_tiny_gemm_against_exact_rationals():
    for (ka, kb, m, n, k) in (("1x128", "128x128", 3, 128, 256), ("1x32", "1x32", 5, 4, 64)):
        aq, as_ = _quantized(m, k, ka, 1)
        bq, bs = _quantized(n, k, kb, 2, 0.02)
        ahat = gemm.dequant_operand(aq, as_, ka)
        bhat = gemm.dequant_operand(bq, bs, kb)
        y32 = gemm.gemm_ref32(aq, as_, ka, bq, bs, kb)
        y64 = gemm.gemm_ref64(aq, as_, ka, bq, bs, kb)
        for i in range(m):
            for j in range(n):
                ex = sum(Fraction(float(ahat[i, t])) * Fraction(float(bhat[j, t])) for t in range(k))
                absum = sum(abs(float(ahat[i, t]) * float(bhat[j, t])) for t in range(k))
                assert abs(float(y64[i, j]) - float(ex)) <= k * 2.0 ** -53 * absum * 1.01
                assert abs(float(y32[i, j]) - float(ex)) <= k * 2.0 ** -24 * absum * 1.01


def test_ref32_sums_in_k_order():
    """The fp32 reference adds the rounded products in the order k = 0..K-1:
    with products 1, 2^24, -2^24 (in that order) the running sum rounds
    1 + 2^24 to 2^24 (ties to even) and ends at 0, where any other order of
    the same three terms, or float64, gives 1.  The operands are MXFP8: code
    0x38 is 1.0 and 0xB8 is -1.0; E8M0 code 127 + X scales by 2^X."""
    k = 96
    aq = np.zeros((1, k), np.uint8)
    bq = np.zeros((1, k), np.uint8)
    aq[0, [0, 32, 64]] = [0x38, 0x38, 0xB8]
    bq[0, [0, 32, 64]] = 0x38
    sa = np.array([[127, 127 + 24, 127 + 24]], np.uint8)
    sb = np.full((1, 3), 127, np.uint8)
    assert gemm.gemm_ref32(aq, sa, "1x32", bq, sb, "1x32")[0, 0] == 0.0
    assert gemm.gemm_ref64(aq, sa, "1x32", bq, sb, "1x32")[0, 0] == 1.0
    # the later term first: 2^24 + (-2^24) + 1 = 1 in any precision
    aq2 = aq.copy()
    aq2[0, [0, 64]] = aq[0, [64, 0]]
    sa2 = np.array([[127 + 24, 127 + 24, 127]], np.uint8)
    assert gemm.gemm_ref32(aq2, sa2, "1x32", bq, sb, "1x32")[0, 0] == 1.0


def test_dequantized_operand_is_code_times_scale():
    aq, as_ = _quantized(4, 256, "1x128", 3)
    ahat = gemm.dequant_operand(aq, as_, "1x128")
    for i in range(4):
        for t in range(0, 256, 17):
            want = np.float32(codec.e4m3_decode(aq[i, t])) * as_[i, t // 128]
            assert ahat[i, t] == want


def test_integer_valued_exact():
    """Codes of small integers with unit scales: every partial sum is an
    integer below 2^24, so the fp32 result is exact."""
    rng = np.random.default_rng(4)
    ints = np.array([0, 1, 2, 3, 4, -1, -2, -3, -4], dtype=np.float64)
    m, n, k = 16, 128, 512
    av = rng.choice(ints, size=(m, k))
    bv = rng.choice(ints, size=(n, k))
    aq = codec.e4m3_encode(av)
    bq = codec.e4m3_encode(bv)
    y = gemm.gemm_ref32(aq, np.ones((m, k // 128), np.float32), "1x128",
                        bq, np.ones((n // 128, k // 128), np.float32), "128x128")
    assert np.array_equal(y.astype(np.float64), av @ bv.T)
    y2 = gemm.gemm_ref32(aq, np.full((m, k // 32), 127, np.uint8), "1x32",
                         bq, np.full((n, k // 32), 127, np.uint8), "1x32")
    assert np.array_equal(y2.astype(np.float64), av @ bv.T)


def test_identity_b_returns_a_hat():
    aq, as_ = _quantized(8, 128, "1x128", 5)
    bq = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(bq, 0x38)                       # 1.0
    y = gemm.gemm_ref32(aq, as_, "1x128", bq, np.ones((1, 1), np.float32), "128x128")
    assert np.array_equal(y, gemm.dequant_operand(aq, as_, "1x128"))


@pytest.mark.parametrize("which", ["a_kblock", "b_nblock", "b_kblock"])
def test_scale_change_confined_to_one_block(which):
    """Doubling one scale changes exactly the outputs that block feeds, by
    exactly that block's partial product."""
    m, n, k = 8, 256, 512
    aq, as_ = _quantized(m, k, "1x128", 6)
    bq, bs = _quantized(n, k, "128x128", 7, 0.02)
    base = gemm.gemm_ref64(aq, as_, "1x128", bq, bs, "128x128")
    as2, bs2 = as_.copy(), bs.copy()
    if which == "a_kblock":
        as2[:, 2] *= 2
        ahat = gemm.dequant_operand(aq, as_, "1x128").astype(np.float64)
        bhat = gemm.dequant_operand(bq, bs, "128x128").astype(np.float64)
        extra = ahat[:, 256:384] @ bhat[:, 256:384].T
    elif which == "b_nblock":
        bs2[1, :] *= 2
        ahat = gemm.dequant_operand(aq, as_, "1x128").astype(np.float64)
        bhat = gemm.dequant_operand(bq, bs, "128x128").astype(np.float64)
        extra = np.zeros_like(base)
        extra[:, 128:256] = ahat @ bhat[128:256].T
    else:
        bs2[0, 3] *= 2
        ahat = gemm.dequant_operand(aq, as_, "1x128").astype(np.float64)
        bhat = gemm.dequant_operand(bq, bs, "128x128").astype(np.float64)
        extra = np.zeros_like(base)
        extra[:, 0:128] = ahat[:, 384:512] @ bhat[0:128, 384:512].T
    new = gemm.gemm_ref64(aq, as2, "1x128", bq, bs2, "128x128")
    assert np.allclose(new - base, extra, rtol=1e-12, atol=1e-12 * np.abs(base).max())
    # only the fed outputs moved
    moved = np.abs(new - base) > 0
    if which != "a_kblock":
        assert not moved[:, (np.abs(extra) == 0).all(axis=0)].any()


def test_entries_match_full_product():
    aq, as_ = _quantized(64, 512, "1x128", 8)
    bq, bs = _quantized(256, 512, "128x128", 9, 0.02)
    full = gemm.gemm_ref64(aq, as_, "1x128", bq, bs, "128x128")
    rows = np.array([0, 5, 63, 17]); cols = np.array([255, 0, 128, 77])
    got = gemm.gemm_entries(gemm.dequant_operand(aq, as_, "1x128"),
                            gemm.dequant_operand(bq, bs, "128x128"), rows, cols)
    assert np.allclose(got, full[rows, cols], rtol=0, atol=1e-12)


def test_grouped_equals_separate_dense_problems():
    rng = np.random.default_rng(10)
    g, n, k = 5, 128, 256
    sizes = [3, 0, 1, 130, 7]                        # includes an empty group and M_g = 1
    off = np.concatenate([[0], np.cumsum(sizes)])
    aq, as_ = _quantized(int(off[-1]), k, "1x128", 11)
    bqs, bss = [], []
    for e in range(g):
        bq, bs = _quantized(n, k, "1x32", 20 + e, 0.02 * (e + 1))
        bqs.append(bq); bss.append(bs)
    bq_all = np.stack(bqs); bs_all = np.stack(bss)
    out = gemm.grouped_gemm_ref(aq, as_, "1x128", bq_all, bs_all, "1x32", off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        want = gemm.gemm_ref32(aq[lo:hi], as_[lo:hi], "1x128", bqs[e], bss[e], "1x32")
        assert out[e].shape == (sizes[e], n)
        assert np.array_equal(out[e], want)
    # a permuted expert stack must change the result of a nonempty group
    out2 = gemm.grouped_gemm_ref(aq, as_, "1x128", bq_all[::-1].copy(), bs_all[::-1].copy(), "1x32", off)
    assert not np.array_equal(out2[3], out[3])


def test_normwise_rel_err():
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    assert gemm.normwise_rel_err(ref, ref) == 0.0
    y = ref.copy(); y[1, 1] = 0.004
    assert gemm.normwise_rel_err(y, ref) == pytest.approx(1e-3)
    assert gemm.normwise_rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
