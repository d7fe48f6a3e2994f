"""Pins of oracle.quant: scale rules, element encoding, invariants.

Checks come from closed forms of the scale rules, exact rational
arithmetic, a per-element brute force, hand-worked examples
(tests/golden/quant_worked_examples.txt) and the method's own invariants:
round trip of exactly representable blocks, the error bound of half an FP8
ulp times the block scale, and outlier isolation between blocks (the point
of block-wise scaling in "DeepSeek-V3 Blog 5", "The Solution: Block-Wise
Quantization").
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec, quant
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALL_BF16_POS = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)  # +0 .. largest finite


def _bf(x):
    return codec.f32_to_bf16(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- scale rules

def test_e8m0_ceil_closed_form_all_bf16():
    """code = clamp(E - 8 + [mant > 0x60], 0, 254) for every finite bf16 amax,
    where 0x60 is the 7-bit mantissa of 1.75 = 448 / 2^8."""
    amax = codec.bf16_to_f32(ALL_BF16_POS)
    X = quant.e8m0_exponent(amax, "ceil")
    e_bits = (ALL_BF16_POS.astype(np.int64) >> 7) & 0xFF
    mant = ALL_BF16_POS.astype(np.int64) & 0x7F
    closed = np.clip(e_bits - 8 + (mant > 0x60), 0, 254)
    closed = np.where(ALL_BF16_POS == 0, 0, closed)
    assert np.array_equal(X + 127, closed)


def test_e8m0_ceil_invariant_exact():
    """448*2^(X-1) < amax <= 448*2^X for unclamped blocks (exact rationals)."""
    amax = codec.bf16_to_f32(ALL_BF16_POS)
    X = quant.e8m0_exponent(amax, "ceil")
    for a, x in zip(amax[::37], X[::37]):
        a = Fraction(float(a))
        if x > -127:
            assert 448 * Fraction(2) ** (int(x) - 1) < a <= 448 * Fraction(2) ** int(x)
        else:
            assert a <= 448 * Fraction(2) ** -127


def test_e8m0_floor_closed_form_all_bf16():
    amax = codec.bf16_to_f32(ALL_BF16_POS)
    X = quant.e8m0_exponent(amax, "floor")
    e_bits = (ALL_BF16_POS.astype(np.int64) >> 7) & 0xFF
    assert np.array_equal(X + 127, np.maximum(e_bits - 8, 0))
    unclamped = X > -127
    scaled = amax[unclamped].astype(np.float64) * np.exp2(-X[unclamped].astype(np.float64))
    assert np.all((scaled >= 256) & (scaled < 512))


def test_fp32_scale_is_correctly_rounded_all_bf16():
    amax = codec.bf16_to_f32(ALL_BF16_POS)
    s = quant.fp32_scale(amax).view(np.uint32)
    for i in range(0, len(amax), 7):
        want = exact.rn_f32(Fraction(float(amax[i])) / 448)
        assert int(s[i]) == want, hex(int(ALL_BF16_POS[i]))


# ------------------------------------------------------------ worked examples

def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "quant_worked_examples.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].strip()
            if ln:
                rows.append(ln.split())
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: "-".join(r[:4]))
def test_worked_examples(row):
    kind, rule, amax_h, x_h, scale_h, c_amax, c_x = row
    br, bc = quant.BLOCK_SHAPE[kind]
    blk = np.zeros((br, bc), dtype=np.uint16)
    blk[0, 0] = int(amax_h, 16)
    blk[0, 1] = int(x_h, 16)
    q, s, _ = quant.quantize(blk, kind, rule if rule != "-" else "ceil")
    if kind == "1x32":
        assert int(s[0, 0]) == int(scale_h, 16)
    else:
        assert int(s.view(np.uint32)[0, 0]) == int(scale_h, 16)
    assert int(q[0, 0]) == int(c_amax, 16)
    assert int(q[0, 1]) == int(c_x, 16)


# ------------------------------------------------------------- invariants

def _data(rows, cols, seed, outlier_frac=0.01):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.uniform(-20, 20, size=(rows, 1))).astype(np.float32)   # per-row magnitudes
    n_out = int(outlier_frac * x.size)
    idx = rng.choice(x.size, n_out, replace=False)
    x.ravel()[idx] *= 100
    return _bf(x)


@pytest.mark.parametrize("kind,rule", [("1x32", "ceil"), ("1x32", "floor"), ("1x128", "ceil"), ("128x128", "ceil")])
def test_roundtrip_exact_blocks(kind, rule):
    """Blocks holding 448*2^k and other values decode(c)*2^k reproduce the
    codes exactly (scale 2^k under every rule)."""
    rng = np.random.default_rng(1)
    br, bc = quant.BLOCK_SHAPE[kind]
    rows, cols = br * 2, bc * 4
    ks = rng.integers(-20, 20, size=(rows // br, cols // bc))
    codes = rng.integers(0, 0x7E, size=(rows, cols)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    codes.reshape(rows // br, br, cols // bc, bc)[:, 0, :, 0] = 0x7E   # the block max
    kk = np.repeat(np.repeat(ks, br, 0), bc, 1)
    vals = codec.e4m3_decode(codes) * np.exp2(kk)
    x = _bf(vals)
    assert np.array_equal(codec.bf16_to_f32(x).astype(np.float64), vals)
    q, s, xdq = quant.quantize(x, kind, rule)
    assert np.array_equal(q, codes)
    if kind == "1x32":
        assert np.array_equal(s.astype(np.int64) - 127, ks)
    else:
        assert np.array_equal(s, np.exp2(ks).astype(np.float32))
    assert np.array_equal(xdq, x)        # the fake-quant of an exact block is itself


def _ulp_e4m3(v):
    v = np.asarray(v, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return np.exp2(e - 3)


@pytest.mark.parametrize("kind", ["1x32", "1x128", "128x128"])
def test_element_error_bound(kind):
    """|decode(q)*scale - x| <= scale*(ulp/2 + [fp32] 2^-24 |x|/scale), in fp64.

    For E8M0 ceil the scaling is exact so only the half-ulp term remains."""
    x = _data(256, 512, seed=2)
    q, s, _ = quant.quantize(x, kind)
    xf = codec.bf16_to_f32(x).astype(np.float64)
    sc = quant.scale_multiplier(s, kind, *x.shape).astype(np.float64)
    got = codec.e4m3_decode(q) * sc
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(sc > 0, np.abs(xf) / sc, 0.0)
    vr = np.abs(np.where(sc > 0, (xf.astype(np.float32) / sc.astype(np.float32)).astype(np.float64), 0))
    if kind == "1x32":
        bound = sc * 0.5 * _ulp_e4m3(v)
    else:
        bound = sc * (0.5 * _ulp_e4m3(np.maximum(v, vr)) + 2.0 ** -24 * v)
    assert np.all(np.abs(got - xf) <= bound * (1 + 1e-12))


def test_floor_rule_error_bound_unclipped_only():
    x = _data(64, 512, seed=4)
    q, s, _ = quant.quantize(x, "1x32", "floor")
    xf = codec.bf16_to_f32(x).astype(np.float64)
    sc = quant.scale_multiplier(s, "1x32", *x.shape).astype(np.float64)
    v = np.abs(xf) / sc
    got = codec.e4m3_decode(q) * sc
    ok = v <= 464
    assert np.all(np.abs(got - xf)[ok] <= (sc * 0.5 * _ulp_e4m3(v))[ok])
    assert np.all(np.abs(codec.e4m3_decode(q[~ok])) == 448)   # clipped ones saturate


def test_fp32_block_max_maps_to_448():
    x = _data(128, 1024, seed=5)
    for kind in ("1x128", "128x128"):
        q, s, _ = quant.quantize(x, kind)
        qb = quant.block_view(q, kind)
        nz = s > 0
        has448 = np.any((qb & 0x7F) == 0x7E, axis=-1)
        assert np.all(has448[nz])


def test_zero_blocks():
    x = np.zeros((128, 256), dtype=np.uint16)
    x[3, 7] = 0x8000     # -0
    for kind in ("1x32", "1x128", "128x128"):
        q, s, xdq = quant.quantize(x, kind)
        assert np.all(s == 0)
        assert q[3, 7] == 0x80 and np.count_nonzero(q) == 1
        assert np.array_equal(xdq, x)


def test_outlier_only_changes_its_own_block():
    x = _data(256, 512, seed=6, outlier_frac=0.0)
    for kind in ("1x32", "1x128", "128x128"):
        q0, s0, _ = quant.quantize(x, kind)
        y = x.copy()
        row_max = np.abs(codec.bf16_to_f32(x[130])).max()
        y[130, 300] = _bf(np.float32(row_max * 1000))
        q1, s1, _ = quant.quantize(y, kind)
        br, bc = quant.BLOCK_SHAPE[kind]
        bi, bj = 130 // br, 300 // bc
        ds = np.argwhere(s0 != s1)
        assert ds.tolist() == [[bi, bj]]
        diff = np.argwhere(q0 != q1)
        assert np.all(diff[:, 0] // br == bi) and np.all(diff[:, 1] // bc == bj)


def test_dequant_matches_torch_casts():
    """RN_bf16(RN32(decode(q)*s)) via torch's float8 decode and casts."""
    x = _data(128, 256, seed=8)
    for kind in ("1x32", "1x128", "128x128"):
        q, s, xdq = quant.quantize(x, kind)
        qt = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
        if kind == "1x32":
            st = torch.from_numpy(s).view(torch.float8_e8m0fnu).float()
            st = st.repeat_interleave(32, dim=1)
        elif kind == "1x128":
            st = torch.from_numpy(s).repeat_interleave(128, dim=1)
        else:
            st = torch.from_numpy(s).repeat_interleave(128, 0).repeat_interleave(128, 1)
        ref = (qt * st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(xdq, ref)


def test_quantize_matches_bruteforce_per_element():
    """Small blocks re-derived one element at a time in exact rationals:
    amax, the scale (ceil rule / RN32 division) and a scan over all codes."""
    rng = np.random.default_rng(9)
    for kind, rows, cols in (("1x32", 3, 64), ("1x128", 2, 256)):
        x = _bf(rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-30, 30, (rows, 1))))
        q, s, _ = quant.quantize(x, kind)
        bc = quant.BLOCK_SHAPE[kind][1]
        for r in range(rows):
            for b in range(cols // bc):
                blk = [Fraction(float(v)) for v in codec.bf16_to_f32(x[r, b * bc:(b + 1) * bc])]
                amax = max(abs(v) for v in blk)
                if kind == "1x32":
                    X = -127
                    while amax > 448 * Fraction(2) ** X:
                        X += 1
                    assert int(s[r, b]) == X + 127
                    for j, v in enumerate(blk):
                        assert int(q[r, b * bc + j]) == exact.e4m3_brute(v * Fraction(2) ** -X) | (
                            0x80 if np.signbit(codec.bf16_to_f32(x[r, b * bc + j])) else 0)
                else:
                    sb = exact.rn_f32(amax / 448)
                    assert int(s.view(np.uint32)[r, b]) == sb
                    sv = exact.f32_value(sb)
                    for j, v in enumerate(blk):
                        qb = exact.rn_f32(v / sv)
                        want = exact.e4m3_brute(exact.f32_value(qb))
                        if qb & 0x80000000:
                            want |= 0x80
                        assert int(q[r, b * bc + j]) == want


def test_128x128_bruteforce_one_block():
    rng = np.random.default_rng(10)
    x = _bf(rng.standard_normal((128, 128)) * 0.02)
    x[5, 9] = _bf(np.float32(3.7))
    q, s, _ = quant.quantize(x, "128x128")
    xf = codec.bf16_to_f32(x)
    amax = Fraction(float(np.abs(xf).max()))
    sb = exact.rn_f32(amax / 448)
    assert int(s.view(np.uint32)[0, 0]) == sb
    sv = exact.f32_value(sb)
    for (i, j) in rng.integers(0, 128, size=(300, 2)):
        v = Fraction(float(xf[i, j]))
        qb = exact.rn_f32(v / sv)
        want = exact.e4m3_brute(exact.f32_value(qb)) | (0x80 if np.signbit(xf[i, j]) else 0)
        assert int(q[i, j]) == want


def test_dequant_overflow_of_e8m0_block_near_bf16_max():
    """amax = 0x7F7F (3.39e38): X = 120 and 255*2^-... rounds up to the e4m3
    value 256, so decode(q) * 2^120 = 2^128 overflows float32 to inf; the
    fake-quant output is then bf16 inf, as IEEE rounding prescribes."""
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x7F7F
    x[0, 1] = 0xFF7F
    q, s, xdq = quant.quantize(x, "1x32", "ceil")
    assert int(s[0, 0]) == 247 and int(q[0, 0]) == 0x78 and int(q[0, 1]) == 0xF8
    assert int(xdq[0, 0]) == 0x7F80 and int(xdq[0, 1]) == 0xFF80
    ref = (torch.from_numpy(q).view(torch.float8_e4m3fn).float()
           * torch.from_numpy(s).view(torch.float8_e8m0fnu).float().repeat_interleave(32, 1)).to(torch.bfloat16)
    assert np.array_equal(xdq, ref.view(torch.int16).numpy().view(np.uint16))


def test_shape_errors():
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((4, 48), np.uint16), "1x32")
    with pytest.raises(ValueError):
        quant.quantize(np.zeros((64, 128), np.uint16), "128x128")


def test_quotient_rounding_sensitive_cases():
    """The fp32 path is e4m3(RN32(x / s)).  Two plausible slips change a
    code only near e4m3 midpoints: multiplying by a rounded reciprocal, and
    rounding the exact quotient straight to e4m3 (skipping the fp32 step).
    Every (amax, x) bf16 pair with amax in [1, 2) is scanned for inputs where
    those slips would differ from the reading, and each such case is
    re-derived in exact rationals."""
    pos = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    xf_all = codec.bf16_to_f32(pos)
    cases = []
    for ab in range(0x3F80, 0x4000):
        amax = codec.bf16_to_f32(np.uint16(ab))
        s = quant.fp32_scale(amax)
        xs = xf_all[xf_all <= amax]
        oracle_codes = codec.e4m3_encode((xs / s).astype(np.float32))
        recip = codec.e4m3_encode(np.minimum((xs * (np.float32(1) / s)).astype(np.float32), 448))
        direct = codec.e4m3_encode(np.minimum(xs.astype(np.float64) / np.float64(s), 448))
        for i in np.nonzero((oracle_codes != recip) | (oracle_codes != direct))[0]:
            cases.append((float(amax), float(xs[i])))
    assert len(cases) >= 50
    for amax, xv in cases:
        blk = np.zeros((1, 128), dtype=np.uint16)
        blk[0, 0] = _bf(np.float32(amax))
        blk[0, 1] = _bf(np.float32(xv))
        q, s, _ = quant.quantize(blk, "1x128")
        sb = exact.rn_f32(Fraction(amax) / 448)
        qb = exact.rn_f32(Fraction(xv) / exact.f32_value(sb))
        assert int(q[0, 1]) == exact.e4m3_brute(exact.f32_value(qb)), (amax, xv)


def test_dequantize_every_code_exact():
    """dequantize on arbitrary codes (every non-NaN e4m3 code) and scales
    spanning the fp32 / E8M0 ranges, against exact rational products rounded
    once to float32 and once to bf16."""
    from tests.exact import e4m3_value, f32_bits, rn_bf16_from_f32_bits, rn_f32
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    q32 = np.resize(codes, (8, 256))                         # 8 rows x 256 cols
    rng = np.random.default_rng(12)
    e8 = np.concatenate([[0, 1, 127, 254], rng.integers(0, 255, 8 * 8 - 4)]).astype(np.uint8).reshape(8, 8)
    f128 = np.array([[1.0, 2.0 ** -130, 3.0e38], [0.015625, 7.1e-3, 1.0e-20]] * 4, dtype=np.float32)[:, :2]
    q128 = np.resize(codes, (128, 256))
    f2 = np.array([[0.5, 1.7e-39]], dtype=np.float32)        # one normal, one subnormal block scale
    cases = [(q32, e8, "1x32"), (q32, f128, "1x128"), (q128, f2, "128x128")]
    for q, sc, kind in cases:
        got = quant.dequantize(q, sc, kind)
        br, bc = quant.BLOCK_SHAPE[kind]
        for (r, c) in [(r, c) for r in range(0, q.shape[0], max(1, q.shape[0] // 16)) for c in range(q.shape[1])]:
            sv = Fraction(2) ** (int(sc[r // br, c // bc]) - 127) if kind == "1x32" else Fraction(float(sc[r // br, c // bc]))
            prod = e4m3_value(int(q[r, c])) * sv
            fb = rn_f32(prod) if abs(prod) < Fraction(2) ** 128 - Fraction(2) ** 103 else (0x7F800000 | (0x80000000 if prod < 0 else 0))
            if prod == 0 and e4m3_value(int(q[r, c])) == 0 and int(q[r, c]) & 0x80:
                fb = 0x80000000                              # -0 * s = -0
            assert int(got[r, c]) == rn_bf16_from_f32_bits(fb), (kind, r, c, hex(int(q[r, c])))
