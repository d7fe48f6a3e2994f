"""Pins of the NVFP4 oracle (oracle/nvfp4.py), CPU only.

  * the 16 E2M1 codes decode to the OCP specification's values
    (tests/golden/e2m1_spec_values.txt);
  * the E2M1 encoder equals a brute-force nearest-value search in exact
    rational arithmetic (ties to the even code, saturation, sign of zero);
  * a hand-derived worked example (tests/golden/nvfp4_worked_example.txt):
    tensor amax, global scale, block scales, codes, packing, dequantized
    values;
  * every element code equals the nearest E2M1 value of the exactly
    computed quotient rounded once to fp32, and every block scale the
    nearest e4m3 value of RN32(a / RN32(6 g)), on random tensors;
  * exactly representable tensors round-trip; stacked tensors get their own
    scales; all-zero tensors and blocks whose scale underflows give zeros.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4
from oracle.codec import bf16_to_f32, e4m3_decode, e4m3_encode, f32_to_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(values):
    return f32_to_bf16(np.asarray(values, dtype=np.float32))


def test_e2m1_decode_matches_spec():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1_spec_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = nvfp4.e2m1_decode(int(code, 16))
        want = float(val)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def _brute_e2m1(v):
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]
    a = abs(Fraction(float(v)))
    if a >= 6:
        best = 7
    else:
        d = [abs(a - m) for m in mags]
        dm = min(d)
        cands = [i for i, x in enumerate(d) if x == dm]
        best = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return best | (8 if np.signbit(v) else 0)


def test_e2m1_encode_brute_force():
    grid = [k / 64.0 for k in range(0, 640)]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    near = []
    for m in mids:
        f = np.float32(m)
        near += [float(np.nextafter(f, np.float32(0))), float(f), float(np.nextafter(f, np.float32(100)))]
    vals = np.array(grid + near + [7.0, 1e30, 1e-30, 0.0], dtype=np.float32)
    vals = np.concatenate([vals, -vals])
    got = nvfp4.e2m1_encode(vals)
    want = np.array([_brute_e2m1(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)
    assert nvfp4.e2m1_encode(np.float32(-0.0)) == 8


def _golden_example():
    rec = {}
    for ln in open(os.path.join(GOLDEN, "nvfp4_worked_example.txt")):
        if ln.strip() and not ln.startswith("#"):
            k, *v = ln.split()
            rec[k] = v
    return rec


def test_worked_example():
    rec = _golden_example()
    x = _bits([float(v) for v in rec["x"]]).reshape(1, 32)
    packed, S, g, A, xdq = nvfp4.quantize(x)
    assert A[0] == float(rec["A"][0])
    assert g[0] == float.fromhex(rec["g"][0])
    assert S.tolist() == [[int(s, 16) for s in rec["S"]]]
    assert nvfp4.unpack(packed)[0].tolist() == [int(c, 16) for c in rec["codes"]]
    assert packed[0].tolist() == [int(b, 16) for b in rec["packed"]]
    want = _bits([float(v) for v in rec["xdq"]])
    assert np.array_equal(xdq[0], want)


def test_pack_order():
    codes = np.arange(16, dtype=np.uint8).reshape(1, 16)
    assert nvfp4.pack(codes)[0].tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(nvfp4.unpack(nvfp4.pack(codes)), codes)


def test_codes_and_scales_against_exact_arithmetic():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 64)).astype(np.float32) * np.float32(0.02)
    x[1, 3] = 0.9                   # a large entry: the tensor amax
    x[4, 16:32] *= np.float32(1e-3)  # a small block
    xb = f32_to_bf16(x)
    packed, S, g, A, xdq = nvfp4.quantize(xb)
    xf = bf16_to_f32(xb)
    assert A[0] == np.abs(xf).max()
    assert g[0] == np.float32(A[0]) / np.float32(2688.0)
    t = np.float32(6.0) * g[0]
    codes = nvfp4.unpack(packed)
    for r in range(6):
        for b in range(4):
            blk = xf[r, 16 * b:16 * b + 16]
            a = np.abs(blk).max()
            ratio = Fraction(float(a)) / Fraction(float(t))
            ratio32 = np.float32(float(ratio))                 # RN32 of the exact quotient
            assert S[r, b] == e4m3_encode(ratio32)
            m = np.float32(e4m3_decode(S[r, b])) * g[0]
            for j in range(16):
                q32 = np.float32(float(Fraction(float(blk[j])) / Fraction(float(m))))
                assert codes[r, 16 * b + j] == _brute_e2m1(q32), (r, b, j)
    # dequantized value: RN_bf16 of the code's value times m, and within
    # half an E2M1 step (times m) of x unless saturated
    deq = bf16_to_f32(xdq).astype(np.float64)
    mrow = np.repeat((e4m3_decode(S).astype(np.float32) * g[0]).astype(np.float64), 16, axis=1)
    q = np.abs(xf / np.where(mrow == 0, 1, mrow))
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    ok = (np.abs(deq - xf) <= 0.5 * step * mrow * (1 + 2 ** -7) + 1e-30) | (q > 6)
    assert np.all(ok)


def test_exact_tensors_round_trip():
    """x = e2m1 * e4m3 * g with g = 2^-7 (A = 21) and every block holding
    the value 6 * S: quantize -> dequantize returns x bit for bit."""
    rng = np.random.default_rng(8)
    grid = nvfp4.e2m1_decode(np.arange(16))
    rows = []
    for S in (0x7E, 0x70, 0x5B, 0x40, 0x38):
        m = float(e4m3_decode(S)) * 2.0 ** -7
        vals = grid[rng.integers(0, 16, 16)] * m
        vals[0] = 6.0 * m
        rows.append(vals)
    x = np.concatenate(rows).reshape(1, -1).astype(np.float32)
    x[0, 0] = 21.0                     # 6 * 448 * 2^-7: the tensor amax
    xb = f32_to_bf16(x)
    assert np.array_equal(bf16_to_f32(xb), x)
    packed, S, g, A, xdq = nvfp4.quantize(xb)
    assert g[0] == 2.0 ** -7
    assert S[0].tolist() == [0x7E, 0x70, 0x5B, 0x40, 0x38]
    assert np.array_equal(xdq, xb)


def test_stacked_tensors_have_their_own_scales():
    rng = np.random.default_rng(9)
    parts = [rng.standard_normal((4, 32)).astype(np.float32) * s for s in (0.01, 3.0, 200.0)]
    xb = f32_to_bf16(np.concatenate(parts))
    packed, S, g, A, xdq = nvfp4.quantize(xb, rows_per_tensor=4)
    assert g.shape == (3,)
    for i in range(3):
        p1, s1, g1, a1, x1 = nvfp4.quantize(xb[4 * i:4 * i + 4])
        assert g[i] == g1[0] and A[i] == a1[0]
        assert np.array_equal(packed[4 * i:4 * i + 4], p1)
        assert np.array_equal(S[4 * i:4 * i + 4], s1)
        assert np.array_equal(xdq[4 * i:4 * i + 4], x1)


def test_zero_tensor_and_underflowing_block():
    z = _bits(np.zeros((2, 32), np.float32))
    z[1, 5] = 0x8000                  # -0
    packed, S, g, A, xdq = nvfp4.quantize(z)
    assert g[0] == 0 and A[0] == 0 and not S.any()
    codes = nvfp4.unpack(packed)
    assert codes[1, 5] == 8 and codes.sum() == 8
    assert np.array_equal(xdq, z)
    # a block whose ratio a / (6 g) is below the smallest e4m3 step: S = 0,
    # codes keep only the sign, values dequantize to +-0
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 3.0e4
    x[0, 16] = -1e-3
    x[0, 17] = 2e-3
    xb = f32_to_bf16(x)
    packed, S, g, A, xdq = nvfp4.quantize(xb)
    assert S[0, 1] == 0
    codes = nvfp4.unpack(packed)
    assert codes[0, 16] == 8 and codes[0, 17] == 0
    assert bf16_to_f32(xdq)[0, 16] == 0 and np.signbit(bf16_to_f32(xdq)[0, 16])


def test_given_amax_is_used():
    xb = _bits(np.linspace(-1, 1, 32, dtype=np.float32).reshape(1, 32))
    _, _, g, A, _ = nvfp4.quantize(xb, amax=np.array([4.0], np.float32))
    assert A[0] == 4.0 and g[0] == np.float32(4.0) / np.float32(2688.0)


def test_shape_checks():
    with pytest.raises(ValueError):
        nvfp4.quantize(np.zeros((2, 24), np.uint16))
    with pytest.raises(ValueError):
        nvfp4.quantize(np.zeros((3, 32), np.uint16), rows_per_tensor=2)
