"""Pins of oracle.codec against the OCP closed forms, brute force and torch.

The pages name float8_e4m3fn and uint8 E8M0 ([prequant] "Quick start",
"Formats") without printing their layout; the OCP 8-bit floating point and
MX specifications fix it.  torch's own float8/bfloat16 casts are an
independent implementation used here as a second opinion.
"""

import os

import numpy as np
import pytest
import torch

from oracle import codec
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = codec.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    nan_ours, nan_theirs = np.isnan(ours), np.isnan(theirs)
    assert np.array_equal(nan_ours, nan_theirs)
    assert sorted(np.nonzero(nan_ours)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan_ours], theirs[~nan_theirs])
    # signed zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0])


def test_decode_matches_exact_closed_form():
    for c in range(256):
        v = exact.e4m3_value(c)
        d = codec.e4m3_decode(c)
        if v is None:
            assert np.isnan(d)
        else:
            assert float(v) == float(d)


def test_spec_values_golden():
    """tests/golden/e4m3_spec_values.txt: values fixed by the OCP layout."""
    with open(os.path.join(GOLDEN, "e4m3_spec_values.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 8
    for code_hex, value in rows:
        d = codec.e4m3_decode(int(code_hex, 16))
        if value == "nan":
            assert np.isnan(d)
        else:
            assert float(d) == float.fromhex(value)


def test_table_strictly_increasing():
    t = codec.e4m3_nonneg_table()
    assert len(t) == 127 and t[0] == 0.0 and t[-1] == 448.0
    assert np.all(np.diff(t) > 0)


def _structured_values():
    """fp32 values around every e4m3 value and every midpoint in (0, 512)."""
    t = codec.e4m3_nonneg_table()
    pts = np.concatenate([t[1:], (t[:-1] + t[1:]) / 2, [448.0, 464.0, 480.0, 496.0, 511.0]])
    bits = pts.astype(np.float32).view(np.uint32).astype(np.int64)
    offs = np.arange(-8, 9)
    allb = (bits[:, None] + offs[None, :]).ravel()
    vals = allb.astype(np.uint32).view(np.float32)
    return vals[(vals >= 2.0 ** -12) & (vals < 512)]


def _brute_nearest_scaled(vals):
    """Nearest code by scanning all 127 codes with exact int64 distances.

    Every float32 in [2^-12, 512) is a multiple of 2^-35 and every e4m3 value
    a multiple of 2^-9, so scaling by 2^35 makes all distances exact int64.
    """
    t = codec.e4m3_nonneg_table()
    tint = np.round(t * 2.0 ** 35).astype(np.int64)
    out = np.empty(len(vals), dtype=np.int64)
    for i0 in range(0, len(vals), 20000):
        v = vals[i0:i0 + 20000].astype(np.float64)
        vint = np.round(v * 2.0 ** 35).astype(np.int64)
        assert np.array_equal(vint.astype(np.float64) / 2.0 ** 35, v)
        d = np.abs(vint[:, None] - tint[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        even = cand & (np.arange(127)[None, :] % 2 == 0)
        # a tie is between two adjacent codes; prefer the even one
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        pick = np.where(v >= 448.0, 126, pick)
        out[i0:i0 + 20000] = pick
    return out


def test_encode_matches_bruteforce_structured_and_random():
    rng = np.random.default_rng(7)
    rnd = np.exp2(rng.uniform(-12, 9, size=400000)).astype(np.float32)
    rnd = rnd[(rnd >= 2.0 ** -12) & (rnd < 512)]
    vals = np.concatenate([_structured_values(), rnd])
    ours = codec.e4m3_encode(vals).astype(np.int64)
    assert np.array_equal(ours, _brute_nearest_scaled(vals))
    # negatives mirror positives with the sign bit
    assert np.array_equal(codec.e4m3_encode(-vals).astype(np.int64), ours | 0x80)


def test_encode_small_values_round_to_zero():
    # (0, 2^-10) -> 0; 2^-10 is the midpoint between codes 0 and 1: tie -> 0 (even)
    small = _f32(np.arange(1, 0x3A800000, 997, dtype=np.uint32))  # 0x3A800000 = 2^-10
    assert np.all(codec.e4m3_encode(small) == 0)
    assert np.all(codec.e4m3_encode(-small) == 0x80)
    assert codec.e4m3_encode(np.float32(2.0 ** -10)) == 0
    assert codec.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 1
    assert codec.e4m3_encode(np.float32(-0.0)) == 0x80
    assert codec.e4m3_encode(np.float32(0.0)) == 0


def test_encode_scalar_bruteforce_fraction():
    """A handful of values checked by a scan over all codes in exact rationals."""
    rng = np.random.default_rng(3)
    vals = list(_structured_values()[::97]) + list(np.exp2(rng.uniform(-11, 9.5, 300)).astype(np.float32))
    for v in vals:
        for s in (1.0, -1.0):
            x = np.float32(v) * np.float32(s)
            assert int(codec.e4m3_encode(x)) == exact.e4m3_brute(float(x)), float(x)


def test_encode_matches_torch_below_464():
    rng = np.random.default_rng(11)
    v = (rng.standard_normal(2_000_000) * np.exp2(rng.uniform(-14, 8, 2_000_000))).astype(np.float32)
    v = np.concatenate([v, _structured_values(), -_structured_values()])
    v = v[np.abs(v) <= 464]
    ours = codec.e4m3_encode(v)
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_encode_saturates_at_448():
    big = np.concatenate([
        _f32(np.arange(0x43E00000, 0x43F00000, 13, dtype=np.uint32)),   # [448, 480)
        np.float32([448.0, 464.0, 464.00003, 1e4, 3.0e38])])
    assert np.all(codec.e4m3_encode(big) == 0x7E)
    assert np.all(codec.e4m3_encode(-big) == 0xFE)
    # just below 448: nearest is 448 once above the 416/448 midpoint (432)
    assert codec.e4m3_encode(np.float32(447.9)) == 0x7E
    # 432 is halfway between 416 (0x7D, odd) and 448 (0x7E, even) -> 0x7E;
    # 400 is halfway between 384 (0x7C, even) and 416 (0x7D) -> 0x7C
    assert codec.e4m3_encode(np.float32(432.0)) == 0x7E
    assert codec.e4m3_encode(np.float32(431.99)) == 0x7D
    assert codec.e4m3_encode(np.float32(400.0)) == 0x7C
    assert codec.e4m3_encode(np.float32(400.01)) == 0x7D


def test_encode_decode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codec.e4m3_decode(codes)
    assert np.array_equal(codec.e4m3_encode(vals), codes)


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        codec.e4m3_encode(np.float32([1.0, np.inf]))


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codec.e8m0_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)
    assert np.isnan(ours[255]) and np.isnan(theirs[255])
    assert np.array_equal(ours[:255], theirs[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_bf16_widen_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codec.bf16_to_f32(bits)
    theirs = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ok = ~np.isnan(theirs)
    assert np.array_equal(ours[ok].view(np.uint32), theirs[ok].view(np.uint32))


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(5)
    # random patterns (finite, below bf16 overflow) + every tie point +-1 ulp
    rb = rng.integers(0, 0x7F7F0000, size=3_000_000, dtype=np.uint32)
    rb = np.concatenate([rb, rb | 0x80000000])
    ties = (np.arange(0, 0x7F7F, dtype=np.uint32) << 16) | 0x8000
    tb = np.concatenate([ties - 1, ties, ties + 1, ties | 0x80000000])
    v = _f32(np.concatenate([rb, tb]))
    ours = codec.f32_to_bf16(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_round_overflow_and_inf_match_torch():
    """Beyond the largest finite bf16 (0x7F7F) the upper neighbour is inf:
    the midpoint 0x7F7F8000 ties to even (inf), values below it stay finite."""
    v = _f32(np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F800000,
                       0xFF7F7FFF, 0xFF7F8000, 0xFF800000], dtype=np.uint32))
    ours = codec.f32_to_bf16(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert ours.tolist() == [0x7F7F, 0x7F80, 0x7F80, 0x7F80, 0x7F80, 0xFF7F, 0xFF80, 0xFF80]
    with pytest.raises(ValueError):
        codec.f32_to_bf16(np.float32([np.nan]))


def test_bf16_round_tie_examples():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: tie -> even (1.0)
    assert codec.f32_to_bf16(np.float32(1 + 2.0 ** -8)) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> up
    assert codec.f32_to_bf16(np.float32(1 + 3 * 2.0 ** -8)) == 0x3F82
    assert codec.f32_to_bf16(np.float32(-0.0)) == 0x8000
