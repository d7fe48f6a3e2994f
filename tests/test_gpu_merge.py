"""GPU parity of fp8_fake_quant_merge against the oracle (bit-exact).

Covers each register-path rank class (r <= 16, <= 32, <= 64), ragged block
counts, the zero-LoRA special case (must equal plain 128x128 quantize), and
the full QAT weight 7168x7168 with rank 16 on sampled blocks.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from oracle import codec, merge, quant
from tests.gpu_helpers import assert_bytes_equal, bf16_from_bits, run_quantize, to_np_u8
from workloads import bf16_bits, qat_forward

pytestmark = pytest.mark.gpu


def _run(w, b, a, dequant=True):
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    s = torch.empty((n // 128, k // 128), dtype=torch.float32, device=w.device)
    wdq = torch.empty_like(w) if dequant else None
    fb.fp8_fake_quant_merge(w, b, a, q, s, wdq)
    torch.cuda.synchronize()
    return to_np_u8(q), s.cpu().numpy(), (bf16_bits(wdq) if dequant else None)


def _bits(shape, sigma, seed, spread=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * sigma
    if spread:
        x = x * np.exp2(rng.integers(-spread, spread, shape))
    return codec.f32_to_bf16(x.astype(np.float32))


@pytest.mark.parametrize("r", [1, 5, 16, 17, 32, 33, 64])
def test_ranks(r):
    n, k = 256, 384
    wb, bb, ab = _bits((n, k), 0.02, 1), _bits((n, r), 0.01, 2, 8), _bits((r, k), 0.01, 3, 8)
    print(f"[merge] r={r} {n}x{k}", flush=True)
    q, s, wdq = _run(bf16_from_bits(wb), bf16_from_bits(bb), bf16_from_bits(ab))
    oq, os_, owdq = merge.fake_quant_merge(wb, bb, ab)
    assert_bytes_equal(q, oq, "codes")
    assert_bytes_equal(s, os_, "scales")
    assert_bytes_equal(wdq, owdq, "dequant")


def test_rank16_tiny_and_mixed_blocks():
    """Rank 16 with blocks whose merged amax is below 2^-60 (the pre-scaled
    quotient), blocks of exact zeros and signed zeros, next to ordinary ones."""
    n, k, r = 384, 512, 16
    wb, bb, ab = _bits((n, k), 0.02, 21), _bits((n, r), 0.01, 22, 4), _bits((r, k), 0.01, 23, 4)
    wf = codec.bf16_to_f32(wb)
    wf[0:128, 128:256] *= np.float32(2.0 ** -80)        # tiny W block (0, 1)
    wf[128:256, 256:384] = 0.0                          # W zero, LoRA term alone: block (1, 2)
    wf[256:384, 128:256] = 0.0                          # W and LoRA zero: block (2, 1)
    wb = codec.f32_to_bf16(wf)
    wb[256:384, 384:512] = 0x8000                       # W = -0, no LoRA term: block (2, 3)
    bf = codec.bf16_to_f32(bb)
    bf[0:128] *= np.float32(2.0 ** -40)                 # tiny LoRA update in block row 0
    bf[256:384] = 0.0                                   # no update in block row 2
    bb = codec.f32_to_bf16(bf)
    af = codec.bf16_to_f32(ab)
    af[:, 0:256] *= np.float32(2.0 ** -40)              # with A: 2^-80 below the rest
    ab = codec.f32_to_bf16(af)
    print(f"[merge] r=16 tiny/zero blocks {n}x{k}", flush=True)
    for dq in (True, False):
        q, s, wdq = _run(bf16_from_bits(wb), bf16_from_bits(bb), bf16_from_bits(ab), dequant=dq)
        oq, os_, owdq = merge.fake_quant_merge(wb, bb, ab)
        assert_bytes_equal(q, oq, "codes")
        assert_bytes_equal(s, os_, "scales")
        if dq:
            assert_bytes_equal(wdq, owdq, "dequant")
    assert (os_ < 2.0 ** -60).any() and (os_ == 0).any()


def test_zero_lora_equals_quantize():
    wb = _bits((384, 256), 0.02, 4)
    w = bf16_from_bits(wb)
    z_b = torch.zeros((384, 16), dtype=torch.bfloat16, device="cuda")
    a = bf16_from_bits(_bits((16, 256), 0.01, 5))
    q, s, wdq = _run(w, z_b, a)
    q2, s2, wdq2 = run_quantize(w, "128x128")
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert np.array_equal(wdq, wdq2)


def test_codes_only_variant():
    wb, bb, ab = _bits((128, 256), 0.02, 6), _bits((128, 16), 0.01, 7), _bits((16, 256), 0.01, 8)
    q, s, _ = _run(bf16_from_bits(wb), bf16_from_bits(bb), bf16_from_bits(ab), dequant=False)
    oq, os_, _ = merge.fake_quant_merge(wb, bb, ab)
    assert_bytes_equal(q, oq, "codes")
    assert_bytes_equal(s, os_, "scales")


def test_qat_weight_full_size_all_blocks():
    """The QAT weight 7168x7168 at rank 16, every one of its 3136 blocks:
    codes, scales and the dequantized weight byte-equal to the oracle's
    merge and fake-quant of the whole matrix (about 30 s of host time)."""
    d = qat_forward("cuda", m=128)
    w, a, b = d["w"], d["lora_a"], d["lora_b"]
    print("[merge] QAT W 7168x7168 r=16 (all 128x128 blocks)", flush=True)
    q, s, wdq = _run(w, b, a)
    oq, os_, owdq = merge.fake_quant_merge(bf16_bits(w), bf16_bits(b), bf16_bits(a))
    assert_bytes_equal(q, oq, "codes")
    assert_bytes_equal(s, os_, "scales")
    assert_bytes_equal(wdq, owdq, "dequantized weight")
    print("[merge] all 3136 blocks byte-equal to the oracle", flush=True)
