"""GPU parity of fp8_block_dequantize and the MXFP8 state-dict prequant
driver against the oracle (bit-exact).

Cases: every non-NaN e4m3 code under scales spanning the fp32 and E8M0
ranges (subnormal, overflow to inf), the round trip quantize -> dequantize
(equal to the quantizer's own fake-quant output), ragged row counts, a
full-size expert projection, and a small DeepSeek-style state dict.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from oracle import quant
from tests.gpu_helpers import assert_bytes_equal, bf16_from_bits, run_quantize
from workloads import bf16_bits, expert_factors, expert_weights, normal_bf16

pytestmark = pytest.mark.gpu

CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _dq(q_np, s_np, kind):
    q = torch.from_numpy(np.ascontiguousarray(q_np)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(s_np)).cuda()
    x = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    fb.fp8_block_dequantize(q, s, kind, x)
    torch.cuda.synchronize()
    return bf16_bits(x)


@pytest.mark.parametrize("kind", ["1x32", "1x128", "128x128"])
def test_every_code_and_scale_range(kind):
    rng = np.random.default_rng(50)
    rows, cols = (256, 512)
    q = np.resize(CODES, (rows, cols))
    br, bc = quant.BLOCK_SHAPE[kind]
    shp = (rows // br, cols // bc)
    if kind == "1x32":
        s = rng.integers(0, 255, shp).astype(np.uint8)
        s.flat[:4] = [0, 1, 247, 254]                 # subnormal scale, overflow to inf
    else:
        s = np.exp2(rng.uniform(-140, 120, shp)).astype(np.float32)
        s.flat[:3] = [np.float32(1.7e-39), np.float32(3.0e38), np.float32(0.0)]
    print(f"[dequant] every code {kind}", flush=True)
    assert_bytes_equal(_dq(q, s, kind), quant.dequantize(q, s, kind), "dequant")


# 128x128 blocks need rows % 128 == 0: ragged row counts go to the row-block kinds
@pytest.mark.parametrize("kind,rule,rows", [(k, r, n) for (k, r) in [("1x32", "ceil"), ("1x32", "floor"),
                                                                     ("1x128", "ceil"), ("128x128", "ceil")]
                                            for n in (128, 384, 1, 3, 1000) if k != "128x128" or n % 128 == 0])
def test_roundtrip_equals_fake_quant(kind, rule, rows):
    cols = 1024
    x = normal_bf16((rows, cols), 1.0, 60 + rows, "cuda", 0.01, 50.0, outlier_channels=True)
    q, s, xdq = run_quantize(x, kind, rule)
    got = _dq(q, s, kind)
    assert_bytes_equal(got, xdq, "dequant vs quantizer fake-quant")
    assert_bytes_equal(got, quant.dequantize(q, s, kind), "dequant vs oracle")


def test_full_size_expert_projection():
    fac = expert_factors()
    gate, up, down = expert_weights(7, "cuda", fac)
    for w in (torch.cat([gate, up], 0), down):
        q, s = fb.quantize(w, "1x32")
        x = fb.dequantize(q, s, "1x32")
        torch.cuda.synchronize()
        want = quant.dequantize(q.view(torch.uint8).cpu().numpy(), s.cpu().numpy(), "1x32")
        assert_bytes_equal(bf16_bits(x), want, f"expert 7 {tuple(w.shape)}, every element")


def test_empty_is_a_no_op():
    q = torch.empty((0, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty((0, 1), dtype=torch.float32, device="cuda")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    fb.fp8_block_dequantize(q, s, "1x128", x)


def test_quantize_state_dict_small_model():
    """Routed expert projections become float8 codes + uint8 E8M0 scales,
    byte-identical to the oracle; everything else passes through."""
    H, I = 256, 128
    state = {}
    for e in range(3):
        for proj, shape in (("gate_proj", (I, H)), ("up_proj", (I, H)), ("down_proj", (H, I))):
            state[f"model.layers.1.mlp.experts.{e}.{proj}.weight"] = normal_bf16(shape, 0.02, 70 + e, "cpu")
    state["model.layers.1.mlp.gate.weight"] = normal_bf16((3, H), 0.02, 80, "cpu")
    state["model.layers.1.mlp.shared_experts.up_proj.weight"] = normal_bf16((I, H), 0.02, 81, "cpu")
    state["model.layers.1.self_attn.q_proj.weight"] = normal_bf16((H, H), 0.02, 82, "cpu")
    state["model.norm.weight"] = torch.ones(H, dtype=torch.float32)
    print("[dequant] quantize_state_dict", flush=True)
    out = fb.quantize_state_dict(state, fmt="mxfp8", device="cuda", out_device="cpu")
    n_expert = 0
    for name, t in state.items():
        if fb.is_routed_expert_weight(name):
            n_expert += 1
            q, s = out[name], out[name[:-len("weight")] + "weight_scale_inv"]
            assert q.dtype == torch.float8_e4m3fn and s.dtype == torch.uint8
            assert s.shape == (t.shape[0], t.shape[1] // 32)
            oq, os_, _ = quant.quantize(bf16_bits(t), "1x32", "ceil")
            assert np.array_equal(q.view(torch.uint8).numpy(), oq)
            assert np.array_equal(s.numpy(), os_)
        else:
            assert out[name] is t
    assert n_expert == 9
    assert len(out) == len(state) + n_expert
