"""GPU parity of fp8_nvfp4_quantize / fp8_nvfp4_dequantize against the
oracle (oracle/nvfp4.py): every output byte-identical.

Cases: the hand-derived worked example; random shapes with one or many
stacked tensors, ragged row counts, wide dynamic ranges and subnormal
inputs (the quotient's prescale path); an exhaustive sweep of every bf16
magnitude below the block amax for several block multipliers (every E2M1
rounding boundary and tie); a caller-given tensor amax; all-zero tensors
and blocks whose scale underflows; every code byte under scales across the
e4m3 range; a full-size expert pair; the state-dict driver.
"""

import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from oracle import nvfp4
from oracle.codec import bf16_to_f32, f32_to_bf16
from tests.gpu_helpers import assert_bytes_equal, bf16_from_bits
from workloads import bf16_bits, expert_factors, expert_weights, normal_bf16

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(xb_bits, rpt=None, amax=None, dq=True):
    x = bf16_from_bits(xb_bits)
    am = None if amax is None else torch.from_numpy(np.asarray(amax, np.float32)).cuda()
    out = fb.nvfp4_quantize(x, rows_per_tensor=rpt, dequant=dq, amax=am)
    torch.cuda.synchronize()
    q, bs, gs, A = out[:4]
    res = (q.cpu().numpy(), bs.view(torch.uint8).cpu().numpy(), gs.cpu().numpy(), A.cpu().numpy())
    return res + ((bf16_bits(out[4]),) if dq else ())


def _compare(xb_bits, rpt=None, amax=None, what=""):
    got = _run(xb_bits, rpt, amax)
    want = nvfp4.quantize(xb_bits, rpt, amax)
    want = (want[0], want[1], want[2], want[3], want[4])
    for name, g, w in zip(("codes", "block scales", "global scales", "tensor amax", "xdq"), got, want):
        assert_bytes_equal(g, w, f"{what} {name}")
    return got


def test_worked_example():
    rec = {}
    for ln in open(os.path.join(GOLDEN, "nvfp4_worked_example.txt")):
        if ln.strip() and not ln.startswith("#"):
            k, *v = ln.split()
            rec[k] = v
    x = f32_to_bf16(np.array([float(v) for v in rec["x"]], np.float32)).reshape(1, 32)
    q, bs, gs, A, xdq = _compare(x, what="worked example")
    assert q[0].tolist() == [int(b, 16) for b in rec["packed"]]


@pytest.mark.parametrize("rows,cols,rpt", [(1, 16, 1), (3, 48, 1), (64, 256, 64), (128, 7168, 32),
                                           (1000, 512, 1000), (96, 1024, 1), (257, 160, 257)])
@pytest.mark.parametrize("dist", ["normal", "wide", "tiny"])
def test_random_shapes(rows, cols, rpt, dist):
    print(f"[nvfp4] {rows}x{cols} rpt={rpt} {dist}", flush=True)
    rng = np.random.default_rng(rows * 7 + cols + len(dist))
    if dist == "normal":
        x = rng.standard_normal((rows, cols)).astype(np.float32) * np.float32(0.02)
        x[rng.random((rows, cols)) < 0.001] *= 100
    elif dist == "wide":
        x = (np.exp2(rng.uniform(-40, 40, (rows, cols))) * rng.choice([-1, 1], (rows, cols))).astype(np.float32)
    else:
        x = (np.exp2(rng.uniform(-133, -110, (rows, cols))) * rng.choice([-1, 1], (rows, cols))).astype(np.float32)
    _compare(f32_to_bf16(x), rpt, what=f"{rows}x{cols}/{rpt} {dist}")


def _bf16_magnitudes_below(a):
    """Every finite positive bf16 value <= a (as float32)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    v = bf16_to_f32(bits)
    return v[v <= a]


@pytest.mark.parametrize("amax", [21.0, 17.25, 0.0371, 3.0e-30, 5.0e30])
def test_every_bf16_value_under_one_multiplier(amax):
    """Blocks whose first element is the tensor amax (so every block has the
    same multiplier m = e4m3(448) g) holding every smaller bf16 magnitude,
    both signs: every E2M1 boundary and tie of x / m is crossed."""
    a32 = bf16_to_f32(f32_to_bf16(np.float32(amax)))
    vals = _bf16_magnitudes_below(a32)
    vals = np.concatenate([vals, -vals, [0.0, -0.0]]).astype(np.float32)
    pad = (-len(vals)) % 15
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 15)
    blocks = np.concatenate([np.full((vals.shape[0], 1), a32, np.float32), vals], axis=1)
    n = blocks.shape[0] - blocks.shape[0] % 8
    x = blocks[:n].reshape(-1, 128)
    print(f"[nvfp4] sweep amax={amax}: {x.size} values", flush=True)
    _compare(f32_to_bf16(x), what=f"sweep amax={amax}")


def test_every_block_multiplier():
    """One block per reachable block scale: block amax = tensor amax * k / 256
    for k = 1..256, each block holding a spread of values."""
    rng = np.random.default_rng(60)
    A = np.float32(300.0)
    rows = []
    for k in range(1, 257):
        a = A * np.float32(k) / np.float32(256)
        blk = (rng.uniform(-1, 1, 16) * a).astype(np.float32)
        blk[0] = a
        rows.append(blk)
    rows.append(np.full(16, A, np.float32))
    x = np.concatenate(rows + [np.zeros(16 * 3, np.float32)]).reshape(-1, 64)
    _compare(f32_to_bf16(x), what="block multipliers")


def test_given_amax():
    rng = np.random.default_rng(61)
    x = f32_to_bf16((rng.standard_normal((64, 128)) * 0.5).astype(np.float32))
    _compare(x, 32, amax=[4.0, 0.75], what="given amax")


def test_zero_tensor_and_underflowing_blocks():
    z = np.zeros((4, 64), np.uint16)
    z[1, 5] = 0x8000
    _compare(z, 2, what="zero tensors")
    x = np.zeros((2, 64), np.float32)
    x[0, 0] = 3.0e4
    x[0, 16:32] = np.linspace(-1e-3, 1e-3, 16)
    x[1, 40] = -0.0
    _compare(f32_to_bf16(x), what="underflowing blocks")


def test_dequantize_every_code_byte():
    rng = np.random.default_rng(62)
    rows, cols = 64, 512
    q = np.resize(np.arange(256, dtype=np.uint8), (rows, cols // 2))
    S = rng.integers(0, 0x7F, (rows, cols // 16)).astype(np.uint8)
    S.flat[:4] = [0, 1, 0x7E, 0x38]
    g = np.array([3.0e-3, 1.7e-38, 5.0e2, 1.0], np.float32)
    want = nvfp4.dequantize(q, S, g, 16)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    fb.fp8_nvfp4_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(S).cuda(), torch.from_numpy(g).cuda(), 16,
                            x)
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_bits(x), want, "nvfp4 dequantize")


def test_roundtrip_equals_fake_quant():
    x = normal_bf16((300, 2048), 0.02, 63, "cuda", 0.01, 30.0)
    q, bs, gs, A, xdq = fb.nvfp4_quantize(x, rows_per_tensor=100, dequant=True)
    back = fb.nvfp4_dequantize(q, bs, gs, 100)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), xdq.view(torch.int16))


def test_full_size_expert_pair():
    """gate and up (2048x7168 each) stacked: two tensors, their own scales;
    every code and block scale byte-exact, global scales and amax exact; the
    dequantize of those codes equals the oracle's fake-quant values on every
    element."""
    fac = expert_factors()
    gate, up, _ = expert_weights(5, "cuda", fac)
    w = torch.cat([gate, up], 0)
    q, bs, gs, A = fb.nvfp4_quantize(w, rows_per_tensor=2048)
    torch.cuda.synchronize()
    wb = bf16_bits(w)
    oA = nvfp4.tensor_amax(wb, 2048)
    assert_bytes_equal(A.cpu().numpy(), oA, "tensor amax")
    assert_bytes_equal(gs.cpu().numpy(), nvfp4.global_scale(oA), "global scales")
    oq, ob, _, _, oxdq = nvfp4.quantize(wb, 2048, amax=oA)
    assert_bytes_equal(q.cpu().numpy(), oq, "codes")
    assert_bytes_equal(bs.view(torch.uint8).cpu().numpy(), ob, "block scales")
    x = fb.nvfp4_dequantize(q, bs, gs, rows_per_tensor=2048)
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_bits(x), oxdq, "dequantized pair")


def test_quantize_state_dict_nvfp4():
    H, I = 256, 128
    state = {}
    for e in range(2):
        for proj, shape in (("gate_proj", (I, H)), ("up_proj", (I, H)), ("down_proj", (H, I))):
            state[f"model.layers.2.mlp.experts.{e}.{proj}.weight"] = normal_bf16(shape, 0.02, 90 + e, "cpu")
    state["model.layers.2.self_attn.o_proj.weight"] = normal_bf16((H, H), 0.02, 95, "cpu")
    out = fb.quantize_state_dict(state, fmt="nvfp4", device="cuda", out_device="cpu")
    n = 0
    for name, t in state.items():
        if not fb.is_routed_expert_weight(name):
            assert out[name] is t
            continue
        n += 1
        stem = name[:-len("weight")]
        q, s, g = out[name], out[stem + "weight_scale_inv"], out[stem + "weight_global_scale"]
        assert q.dtype == torch.uint8 and q.shape == (t.shape[0], t.shape[1] // 2)
        assert s.dtype == torch.float8_e4m3fn and s.shape == (t.shape[0], t.shape[1] // 16)
        oq, os_, og, _, _ = nvfp4.quantize(bf16_bits(t))
        assert np.array_equal(q.numpy(), oq)
        assert np.array_equal(s.view(torch.uint8).numpy(), os_)
        assert np.array_equal(g.numpy(), og)
    assert n == 6 and len(out) == len(state) + 2 * n
