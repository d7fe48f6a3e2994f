"""GPU parity of fp8_lora_backward against the oracle (oracle/lora_grad.py).

Tolerance, derived from the kernel's arithmetic: products of bf16 values
are exact in fp32; the rank-r intermediates P = X.A^T and Q = dY.B are
carried with 16 significant bits (hi + lo bf16, relative error <= 2^-17)
after an fp32 sum of at most ~64 blocked steps, and the token reduction
runs through at most ~64 fp32 additions at full size.  The fp32 result c
therefore satisfies |c - ref| <= 2^-14 * mag, where mag is the same double
sum over absolute values:
    mag_B = |dY|^T . (|X| . |A|^T),   mag_A = (|dY| . |B|)^T . |X|.
A bf16 output adds one rounding: |out - ref| <= 2^-8 |ref| + 2^-14 mag.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from oracle import lora_grad
from oracle.codec import bf16_to_f32
from workloads import bf16_bits, qat_backward

pytestmark = pytest.mark.gpu
EPS_MAG = 2.0 ** -14


def _f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


def _mags(dy_b, x_b, b_b, a_b):
    dy, x, b, a = (np.abs(_f64(t)) for t in (dy_b, x_b, b_b, a_b))
    return dy.T @ (x @ a.T), ((dy @ b).T @ x)


def _grads_np(db, da):
    if db.dtype == torch.float32:
        return db.cpu().numpy().astype(np.float64), da.cpu().numpy().astype(np.float64)
    return _f64(bf16_bits(db)), _f64(bf16_bits(da))


def _check(got, ref, mag, bf16, what):
    tol = EPS_MAG * mag + (2.0 ** -8 * np.abs(ref) if bf16 else 0.0)
    err = np.abs(got - ref)
    bad = np.argwhere(err > tol)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {err.size} outside tolerance, first at {i}: "
                             f"got {got[i]!r} want {ref[i]!r} tol {tol[i]!r}")


def _inputs(m, n, k, r, seed):
    d = qat_backward("cuda", m, n, k, r, seed)
    return d["dy"], d["x"], d["lora_b"], d["lora_a"]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("m,n,k,r", [
    (64, 256, 384, 16),
    (1, 128, 128, 1),
    (33, 384, 256, 5),
    (100, 640, 1152, 16),       # partial column groups on both outputs
    (257, 128, 512, 17),        # rank 17..32
    (96, 256, 128, 32),
    (70, 128, 256, 33),         # rank 33..64
    (64, 512, 512, 64),
    (4096, 512, 640, 16),       # many token slices
    (1000, 1024, 256, 8),
    (80, 256, 384, 12),         # rank <= 16 runs 64 tokens per projection workgroup: odd count of 32-token blocks
])
def test_small_shapes(m, n, k, r, out):
    print(f"[lora_bwd] m={m} n={n} k={k} r={r} {out}", flush=True)
    dy, x, b, a = _inputs(m, n, k, r, 400 + m + r)
    db, da = fb.lora_backward(dy, x, b, a, out_dtype=out)
    torch.cuda.synchronize()
    got_b, got_a = _grads_np(db, da)
    bits = [bf16_bits(t) for t in (dy, x, b, a)]
    ref_b, ref_a = lora_grad.lora_grads(*bits)
    mag_b, mag_a = _mags(*bits)
    bf = out == torch.bfloat16
    _check(got_b, ref_b, mag_b, bf, "dB")
    _check(got_a, ref_a, mag_a, bf, "dA")


def test_no_tokens_writes_zeros():
    n, k, r = 256, 384, 16
    b = torch.ones((n, r), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((r, k), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((0, n), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, k), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((fb.fp8_lora_backward_workspace(0, n, k, r),), 0x7F, dtype=torch.uint8, device="cuda")
    db = torch.full((n, r), 7.0, dtype=torch.float32, device="cuda")
    da = torch.full((r, k), 7.0, dtype=torch.float32, device="cuda")
    fb.fp8_lora_backward(dy, x, b, a, ws, db, da)
    torch.cuda.synchronize()
    assert torch.count_nonzero(db).item() == 0 and torch.count_nonzero(da).item() == 0


def test_empty_hidden_dimension():
    """n == 0 (no output features): dA = 0; k == 0: dB = 0."""
    m, r = 64, 16
    dy, x, b, a = _inputs(m, 256, 256, r, 450)
    dy0 = torch.empty((m, 0), dtype=torch.bfloat16, device="cuda")
    b0 = torch.empty((0, r), dtype=torch.bfloat16, device="cuda")
    db, da = fb.lora_backward(dy0, x, b0, a, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert db.numel() == 0 and torch.count_nonzero(da).item() == 0
    x0 = torch.empty((m, 0), dtype=torch.bfloat16, device="cuda")
    a0 = torch.empty((r, 0), dtype=torch.bfloat16, device="cuda")
    db, da = fb.lora_backward(dy, x0, b, a0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert da.numel() == 0 and torch.count_nonzero(db).item() == 0


def test_workspace_reuse_and_determinism():
    """A workspace holding a previous, larger call's data gives the same
    bytes as a fresh one; repeated calls are bit-identical."""
    big = _inputs(512, 1024, 1024, 16, 460)
    small = _inputs(96, 384, 256, 16, 461)
    ws = torch.empty(fb.fp8_lora_backward_workspace(512, 1024, 1024, 16), dtype=torch.uint8, device="cuda")
    fb.lora_backward(*big, workspace=ws)
    r1 = fb.lora_backward(*small, workspace=ws)
    r2 = fb.lora_backward(*small)
    r3 = fb.lora_backward(*small, workspace=ws)
    torch.cuda.synchronize()
    for t1, t2, t3 in zip(r1, r2, r3):
        assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))
        assert torch.equal(t1.view(torch.int16), t3.view(torch.int16))


def test_full_size_qat_backward():
    """M 8192 tokens, N = K = 7168, rank 16, on fake-quantized activations
    (1x128 fake-quant of X, as the QAT forward feeds the GEMM): every element
    of dB and dA against the oracle (dW formed in float64), and the identity
    sum_n dB[n,c] B[n,c] = sum_k dA[c,k] A[c,k] (both equal
    sum_{n,k} B[n,c] dW[n,k] A[c,k]) over every c at full size."""
    M, N, K, R = 8192, 7168, 7168, 16
    print("[lora_bwd] full size", flush=True)
    dy, x, b, a = _inputs(M, N, K, R, 470)
    _, _, xdq = fb.quantize(x, "1x128", dequant=True)
    del x
    db, da = fb.lora_backward(dy, xdq, b, a, out_dtype=torch.float32)
    db16, da16 = fb.lora_backward(dy, xdq, b, a, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # bf16 output is the rounding of the same fp32 result
    assert torch.equal(db.to(torch.bfloat16).view(torch.int16), db16.view(torch.int16))
    assert torch.equal(da.to(torch.bfloat16).view(torch.int16), da16.view(torch.int16))

    bits = [bf16_bits(t) for t in (dy, xdq, b, a)]
    ref_b, ref_a = lora_grad.lora_grads(*bits)
    mag_b, mag_a = _mags(*bits)
    got_b, got_a = _grads_np(db, da)
    _check(got_b, ref_b, mag_b, False, "dB")
    _check(got_a, ref_a, mag_a, False, "dA")

    bf, af = _f64(bits[2]), _f64(bits[3])
    lhs = np.sum(got_b * bf, axis=0)
    rhs = np.sum(got_a * af, axis=1)
    bound = EPS_MAG * (np.sum(mag_b * np.abs(bf), axis=0) + np.sum(mag_a * np.abs(af), axis=1))
    assert np.all(np.abs(lhs - rhs) <= bound), (lhs, rhs, bound)
