"""Shared helpers for the GPU parity tests (tests only)."""

import numpy as np
import torch

import block_scaled_fp8_amax_amd as fb
from workloads import bf16_bits

DEV = "cuda"


def to_np_u8(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def to_np_scale(t):
    return t.cpu().numpy()


def run_quantize(x, kind, rule="ceil", dequant=True):
    """Quantize a bf16 cuda tensor through the C ABI; numpy results."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    shp, dt = fb.scale_shape(rows, cols, kind)
    s = torch.full(shp, 0, dtype=dt, device=x.device)
    xdq = torch.empty_like(x) if dequant else None
    fb.fp8_block_quantize(x, kind, rule, q, s, xdq)
    torch.cuda.synchronize()
    return to_np_u8(q), to_np_scale(s), (bf16_bits(xdq) if dequant else None)


def bf16_from_bits(bits, device=DEV):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        want = np.asarray(want, dtype=np.float32).view(np.uint32)
    bad = np.argwhere(got != want)
    if len(bad):
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}")
