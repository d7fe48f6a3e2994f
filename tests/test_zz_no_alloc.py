"""GPU test of fp8_lora_backward_noalloc (the entry point that allocates
nothing): through the C ABI it gives the same bytes as fp8_lora_backward
with a caller-owned workspace, on consecutive calls that leave the fixed
scratch dirty for the next one (the second call smaller than the first),
for both output types; a problem too large for the scratch is refused."""

import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from workloads import qat_backward

pytestmark = pytest.mark.gpu


def _inputs(m, n, k, r, seed):
    d = qat_backward("cuda", m, n, k, r, seed)
    return d["dy"], d["x"], d["lora_b"], d["lora_a"]


def _with_workspace(dy, x, b, a, dtype):
    m, n = dy.shape
    k, r = x.shape[1], a.shape[0]
    ws = torch.empty(fb.fp8_lora_backward_workspace(m, n, k, r), dtype=torch.uint8, device="cuda")
    db = torch.empty((n, r), dtype=dtype, device="cuda")
    da = torch.empty((r, k), dtype=dtype, device="cuda")
    fb.fp8_lora_backward(dy, x, b, a, ws, db, da)
    return db, da


def _no_alloc(dy, x, b, a, dtype):
    n, k, r = dy.shape[1], x.shape[1], a.shape[0]
    db = torch.full((n, r), 7.0, dtype=dtype, device="cuda")
    da = torch.full((r, k), 7.0, dtype=dtype, device="cuda")
    fb.fp8_lora_backward_noalloc(dy, x, b, a, db, da)
    return db, da


def _same(u, v):
    w = torch.int32 if u.dtype == torch.float32 else torch.int16
    return torch.equal(u.view(w), v.view(w))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_no_alloc_matches_workspace_call(dtype):
    cases = [(2048, 1024, 1536, 32, 700), (300, 512, 256, 5, 701)]   # second call smaller
    for (m, n, k, r, seed) in cases:
        print(f"[no-alloc] lora backward m={m} n={n} k={k} r={r} {dtype}", flush=True)
        dy, x, b, a = _inputs(m, n, k, r, seed)
        got = _no_alloc(dy, x, b, a, dtype)
        want = _with_workspace(dy, x, b, a, dtype)
        torch.cuda.synchronize()
        assert _same(got[0], want[0]) and _same(got[1], want[1]), (m, n, k, r)


def test_no_alloc_refuses_oversize():
    m, n, k, r = 65536, 7168, 7168, 64
    assert fb.fp8_lora_backward_workspace(m, n, k, r) > fb.NOALLOC_SCRATCH_BYTES
    dy = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((n, r), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((r, k), dtype=torch.bfloat16, device="cuda")
    db = torch.empty((n, r), dtype=torch.bfloat16, device="cuda")
    da = torch.empty((r, k), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fb.Fp8Error) as e:
        fb.fp8_lora_backward_noalloc(dy, x, b, a, db, da)
    assert e.value.status == 6
