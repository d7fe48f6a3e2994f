"""The hot path captured into a HIP graph: every replay equals an eager run.

The library's entry points only enqueue kernels on the caller's stream (no
allocation, memset, copy or synchronization; the NVFP4 call clears its
tensor amax with a kernel of its own), so a caller may capture them.  Each
test captures a sequence of calls on static buffers once, then three times:
writes new inputs into those buffers with eager work, runs the same calls
eagerly into separate outputs, synchronizes, replays the graph, and compares
every output byte with the eager result.
"""

import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from workloads import normal_bf16

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _replays(capture, refill, outputs, eager):
    """capture() enqueues the calls on static buffers; refill(i) writes input
    set i into them; eager() runs the calls into fresh outputs and returns
    them in the order of ``outputs``."""
    torch.cuda.synchronize()
    capture()                      # warm-up outside the graph
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    for i in range(3):
        refill(i)
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        for o in outputs:
            o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("out%d" % j for j in range(len(outputs))), outputs, want):
            assert _same(got, ref), f"replay {i}: {name} differs from the eager call"
        print(f"[graph] replay {i}: {len(outputs)} outputs equal the eager calls", flush=True)


def test_graph_quantize_then_grouped_gemm():
    """1x128 activation quantize, then the grouped GEMM over MXFP8 experts."""
    tokens, k, n, experts = 384, 1024, 512, 4
    x = torch.zeros((tokens, k), dtype=torch.bfloat16, device="cuda")
    wq, ws = fb.quantize(normal_bf16((experts * n, k), 0.02, 700, "cuda"), "1x32")
    wq = wq.view(torch.uint8).view(experts, n, k)
    ws = ws.view(experts, n, k // 32)
    offsets = torch.tensor([0, 100, 101, 300, tokens], dtype=torch.int32, device="cuda")
    q = torch.empty((tokens, k), dtype=torch.uint8, device="cuda")
    s = torch.empty((tokens, k // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((tokens, n), dtype=torch.bfloat16, device="cuda")

    def capture():
        fb.fp8_block_quantize(x, "1x128", "ceil", q, s)
        fb.fp8_grouped_gemm(q, s, "1x128", wq, ws, "1x32", offsets, y)

    def refill(i):
        x.copy_(normal_bf16((tokens, k), 1.0, 710 + i, "cuda"))

    def eager():
        q2, s2 = fb.quantize(x, "1x128")
        y2 = fb.grouped_gemm(q2.view(torch.uint8), s2, "1x128", wq, ws, "1x32", offsets)
        return q2, s2, y2

    _replays(capture, refill, [q, s, y], eager)


def test_graph_batch_quantize_then_dense_gemm():
    """W (128x128) and X (1x128) in one batched launch, then the dense GEMM."""
    m, n, k = 256, 384, 1024
    w = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    wq = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    wsc = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda")
    xq = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    xsc = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

    def capture():
        fb.fp8_block_quantize_batch([(w, "128x128", "ceil", wq, wsc), (x, "1x128", "ceil", xq, xsc)])
        fb.fp8_block_scaled_gemm(xq, xsc, "1x128", wq, wsc, "128x128", y)

    def refill(i):
        w.copy_(normal_bf16((n, k), 0.02, 720 + i, "cuda"))
        x.copy_(normal_bf16((m, k), 1.0, 730 + i, "cuda"))

    def eager():
        wq2, ws2 = fb.quantize(w, "128x128")
        xq2, xs2 = fb.quantize(x, "1x128")
        y2 = fb.block_scaled_gemm(xq2.view(torch.uint8), xs2, "1x128", wq2.view(torch.uint8), ws2, "128x128")
        return wq2, ws2, xq2, xs2, y2

    _replays(capture, refill, [wq, wsc, xq, xsc, y], eager)


def test_graph_nvfp4_quantize():
    """The three-kernel NVFP4 call: its amax zero fill and atomic maxima run
    again on every replay."""
    rows, cols, rpt = 256, 512, 64
    x = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    t = rows // rpt
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    bs = torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda")
    gs = torch.empty(t, dtype=torch.float32, device="cuda")
    am = torch.empty(t, dtype=torch.float32, device="cuda")

    def capture():
        fb.fp8_nvfp4_quantize(x, rpt, q, bs, gs, am)

    def refill(i):
        x.copy_(normal_bf16((rows, cols), 0.02 * (i + 1), 740 + i, "cuda"))

    def eager():
        q2 = torch.empty_like(q)
        bs2 = torch.empty_like(bs)
        gs2 = torch.empty_like(gs)
        am2 = torch.empty_like(am)
        fb.fp8_nvfp4_quantize(x, rpt, q2, bs2, gs2, am2)
        return q2, bs2, gs2, am2

    _replays(capture, refill, [q, bs, gs, am], eager)
