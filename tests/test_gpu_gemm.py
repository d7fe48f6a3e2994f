"""GPU parity of fp8_block_scaled_gemm and fp8_grouped_gemm against the oracle.

Tolerance (the stated error bound of the block-scaled GEMM): with
fp32 output, max|Y - ref32| / max|ref32| <= 2e-3 where ref32 is the oracle's
fp32-accumulated product of the same dequantized operands; the bf16 output
must equal RN_bf16 of the kernel's own fp32 output bit for bit and lie within
2^-8 |ref| + 2e-3 max|ref| elementwise.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_amax_amd as fb
from oracle import codec, gemm, quant
from tests.gpu_helpers import bf16_from_bits, to_np_u8
from workloads import (bf16_bits, dense_projection, expert_factors, expert_weights, moe_tokens, mx_small,
                       normal_bf16, qat_forward, zipf_routing)

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _q(x, kind):
    q, s = fb.quantize(x, kind)
    return q.view(torch.uint8), s


def _gemm(aq, sa, ka, bq, sb, kb, out=torch.float32):
    y = fb.block_scaled_gemm(aq, sa, ka, bq, sb, kb, out_dtype=out)
    torch.cuda.synchronize()
    return y


def _check_gemm(aq, sa, ka, bq, sb, kb, rows=None, label=""):
    print(f"[gemm] {label} A{tuple(aq.shape)} B{tuple(bq.shape)} {ka}x{kb}", flush=True)
    y32 = _gemm(aq, sa, ka, bq, sb, kb, torch.float32)
    y16 = _gemm(aq, sa, ka, bq, sb, kb, torch.bfloat16)
    aqn, san = aq.cpu().numpy(), sa.cpu().numpy()
    if rows is not None:
        aqn, san = aqn[rows], san[rows]
        y32n, y16n = y32.cpu().numpy()[rows], bf16_bits(y16)[rows]
    else:
        y32n, y16n = y32.cpu().numpy(), bf16_bits(y16)
    bqn, sbn = bq.cpu().numpy(), sb.cpu().numpy()
    ref = gemm.gemm_ref32(aqn, san, ka, bqn, sbn, kb)
    ref64 = gemm.gemm_ref64(aqn, san, ka, bqn, sbn, kb)
    err = gemm.normwise_rel_err(y32n, ref)
    err64 = gemm.normwise_rel_err(y32n, ref64)
    gap = gemm.normwise_rel_err(ref, ref64)
    print(f"[gemm] {label} normwise rel err {err:.3e} (vs fp64 {err64:.3e}; fp32 reference vs fp64 {gap:.3e})",
          flush=True)
    assert err <= TOL
    assert err64 <= TOL
    assert np.array_equal(y16n, codec.f32_to_bf16(y32n))
    yb = codec.bf16_to_f32(y16n).astype(np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + TOL * np.abs(ref).max()
    assert np.all(np.abs(yb - ref) <= bound)
    return err


def _rand_bf16(shape, sigma, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * sigma).to(torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [(128, 128, 128), (257, 384, 512), (1, 128, 256), (64, 256, 1024), (300, 512, 384),
                                   (700, 768, 384)])
def test_dense_f32_scales_small(m, n, k):
    aq, sa = _q(_rand_bf16((m, k), 1.0, m + k), "1x128")
    bq, sb = _q(_rand_bf16((n, k), 0.02, n + k), "128x128")
    _check_gemm(aq, sa, "1x128", bq, sb, "128x128", label=f"f32 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(64, 256, 512), (129, 128, 128), (200, 384, 640), (300, 512, 256)])
def test_mx_small(m, n, k):
    aq, sa = _q(_rand_bf16((m, k), 1.0, m), "1x32")
    bq, sb = _q(_rand_bf16((n, k), 1.0, n), "1x32")
    _check_gemm(aq, sa, "1x32", bq, sb, "1x32", label=f"mx {m}x{n}x{k}")


def test_mx_config():
    d = mx_small("cuda")
    aq, sa = _q(d["x"], "1x32")
    bq, sb = _q(d["w"], "1x32")
    _check_gemm(aq, sa, "1x32", bq, sb, "1x32", label="MXFP8 64x256x512")


def test_scale_placement_probe():
    """One K block of A and one N block of B carry a different scale: catches
    transposed or shifted scale indexing."""
    m, n, k = 128, 256, 512
    a = _rand_bf16((m, k), 1.0, 1)
    a[:, 256:384] *= 64
    b = _rand_bf16((n, k), 0.02, 2)
    b[128:256, :] *= 1 / 32
    b[0:128, 384:512] *= 16
    aq, sa = _q(a, "1x128")
    bq, sb = _q(b, "128x128")
    _check_gemm(aq, sa, "1x128", bq, sb, "128x128", label="scale placement")


def _check_whole_output64(aq, sa, ka, bq, sb, kb, label):
    """Every output element: normwise error against the fp64 product within
    the bound, and the bf16 output equal to RN_bf16 of the fp32 output."""
    y32 = _gemm(aq, sa, ka, bq, sb, kb, torch.float32)
    y16 = _gemm(aq, sa, ka, bq, sb, kb, torch.bfloat16)
    ref64 = gemm.gemm_ref64(aq.cpu().numpy(), sa.cpu().numpy(), ka, bq.cpu().numpy(), sb.cpu().numpy(), kb)
    y32n = y32.cpu().numpy()
    err64 = gemm.normwise_rel_err(y32n, ref64)
    print(f"[gemm] {label} whole output: normwise rel err vs fp64 {err64:.3e}", flush=True)
    assert err64 <= TOL
    assert np.array_equal(bf16_bits(y16), codec.f32_to_bf16(y32n))


def test_dense_projection_full():
    d = dense_projection("cuda")
    aq, sa = _q(d["x"], "1x128")
    bq, sb = _q(d["w"], "128x128")
    # random rows plus the first row of every 128-row tile (full rows: every n-tile)
    rows = np.union1d(np.random.default_rng(3).choice(4096, 256, replace=False), np.arange(0, 4096, 128))
    _check_gemm(aq, sa, "1x128", bq, sb, "128x128", rows=rows, label="dense projection 4096x2048x7168")
    _check_whole_output64(aq, sa, "1x128", bq, sb, "128x128", "dense projection 4096x2048x7168")


def test_qat_gemm_full_sampled():
    d = qat_forward("cuda")
    aq, sa = _q(d["x"], "1x128")
    wq, ws = fb.fake_quant_merge(d["w"], d["lora_b"], d["lora_a"])
    # random rows plus the last row of every 128-row tile (full rows: every n-tile)
    rows = np.union1d(np.random.default_rng(4).choice(8192, 96, replace=False), np.arange(127, 8192, 128))
    _check_gemm(aq, sa, "1x128", wq.view(torch.uint8), ws, "128x128", rows=rows,
                label="QAT 8192x7168x7168")
    _check_whole_output64(aq, sa, "1x128", wq.view(torch.uint8), ws, "128x128", "QAT 8192x7168x7168")


def test_determinism():
    aq, sa = _q(_rand_bf16((512, 1024), 1.0, 5), "1x128")
    bq, sb = _q(_rand_bf16((256, 1024), 0.02, 6), "128x128")
    y1 = _gemm(aq, sa, "1x128", bq, sb, "128x128")
    y2 = _gemm(aq, sa, "1x128", bq, sb, "128x128")
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    # a row slice computed on its own gives the same bytes
    y3 = _gemm(aq[128:384].contiguous(), sa[128:384].contiguous(), "1x128", bq, sb, "128x128")
    assert torch.equal(y3.view(torch.int32), y1[128:384].view(torch.int32))


# ------------------------------------------------------------------ grouped

def _grouped(aq, sa, bq, sb, bkind, off, out=torch.float32):
    y = fb.grouped_gemm(aq, sa, "1x128", bq, sb, bkind, off, out_dtype=out)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("n", [256, 384, 512])
@pytest.mark.parametrize("bkind", ["1x32", "128x128"])
def test_grouped_edge_cases(bkind, n):
    """Empty groups (first, middle, last), 1 row, tile-boundary sizes, and n
    both a multiple of 256 (128x256 tiles) and not (256x128 tiles)."""
    sizes = [0, 1, 127, 128, 129, 0, 300, 5, 0]
    g, k = len(sizes), 512
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    aq, sa = _q(_rand_bf16((total, k), 1.0, 10), "1x128")
    bs = [_q(_rand_bf16((n, k), 0.02 * (e + 1), 20 + e), bkind) for e in range(g)]
    bq = torch.stack([b[0] for b in bs]).contiguous()
    sb = torch.stack([b[1] for b in bs]).contiguous()
    offt = torch.from_numpy(off).cuda()
    print(f"[grouped] edge cases {bkind} sizes={sizes}", flush=True)
    y32 = _grouped(aq, sa, bq, sb, bkind, offt).cpu().numpy()
    y16 = bf16_bits(_grouped(aq, sa, bq, sb, bkind, offt, torch.bfloat16))
    ref = gemm.grouped_gemm_ref(aq.cpu().numpy(), sa.cpu().numpy(), "1x128", bq.cpu().numpy(),
                                sb.cpu().numpy(), bkind, off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        assert gemm.normwise_rel_err(y32[lo:hi], ref[e]) <= TOL, e
    assert np.array_equal(y16, codec.f32_to_bf16(y32))


@pytest.mark.parametrize("n,k", [(256, 384), (384, 640), (256, 1152), (384, 128)])
@pytest.mark.parametrize("bkind", ["1x32", "128x128"])
def test_grouped_scale_chunk_tails(bkind, n, k):
    """K steps (K / 128) that are not a multiple of the scale-chunk length
    (4 steps), with both tile shapes; K / 32 not a multiple of 16 (E8M0 B
    scales in dword pieces)."""
    sizes = [130, 0, 257, 64]
    g = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    aq, sa = _q(_rand_bf16((total, k), 1.0, 40 + k), "1x128")
    bs = [_q(_rand_bf16((n, k), 0.02 * (e + 1), 50 + e), bkind) for e in range(g)]
    bq = torch.stack([b[0] for b in bs]).contiguous()
    sb = torch.stack([b[1] for b in bs]).contiguous()
    offt = torch.from_numpy(off).cuda()
    print(f"[grouped] scale-chunk tails {bkind} n={n} k={k}", flush=True)
    y32 = _grouped(aq, sa, bq, sb, bkind, offt).cpu().numpy()
    ref = gemm.grouped_gemm_ref(aq.cpu().numpy(), sa.cpu().numpy(), "1x128", bq.cpu().numpy(),
                                sb.cpu().numpy(), bkind, off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        assert gemm.normwise_rel_err(y32[lo:hi], ref[e]) <= TOL, e


@pytest.mark.parametrize("bkind", ["1x32", "128x128"])
def test_grouped_many_groups(bkind):
    """1000 groups of random sizes 0..400 (a quarter of them empty): more
    groups than threads in the tile-order scan and a tile count that is not
    a multiple of the XCD count; every group is checked."""
    rng = np.random.default_rng(31)
    g, n, k = 1000, 256, 256
    sizes = rng.integers(0, 401, g)
    sizes[rng.choice(g, g // 4, replace=False)] = 0
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    aq, sa = _q(_rand_bf16((total, k), 1.0, 40), "1x128")
    bq, sb = _q(_rand_bf16((g * n, k), 0.02, 41), bkind)
    bq = bq.view(g, n, k)
    sb = sb.view(g, n, k // 32) if bkind == "1x32" else sb.view(g, n // 128, k // 128)
    offt = torch.from_numpy(off).cuda()
    print(f"[grouped] {g} groups {bkind} total rows {total}", flush=True)
    y32 = _grouped(aq, sa, bq, sb, bkind, offt).cpu().numpy()
    ref = gemm.grouped_gemm_ref(aq.cpu().numpy(), sa.cpu().numpy(), "1x128", bq.cpu().numpy(),
                                sb.cpu().numpy(), bkind, off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert gemm.normwise_rel_err(y32[lo:hi], ref[e]) <= TOL, e


@pytest.mark.parametrize("k", [512, 384])
def test_grouped_max_groups(k):
    """The largest group count the library takes (1024; the kernel keeps one
    m-tile prefix per group in LDS), E8M0 B with K a multiple of 512 (B scales
    in 16-byte pieces) and not; every nonempty group is checked."""
    rng = np.random.default_rng(33)
    g, n = 1024, 256
    sizes = rng.integers(0, 65, g)
    sizes[rng.choice(g, g // 8, replace=False)] = 0
    sizes[-1] = 3                                   # the last table entry holds rows
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    aq, sa = _q(_rand_bf16((total, k), 1.0, 60), "1x128")
    bq, sb = _q(_rand_bf16((g * n, k), 0.02, 61), "1x32")
    bq = bq.view(g, n, k)
    sb = sb.view(g, n, k // 32)
    offt = torch.from_numpy(off).cuda()
    print(f"[grouped] {g} groups k={k} total rows {total}", flush=True)
    y32 = _grouped(aq, sa, bq, sb, "1x32", offt).cpu().numpy()
    ref = gemm.grouped_gemm_ref(aq.cpu().numpy(), sa.cpu().numpy(), "1x128", bq.cpu().numpy(),
                                sb.cpu().numpy(), "1x32", off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert gemm.normwise_rel_err(y32[lo:hi], ref[e]) <= TOL, e


def _offset_copy(t, byte_offset):
    """A contiguous copy of t whose data starts byte_offset bytes past a
    256-byte aligned allocation (4-byte aligned, not 16-byte aligned)."""
    nbytes = t.numel() * t.element_size()
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=t.device)
    view = buf[byte_offset:byte_offset + nbytes].view(t.dtype).view(t.shape)
    view.copy_(t)
    assert view.data_ptr() % 16 == byte_offset % 16
    return view


@pytest.mark.parametrize("n", [256, 384])
def test_b_scale_load_paths_agree(n):
    """E8M0 B scales 16-byte aligned (loaded 16 bytes per column) and only
    4-byte aligned (loaded by dwords) give the same bytes, for the grouped
    fp32 x MXFP8 GEMM and the dense MXFP8 x MXFP8 GEMM, both tile shapes."""
    sizes = [200, 0, 129, 64]
    g, k = len(sizes), 1024
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    aq, sa = _q(_rand_bf16((total, k), 1.0, 70), "1x128")
    bq, sb = _q(_rand_bf16((g * n, k), 0.02, 71), "1x32")
    bq = bq.view(g, n, k)
    sb = sb.view(g, n, k // 32)
    offt = torch.from_numpy(off).cuda()
    print(f"[grouped] B-scale load paths n={n}", flush=True)
    y_vec = _grouped(aq, sa, bq, sb, "1x32", offt)
    y_dw = _grouped(aq, sa, bq, _offset_copy(sb, 4), "1x32", offt)
    assert torch.equal(y_vec.view(torch.int32), y_dw.view(torch.int32))
    ref = gemm.grouped_gemm_ref(aq.cpu().numpy(), sa.cpu().numpy(), "1x128", bq.cpu().numpy(),
                                sb.cpu().numpy(), "1x32", off)
    y = y_vec.cpu().numpy()
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        assert gemm.normwise_rel_err(y[lo:hi], ref[e]) <= TOL, e
    ma, sma = _q(_rand_bf16((300, k), 1.0, 72), "1x32")
    mb, smb = _q(_rand_bf16((n, k), 1.0, 73), "1x32")
    print(f"[gemm] MX x MX B-scale load paths n={n}", flush=True)
    d_vec = _gemm(ma, sma, "1x32", mb, smb, "1x32")
    d_dw = _gemm(ma, sma, "1x32", mb, _offset_copy(smb, 4), "1x32")
    assert torch.equal(d_vec.view(torch.int32), d_dw.view(torch.int32))
    ref = gemm.gemm_ref32(ma.cpu().numpy(), sma.cpu().numpy(), "1x32", mb.cpu().numpy(), smb.cpu().numpy(), "1x32")
    assert gemm.normwise_rel_err(d_vec.cpu().numpy(), ref) <= TOL


def test_grouped_moe_full():
    """Zipf(1.1) top-8 routing of 16384 tokens over 256 experts with gate||up
    MXFP8 weights (N = 4096, K = 7168); checked on the largest, smallest and
    a spread of groups (rows subsampled inside big groups)."""
    tok, off = zipf_routing()
    x = moe_tokens("cuda")
    xq, xs = _q(x, "1x128")
    idx = tok.cuda()
    aq = xq.index_select(0, idx).contiguous()
    sa = xs.index_select(0, idx).contiguous()
    del xq, xs, x
    fac = expert_factors()
    bq = torch.empty((256, 4096, 7168), dtype=torch.uint8, device="cuda")
    sb = torch.empty((256, 4096, 224), dtype=torch.uint8, device="cuda")
    for e in range(256):
        gate, up, _ = expert_weights(e, "cuda", fac)
        wq, ws = _q(torch.cat([gate, up], 0), "1x32")
        bq[e].copy_(wq)
        sb[e].copy_(ws)
    offt = off.cuda()
    print("[grouped] MoE 131072x4096x7168, 256 groups", flush=True)
    y = _grouped(aq, sa, bq, sb, "1x32", offt, torch.bfloat16)
    y32 = _grouped(aq, sa, bq, sb, "1x32", offt, torch.float32)
    offn = off.numpy()
    sizes = offn[1:] - offn[:-1]
    order = np.argsort(sizes)
    groups = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2])] +
                        list(np.random.default_rng(5).choice(256, 5, replace=False))))
    _check_sampled_groups(y, y32, aq, sa, bq, sb, offn, groups, np.random.default_rng(6), "gate||up")
    _check_group_boundaries(y, y32, aq, sa, bq, sb, offn, np.random.default_rng(9), "gate||up")


def _check_sampled_groups(y, y32, aq, sa, bq, sb, offn, groups, rng, label, per_group=64):
    """Sampled rows of the given groups against the oracle: the k-ordered
    fp32 reference (the bound), the fp64 product, and the gap between the
    two references; bf16 output equal to RN_bf16 of the fp32 output."""
    for g in groups:
        lo, hi = int(offn[g]), int(offn[g + 1])
        rows = np.arange(lo, hi) if hi - lo <= per_group else np.sort(rng.choice(np.arange(lo, hi), per_group,
                                                                                 replace=False))
        an, san = aq[rows].cpu().numpy(), sa[rows].cpu().numpy()
        bn, sbn = bq[g].cpu().numpy(), sb[g].cpu().numpy()
        ref = gemm.gemm_ref32(an, san, "1x128", bn, sbn, "1x32")
        ref64 = gemm.gemm_ref64(an, san, "1x128", bn, sbn, "1x32")
        got = y32[rows].cpu().numpy()
        err = gemm.normwise_rel_err(got, ref)
        err64 = gemm.normwise_rel_err(got, ref64)
        gap = gemm.normwise_rel_err(ref, ref64)
        print(f"[grouped] {label} group {g} rows {hi - lo} err {err:.3e} (vs fp64 {err64:.3e}; fp32 reference vs "
              f"fp64 {gap:.3e})", flush=True)
        assert err <= TOL
        assert err64 <= TOL
        assert np.array_equal(bf16_bits(y[rows]), codec.f32_to_bf16(got))


def _check_group_boundaries(y, y32, aq, sa, bq, sb, offn, rng, label, ncols=256):
    """Every group's first and last row (the rows next to the group
    boundaries, which start and end its m-tiles) on a sample of output
    columns, against the fp64 product of the same sampled operands (the
    kernel meets the 2e-3 bound against it as against the k-ordered fp32
    reference, which the sampled-group check above evaluates; the fp64
    product is a library matmul, so every group fits in the test's time);
    bf16 output equal to RN_bf16 of the fp32 output."""
    n = y32.shape[1]
    cols = np.sort(rng.choice(n, ncols, replace=False))
    colt = torch.from_numpy(cols).cuda()
    worst = 0.0
    for g in range(len(offn) - 1):
        lo, hi = int(offn[g]), int(offn[g + 1])
        if hi == lo:
            continue
        rows = sorted({lo, hi - 1})
        an, san = aq[rows].cpu().numpy(), sa[rows].cpu().numpy()
        bn = bq[g].index_select(0, colt).cpu().numpy()
        sbn = sb[g].index_select(0, colt).cpu().numpy()
        ref = gemm.gemm_ref64(an, san, "1x128", bn, sbn, "1x32")
        got = y32[rows].index_select(1, colt).cpu().numpy()
        err = gemm.normwise_rel_err(got, ref)
        worst = max(worst, err)
        assert err <= TOL, f"{label} group {g}: err {err:.3e}"
        assert np.array_equal(bf16_bits(y[rows].index_select(1, colt)), codec.f32_to_bf16(got))
    print(f"[grouped] {label}: first and last row of all {len(offn) - 1} groups on {ncols} columns, worst normwise "
          f"rel err {worst:.3e}", flush=True)


def test_grouped_moe_down_full():
    """The experts' down projection at its full shape: 131072 routed rows of
    the intermediate activations (K 2048, quantized per row in 1x128 tiles)
    against 256 MXFP8 down weights (N 7168, K 2048); the largest, smallest
    and median groups and 5 random ones are checked on sampled rows."""
    tok, off = zipf_routing()
    total = int(off[-1])
    h = normal_bf16((total, 2048), 1.0, 510, "cuda")
    hq, hs = _q(h, "1x128")
    del h
    fac = expert_factors()
    bq = torch.empty((256, 7168, 2048), dtype=torch.uint8, device="cuda")
    sb = torch.empty((256, 7168, 64), dtype=torch.uint8, device="cuda")
    for e in range(256):
        _, _, down = expert_weights(e, "cuda", fac)
        wq, ws = _q(down, "1x32")
        bq[e].copy_(wq)
        sb[e].copy_(ws)
    offt = off.cuda()
    print("[grouped] MoE down projection 131072x7168x2048, 256 groups", flush=True)
    y = _grouped(hq, hs, bq, sb, "1x32", offt, torch.bfloat16)
    y32 = _grouped(hq, hs, bq, sb, "1x32", offt, torch.float32)
    offn = off.numpy()
    sizes = offn[1:] - offn[:-1]
    order = np.argsort(sizes)
    groups = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2])] +
                        list(np.random.default_rng(7).choice(256, 5, replace=False))))
    _check_sampled_groups(y, y32, hq, hs, bq, sb, offn, groups, np.random.default_rng(8), "down")
    _check_group_boundaries(y, y32, hq, hs, bq, sb, offn, np.random.default_rng(10), "down")


# ------------------------------------------------------------ gathered rows

@pytest.mark.parametrize("bkind", ["1x32", "128x128"])
def test_grouped_gather_small(bkind):
    """Rows gathered through row_index equal the oracle on the permuted copy
    and, bit for bit, the plain grouped kernel run on that copy."""
    rng = np.random.default_rng(90)
    tokens, g, n, k, top = 300, 9, 256, 512, 2
    experts = np.stack([rng.choice(g - 2, top, replace=False) for _ in range(tokens)])   # groups 7, 8 empty
    flat = experts.reshape(-1)
    tok = np.repeat(np.arange(tokens), top)
    order = np.lexsort((tok, flat))
    row_index = tok[order].astype(np.int32)
    off = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=g))]).astype(np.int32)
    aq, sa = _q(_rand_bf16((tokens, k), 1.0, 91), "1x128")
    bq, sb = _q(_rand_bf16((g * n, k), 0.02, 92), bkind)
    bq = bq.view(g, n, k)
    sb = sb.view(g, n, k // 32) if bkind == "1x32" else sb.view(g, n // 128, k // 128)
    offt = torch.from_numpy(off).cuda()
    idx = torch.from_numpy(row_index).cuda()
    print(f"[grouped] gather {bkind} tokens {tokens} rows {len(row_index)}", flush=True)
    y = fb.grouped_gemm(aq, sa, "1x128", bq, sb, bkind, offt, out_dtype=torch.float32, row_index=idx)
    y16 = fb.grouped_gemm(aq, sa, "1x128", bq, sb, bkind, offt, row_index=idx)
    ap, sp = aq.index_select(0, idx.long()).contiguous(), sa.index_select(0, idx.long()).contiguous()
    yp = fb.grouped_gemm(ap, sp, "1x128", bq, sb, bkind, offt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), yp.view(torch.int32))
    ref = gemm.grouped_gemm_ref(ap.cpu().numpy(), sp.cpu().numpy(), "1x128", bq.cpu().numpy(), sb.cpu().numpy(),
                                bkind, off)
    y32 = y.cpu().numpy()
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert gemm.normwise_rel_err(y32[lo:hi], ref[e]) <= TOL, e
    assert np.array_equal(bf16_bits(y16), codec.f32_to_bf16(y32))


def test_grouped_gather_moe_full():
    """The MoE gate||up GEMM (131072 routed rows over 256 experts) reading the
    16384 per-token quantized rows through row_index gives the same bytes as
    the grouped GEMM on the materialized permuted copy."""
    tok, off = zipf_routing()
    x = moe_tokens("cuda")
    xq, xs = _q(x, "1x128")
    del x
    fac = expert_factors()
    bq = torch.empty((256, 4096, 7168), dtype=torch.uint8, device="cuda")
    sb = torch.empty((256, 4096, 224), dtype=torch.uint8, device="cuda")
    for e in range(256):
        gate, up, _ = expert_weights(e, "cuda", fac)
        wq, ws = _q(torch.cat([gate, up], 0), "1x32")
        bq[e].copy_(wq)
        sb[e].copy_(ws)
    offt = off.cuda()
    idx = tok.to(torch.int32).cuda()
    print("[grouped] gather MoE 131072x4096x7168", flush=True)
    y = fb.grouped_gemm(xq, xs, "1x128", bq, sb, "1x32", offt, row_index=idx)
    ap = xq.index_select(0, idx.long()).contiguous()
    sp = xs.index_select(0, idx.long()).contiguous()
    yp = fb.grouped_gemm(ap, sp, "1x128", bq, sb, "1x32", offt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yp.view(torch.int16))
