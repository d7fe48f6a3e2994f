"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every function include/fp8blk.h declares, and
its argument validation returns the documented status codes before any
device work (the checks below never reach a kernel launch).
"""

import ctypes
import os
import re

import pytest

import block_scaled_fp8_amax_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")

OK, INVALID, SHAPE, ALIGN, UNSUP, HIPERR = 0, 1, 2, 3, 4, 5
A16 = 0x10000          # a fake, 16-byte aligned address (never dereferenced)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fp8_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.library_path):
        pytest.fail("libfp8blk.so is not built (run __graft_entry__.build())")
    return fb.library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == {"fp8_block_quantize", "fp8_block_quantize_batch", "fp8_block_dequantize",
                          "fp8_fake_quant_merge",
                          "fp8_block_scaled_gemm", "fp8_grouped_gemm", "fp8_grouped_gemm_gather",
                          "fp8_lora_backward", "fp8_lora_backward_workspace", "fp8_lora_backward_noalloc",
                          "fp8_nvfp4_quantize", "fp8_nvfp4_dequantize",
                          "fp8_status_string", "fp8_abi_version"}
    raw = ctypes.CDLL(fb.library_path)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(lib):
    assert lib.fp8_abi_version() == 6
    for s in range(7):
        assert len(lib.fp8_status_string(s)) > 0
    assert lib.fp8_status_string(99) == b"unknown status"


def test_quantize_validation(lib):
    q = lib.fp8_block_quantize
    assert q(A16, 4, 64, 7, 0, A16, A16, None, None) == INVALID           # unknown kind
    assert q(A16, 4, 64, 0, 5, A16, A16, None, None) == INVALID           # unknown rule (1x32)
    assert q(A16, 4, 48, 0, 0, A16, A16, None, None) == SHAPE             # 48 % 32
    assert q(A16, 4, 64, 1, 0, A16, A16, None, None) == SHAPE             # 64 % 128
    assert q(A16, 64, 128, 2, 0, A16, A16, None, None) == SHAPE           # rows % 128
    assert q(A16, -1, 128, 1, 0, A16, A16, None, None) == SHAPE
    assert q(None, 0, 128, 1, 0, None, None, None, None) == OK            # empty: nothing to do
    assert q(None, 4, 0, 0, 0, None, None, None, None) == OK
    assert q(None, 4, 128, 1, 0, A16, A16, None, None) == INVALID         # null input
    assert q(A16 + 8, 4, 128, 1, 0, A16, A16, None, None) == ALIGN        # x not 16-B aligned
    assert q(A16, 4, 128, 1, 0, A16, A16 + 2, None, None) == ALIGN        # fp32 scale not 4-B aligned
    assert q(A16, 4, 128, 1, 0, A16, A16, A16 + 4, None) == ALIGN         # xdq not 16-B aligned
    assert q(A16, 1 << 40, 1 << 30, 1, 0, A16, A16, None, None) == SHAPE   # element count overflows


def test_quantize_batch_validation(lib):
    Job = fb.QuantizeJob
    b = lib.fp8_block_quantize_batch

    def arr(*jobs):
        a = (Job * max(1, len(jobs)))()
        for i, j in enumerate(jobs):
            a[i] = j
        return a

    good = Job(A16, 4, 128, 1, 0, A16, A16, None)
    assert ctypes.sizeof(Job) == 56
    assert b(None, 0, None) == OK                                            # nothing to do
    assert b(arr(), -1, None) == INVALID
    assert b(arr(*([good] * 17)), 17, None) == INVALID                       # more than 16 jobs
    assert b(None, 1, None) == INVALID
    assert b(arr(good, Job(A16, 4, 48, 0, 0, A16, A16, None)), 2, None) == SHAPE     # second job: 48 % 32
    assert b(arr(Job(A16, 4, 128, 7, 0, A16, A16, None), good), 2, None) == INVALID  # unknown kind
    assert b(arr(good, Job(A16, 64, 128, 2, 0, A16, A16, None)), 2, None) == SHAPE   # 128x128 rows % 128
    assert b(arr(good, Job(A16 + 8, 4, 128, 1, 0, A16, A16, None)), 2, None) == ALIGN
    assert b(arr(Job(None, 0, 128, 1, 0, None, None, None)), 1, None) == OK          # empty job only


def test_dequantize_validation(lib):
    d = lib.fp8_block_dequantize
    assert d(A16, A16, 4, 64, 7, A16, None) == INVALID             # unknown kind
    assert d(A16, A16, 4, 48, 0, A16, None) == SHAPE               # 48 % 32
    assert d(A16, A16, 4, 64, 1, A16, None) == SHAPE               # 64 % 128
    assert d(A16, A16, 64, 128, 2, A16, None) == SHAPE             # rows % 128
    assert d(A16, A16, -1, 128, 1, A16, None) == SHAPE
    assert d(A16, A16, 1 << 22, 1 << 13, 1, A16, None) == SHAPE    # rows * cols / 8 >= 2^32
    assert d(None, None, 0, 128, 1, None, None) == OK              # empty
    assert d(None, A16, 4, 128, 1, A16, None) == INVALID           # null codes
    assert d(A16, A16, 4, 128, 1, None, None) == INVALID           # null output
    assert d(A16 + 4, A16, 4, 128, 1, A16, None) == ALIGN          # codes not 16-B aligned
    assert d(A16, A16 + 2, 4, 128, 1, A16, None) == ALIGN          # fp32 scale not 4-B aligned
    assert d(A16, A16, 4, 128, 1, A16 + 8, None) == ALIGN          # output not 16-B aligned


def test_merge_validation(lib):
    m = lib.fp8_fake_quant_merge
    assert m(A16, A16, A16, 128, 128, 0, A16, A16, None, None) == INVALID    # rank 0
    assert m(A16, A16, A16, 128, 128, 65, A16, A16, None, None) == INVALID   # rank > 64
    assert m(A16, A16, A16, 100, 128, 16, A16, A16, None, None) == SHAPE
    assert m(A16, A16, A16, 0, 128, 16, A16, A16, None, None) == OK
    assert m(A16, None, A16, 128, 128, 16, A16, A16, None, None) == INVALID
    assert m(A16 + 2, A16, A16, 128, 128, 16, A16, A16, None, None) == ALIGN
    assert m(A16, A16 + 2, A16, 128, 128, 16, A16, A16, None, None) == ALIGN    # lora_b: 4 B (dword reads)
    assert m(A16, A16, A16 + 2, 128, 128, 16, A16, A16, None, None) == ALIGN    # lora_a: 4 B


def test_gemm_validation(lib):
    g = lib.fp8_block_scaled_gemm
    assert g(A16, A16, 1, A16, A16, 1, 8, 128, 128, A16, 0, None) == UNSUP       # (1x128, 1x128)
    assert g(A16, A16, 0, A16, A16, 2, 8, 128, 128, A16, 0, None) == UNSUP
    assert g(A16, A16, 9, A16, A16, 2, 8, 128, 128, A16, 0, None) == INVALID
    assert g(A16, A16, 1, A16, A16, 2, 8, 128, 128, A16, 3, None) == INVALID     # bad out type
    assert g(A16, A16, 1, A16, A16, 2, 8, 100, 128, A16, 0, None) == SHAPE
    assert g(A16, A16, 1, A16, A16, 2, 8, 128, 96, A16, 0, None) == SHAPE
    assert g(A16, A16, 1, A16, A16, 2, 0, 128, 128, None, 0, None) == OK         # m = 0
    assert g(A16, A16, 1, A16, A16, 2, 8, 128, 0, A16, 0, None) == SHAPE         # empty reduction
    assert g(A16 + 1, A16, 1, A16, A16, 2, 8, 128, 128, A16, 0, None) == ALIGN
    assert g(A16, A16, 0, A16, A16 + 1, 0, 8, 128, 128, A16, 0, None) == ALIGN    # E8M0 scales: 4 B
    assert g(A16, A16, 1, A16, A16, 2, 8, 128, 128, A16 + 4, 1, None) == ALIGN    # y: 16 B
    assert g(A16, A16, 1, A16, A16, 2, 8, 128, 128, A16 + 2, 0, None) == ALIGN
    assert g(A16, A16, 1, A16, A16, 2, 8, 128, (1 << 24) + 128, A16, 0, None) == SHAPE   # K beyond 2^24
    assert g(A16, A16, 1, A16, A16, 2, 1 << 31, 128, 128, A16, 0, None) == SHAPE        # M beyond 2^31 - 1


def test_grouped_validation(lib):
    g = lib.fp8_grouped_gemm
    assert g(A16, A16, 1, A16, A16, 0, A16, 0, 8, 128, 128, A16, 0, None) == INVALID     # no groups
    assert g(A16, A16, 1, A16, A16, 0, A16, 1025, 8, 128, 128, A16, 0, None) == INVALID  # too many
    assert g(A16, A16, 0, A16, A16, 0, A16, 4, 8, 128, 128, A16, 0, None) == UNSUP       # A must be 1x128
    assert g(A16, A16, 1, A16, A16, 1, A16, 4, 8, 128, 128, A16, 0, None) == UNSUP       # B 1x128
    assert g(A16, A16, 1, A16, A16, 0, A16, 4, 8, 130, 128, A16, 0, None) == SHAPE
    assert g(A16, A16, 1, A16, A16, 0, A16, 4, 0, 128, 128, A16, 0, None) == OK          # no rows
    assert g(A16, A16, 1, A16, A16, 0, None, 4, 8, 128, 128, A16, 0, None) == INVALID
    assert g(A16, A16, 1, A16, A16, 0, A16 + 2, 4, 8, 128, 128, A16, 0, None) == ALIGN
    assert g(A16, A16, 1, A16, A16, 0, A16, 4, 8, 128, (1 << 24) + 128, A16, 0, None) == SHAPE   # K beyond 2^24


def test_grouped_gather_validation(lib):
    g = lib.fp8_grouped_gemm_gather
    assert g(A16, A16, 1, 16, None, A16, A16, 0, A16, 4, 8, 128, 128, A16, 0, None) == INVALID   # no row_index
    assert g(A16, A16, 1, 16, A16 + 2, A16, A16, 0, A16, 4, 8, 128, 128, A16, 0, None) == ALIGN  # row_index 4 B
    assert g(A16, A16, 1, 1 << 20, A16, A16, A16, 0, A16, 4, 8, 128, 1 << 13, A16, 0, None) == SHAPE  # A > 2^32 B
    assert g(A16, A16, 1, 0, A16, A16, A16, 0, A16, 4, 8, 128, 128, A16, 0, None) == SHAPE       # no A rows
    assert g(A16, A16, 1, 0, None, A16, A16, 0, A16, 4, 0, 128, 128, A16, 0, None) == OK          # no grouped rows
    assert g(A16, A16, 0, 16, A16, A16, A16, 0, A16, 4, 8, 128, 128, A16, 0, None) == UNSUP       # A must be 1x128


def test_lora_backward_workspace(lib):
    out = ctypes.c_size_t(0)
    w = lib.fp8_lora_backward_workspace
    assert w(64, 256, 384, 16, None) == INVALID
    assert w(64, 256, 384, 0, ctypes.byref(out)) == INVALID            # rank 0
    assert w(64, 256, 384, 65, ctypes.byref(out)) == INVALID           # rank > 64
    assert w(64, 200, 384, 16, ctypes.byref(out)) == SHAPE
    assert w(-1, 256, 384, 16, ctypes.byref(out)) == SHAPE
    assert w(64, 256, 1 << 25, 16, ctypes.byref(out)) == SHAPE
    assert w(64, 256, 384, 16, ctypes.byref(out)) == OK
    small = out.value
    assert small > 0 and small % 256 == 0
    assert w(8192, 7168, 7168, 16, ctypes.byref(out)) == OK
    assert small < out.value < 64 << 20                                 # a few MiB at the full QAT size
    assert w(8192, 7168, 7168, 64, ctypes.byref(out)) == OK and out.value < 256 << 20
    assert w(0, 256, 384, 16, ctypes.byref(out)) == OK and out.value > 0


def test_lora_backward_validation(lib):
    b = lib.fp8_lora_backward
    need = ctypes.c_size_t(0)
    assert lib.fp8_lora_backward_workspace(64, 256, 384, 16, ctypes.byref(need)) == OK
    ws = need.value
    args = [A16, A16, A16, A16, 64, 256, 384, 16, A16, ws, A16, A16, 0, None]

    def call(**kw):
        a = list(args)
        names = ["dy", "x", "lb", "la", "m", "n", "k", "r", "wsp", "wsb", "db", "da", "out", "st"]
        for key, v in kw.items():
            a[names.index(key)] = v
        return b(*a)

    assert call(out=2) == INVALID                                      # unknown output type
    assert call(r=0) == INVALID and call(r=65) == INVALID
    assert call(n=100) == SHAPE and call(k=64) == SHAPE and call(m=-1) == SHAPE
    assert call(n=0, k=0, dy=None, x=None, lb=None, la=None, wsp=None, db=None, da=None) == OK
    assert call(wsp=None) == INVALID
    assert call(wsb=ws - 1) == INVALID                                 # workspace too small
    assert call(dy=None) == INVALID and call(x=None) == INVALID
    assert call(lb=None) == INVALID and call(da=None) == INVALID
    assert call(dy=A16 + 8) == ALIGN and call(x=A16 + 2) == ALIGN
    assert call(la=A16 + 4) == ALIGN and call(lb=A16 + 1) == ALIGN
    assert call(wsp=A16 + 128) == ALIGN                                 # workspace: 256 B
    assert call(db=A16 + 2, out=1) == ALIGN                             # fp32 gradients: 4 B
    assert call(db=A16 + 1) == ALIGN


def test_lora_backward_noalloc_validation(lib):
    """The no-allocation LoRA backward checks its arguments like
    fp8_lora_backward and refuses problems whose workspace exceeds the fixed
    scratch (before touching a device)."""
    TOO_LARGE = 6
    f = lib.fp8_lora_backward_noalloc

    def call(m=64, n=128, k=256, r=16, dy=A16, x=A16, lb=A16, la=A16, db=A16, da=A16, out=0):
        return f(dy, x, lb, la, m, n, k, r, db, da, out, None)

    assert call(r=0) == INVALID and call(r=65) == INVALID
    assert call(n=100) == SHAPE and call(m=-1) == SHAPE
    assert call(out=2) == INVALID
    assert call(n=0, k=0) == OK
    assert call(dy=None) == INVALID and call(lb=None) == INVALID
    assert call(dy=A16 + 8) == ALIGN and call(db=A16 + 2, out=1) == ALIGN
    ws = ctypes.c_size_t(0)
    m, n, k, r = 8192, 7168, 7168, 64
    assert lib.fp8_lora_backward_workspace(m, n, k, r, ctypes.byref(ws)) == OK
    assert ws.value <= fb.NOALLOC_SCRATCH_BYTES                # the documented fit
    assert lib.fp8_lora_backward_workspace(4 * m, n, k, r, ctypes.byref(ws)) == OK
    assert ws.value > fb.NOALLOC_SCRATCH_BYTES
    assert call(m=4 * m, n=n, k=k, r=r) == TOO_LARGE


def test_python_binding_rejects_host_tensors(lib):
    """Host tensors never reach the library: their pointers are not device
    addresses.  (The status path of the binding is covered on the GPU.)"""
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    q = torch.zeros((4, 64), dtype=torch.uint8)
    s = torch.zeros((4, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="on a GPU"):
        fb.fp8_block_quantize(x, "1x32", "ceil", q, s)
    w = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on a GPU"):
        fb.fp8_block_scaled_gemm(torch.zeros((4, 128), dtype=torch.uint8), torch.zeros((4, 1), dtype=torch.float32),
                                 "1x128", torch.zeros((128, 128), dtype=torch.uint8),
                                 torch.zeros((1, 1), dtype=torch.float32), "128x128",
                                 torch.zeros((4, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="on a GPU"):
        fb.fp8_fake_quant_merge(w, torch.zeros((128, 4), dtype=torch.bfloat16),
                                torch.zeros((4, 128), dtype=torch.bfloat16), torch.zeros((128, 128), dtype=torch.uint8),
                                torch.zeros((1, 1), dtype=torch.float32))


def test_python_binding_checks_dtypes_and_sizes(lib):
    """Wrong dtypes and buffers smaller than the sizes passed with them are
    refused before any device pointer is used (checked before the device)."""
    import torch
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    x = torch.zeros((4, 256), dtype=bf)
    q = torch.zeros((4, 256), dtype=u8)
    with pytest.raises(ValueError, match="x has dtype"):
        fb.fp8_block_quantize(x.float(), "1x128", "ceil", q, torch.zeros((4, 2), dtype=f32))
    with pytest.raises(ValueError, match="q holds 512 elements"):
        fb.fp8_block_quantize(x, "1x128", "ceil", torch.zeros((2, 256), dtype=u8), torch.zeros((4, 2), dtype=f32))
    with pytest.raises(ValueError, match="scale has dtype"):
        fb.fp8_block_quantize(x, "1x32", "ceil", q, torch.zeros((4, 8), dtype=f32))
    with pytest.raises(ValueError, match="scale holds 7 elements"):
        fb.fp8_block_quantize(x, "1x128", "ceil", q, torch.zeros((7,), dtype=f32))
    with pytest.raises(ValueError, match="job 0: xdq"):
        fb.fp8_block_quantize_batch([(x, "1x32", "ceil", q, torch.zeros((4, 8), dtype=u8), torch.zeros((4, 255), dtype=bf)),
                                     (x, "1x128", "ceil", q, torch.zeros((4, 2), dtype=f32))])
    with pytest.raises(ValueError, match="x holds"):
        fb.fp8_block_dequantize(q, torch.zeros((4, 8), dtype=u8), "1x32", torch.zeros((4, 128), dtype=bf))
    a = torch.zeros((8, 256), dtype=u8)
    b = torch.zeros((256, 256), dtype=u8)
    sa, sb = torch.zeros((8, 2), dtype=f32), torch.zeros((2, 2), dtype=f32)
    with pytest.raises(ValueError, match="y holds"):
        fb.fp8_block_scaled_gemm(a, sa, "1x128", b, sb, "128x128", torch.zeros((8, 255), dtype=bf))
    with pytest.raises(ValueError, match="b_scale holds"):
        fb.fp8_block_scaled_gemm(a, sa, "1x128", b, sb[:1], "128x128", torch.zeros((8, 256), dtype=bf))
    with pytest.raises(ValueError, match="y has dtype"):
        fb.fp8_block_scaled_gemm(a, sa, "1x128", b, sb, "128x128", torch.zeros((8, 256), dtype=torch.float16))
    bg = torch.zeros((3, 256, 256), dtype=u8)
    sbg = torch.zeros((3, 256, 8), dtype=u8)
    offs = torch.zeros((4,), dtype=torch.int32)
    with pytest.raises(ValueError, match="b_scale holds"):
        fb.fp8_grouped_gemm(a, sa, "1x128", bg, sbg[:2], "1x32", offs, torch.zeros((8, 256), dtype=bf))
    with pytest.raises(ValueError, match="group_offsets holds"):
        fb.fp8_grouped_gemm(a, sa, "1x128", bg, sbg, "1x32", offs[:3], torch.zeros((8, 256), dtype=bf))
    with pytest.raises(ValueError, match="y holds"):
        fb.fp8_grouped_gemm_gather(a, sa, "1x128", torch.zeros((9,), dtype=torch.int32), bg, sbg, "1x32", offs,
                                   torch.zeros((8, 256), dtype=bf))
    with pytest.raises(ValueError, match="block_scale holds"):
        fb.fp8_nvfp4_quantize(x, 4, torch.zeros((4, 128), dtype=u8), torch.zeros((4, 15), dtype=u8),
                              torch.zeros((1,), dtype=f32), torch.zeros((1,), dtype=f32))
    with pytest.raises(ValueError, match="global_scale holds"):
        fb.fp8_nvfp4_dequantize(torch.zeros((4, 128), dtype=u8), torch.zeros((4, 16), dtype=u8),
                                torch.zeros((0,), dtype=f32), 2, x)
    dy, xx = torch.zeros((8, 128), dtype=bf), torch.zeros((8, 256), dtype=bf)
    lb, la = torch.zeros((128, 4), dtype=bf), torch.zeros((4, 256), dtype=bf)
    with pytest.raises(ValueError, match="d_lora_a holds"):
        fb.fp8_lora_backward(dy, xx, lb, la, torch.zeros((1024,), dtype=u8), torch.zeros((128, 4), dtype=bf),
                             torch.zeros((4, 255), dtype=bf))


def test_python_binding_checks_shapes(lib):
    """Operands whose shapes disagree with the sizes the library derives
    (a wider B row, LoRA factors of another rank or width, a transposed
    scale array) are refused: the kernels would read them with the wrong
    strides."""
    import torch
    bf, u8, f32 = torch.bfloat16, torch.uint8, torch.float32
    a = torch.zeros((8, 256), dtype=u8)
    sa = torch.zeros((8, 2), dtype=f32)
    b = torch.zeros((128, 256), dtype=u8)
    sb = torch.zeros((1, 2), dtype=f32)
    y = torch.zeros((8, 128), dtype=bf)
    with pytest.raises(ValueError, match="b_q has shape"):
        fb.fp8_block_scaled_gemm(a, sa, "1x128", torch.zeros((128, 384), dtype=u8), sb, "128x128", y)
    with pytest.raises(ValueError, match="a_scale has shape"):
        fb.fp8_block_scaled_gemm(a, torch.zeros((2, 8), dtype=f32), "1x128", b, sb, "128x128", y)
    with pytest.raises(ValueError, match="b_scale has shape"):
        fb.fp8_block_scaled_gemm(a, sa, "1x128", b, torch.zeros((2, 1), dtype=f32), "128x128", y)
    with pytest.raises(ValueError, match="y has shape"):
        fb.fp8_block_scaled_gemm(a, sa, "1x128", b, sb, "128x128", torch.zeros((16, 64), dtype=bf))
    bg = torch.zeros((3, 128, 256), dtype=u8)
    sbg = torch.zeros((3, 128, 8), dtype=u8)
    offs = torch.zeros((4,), dtype=torch.int32)
    with pytest.raises(ValueError, match="b_q has shape"):
        fb.fp8_grouped_gemm(a, sa, "1x128", torch.zeros((3, 128, 384), dtype=u8), sbg, "1x32", offs, y)
    with pytest.raises(ValueError, match="b_scale has shape"):
        fb.fp8_grouped_gemm(a, sa, "1x128", bg, torch.zeros((3, 8, 128), dtype=u8), "1x32", offs, y)
    w = torch.zeros((128, 256), dtype=bf)
    q = torch.zeros((128, 256), dtype=u8)
    s = torch.zeros((1, 2), dtype=f32)
    with pytest.raises(ValueError, match="lora_b"):
        fb.fp8_fake_quant_merge(w, torch.zeros((128, 8), dtype=bf), torch.zeros((4, 256), dtype=bf), q, s)
    with pytest.raises(ValueError, match="lora_b"):
        fb.fp8_fake_quant_merge(w, torch.zeros((128, 4), dtype=bf), torch.zeros((4, 512), dtype=bf), q, s)
    with pytest.raises(ValueError, match="q has shape"):
        fb.fp8_block_quantize(torch.zeros((4, 256), dtype=bf), "1x128", "ceil", torch.zeros((8, 128), dtype=u8),
                              torch.zeros((4, 2), dtype=f32))
    with pytest.raises(ValueError, match="block_scale has shape"):
        fb.fp8_nvfp4_dequantize(torch.zeros((4, 16), dtype=u8), torch.zeros((2, 4), dtype=u8),
                                torch.zeros((1,), dtype=f32), 4, torch.zeros((4, 32), dtype=bf))


def test_routed_expert_name_rule():
    yes = ["model.layers.3.mlp.experts.0.gate_proj.weight",
           "model.layers.60.mlp.experts.255.up_proj.weight",
           "layers.1.mlp.experts.7.down_proj.weight",
           "language_model.model.layers.12.mlp.experts.31.down_proj.weight"]
    no = ["model.layers.3.mlp.gate.weight",                       # router
          "model.layers.3.mlp.shared_experts.gate_proj.weight",   # shared expert
          "model.layers.0.mlp.gate_proj.weight",                  # dense MLP
          "model.layers.3.self_attn.q_proj.weight",
          "model.layers.3.mlp.experts.0.gate_proj.weight_scale_inv",
          "model.layers.3.mlp.experts.0.gate_proj.bias",
          "model.embed_tokens.weight"]
    assert all(fb.is_routed_expert_weight(n) for n in yes)
    assert not any(fb.is_routed_expert_weight(n) for n in no)


def test_quantize_state_dict_rejects_other_formats():
    with pytest.raises(ValueError):
        fb.quantize_state_dict({}, fmt="mxfp4")
    assert fb.quantize_state_dict({"a": 1}, fmt="nvfp4") == {"a": 1}


def test_nvfp4_validation(lib):
    q = lib.fp8_nvfp4_quantize
    #      x    rows cols rpt amax given q    bs   gs   xdq  stream
    assert q(A16, 4, 32, 4, A16, 2, A16, A16, A16, None, None) == INVALID     # amax_given not 0/1
    assert q(A16, 4, 24, 4, A16, 0, A16, A16, A16, None, None) == SHAPE       # cols % 16
    assert q(A16, 4, 32, 3, A16, 0, A16, A16, A16, None, None) == SHAPE       # rows % rows_per_tensor
    assert q(A16, 4, 32, 0, A16, 0, A16, A16, A16, None, None) == SHAPE
    assert q(A16, -4, 32, 4, A16, 0, A16, A16, A16, None, None) == SHAPE
    assert q(A16, 1 << 22, 1 << 13, 1, A16, 0, A16, A16, A16, None, None) == SHAPE   # >= 2^32 chunks
    assert q(A16, 1 << 50, 1 << 20, 1, A16, 0, A16, A16, A16, None, None) == SHAPE   # element count overflows
    assert q(None, 0, 32, 1, None, 0, None, None, None, None, None) == OK     # empty
    assert q(None, 4, 32, 4, A16, 0, A16, A16, A16, None, None) == INVALID
    assert q(A16, 4, 32, 4, None, 0, A16, A16, A16, None, None) == INVALID    # no tensor_amax
    assert q(A16, 4, 32, 4, A16, 0, A16, None, A16, None, None) == INVALID    # no block scales
    assert q(A16 + 8, 4, 32, 4, A16, 0, A16, A16, A16, None, None) == ALIGN
    assert q(A16, 4, 32, 4, A16, 0, A16 + 4, A16, A16, None, None) == ALIGN   # codes: 8 B
    assert q(A16, 4, 32, 4, A16 + 1, 0, A16, A16, A16, None, None) == ALIGN
    assert q(A16, 4, 32, 4, A16, 0, A16, A16, A16, A16 + 4, None) == ALIGN    # xdq: 16 B
    d = lib.fp8_nvfp4_dequantize
    assert d(A16, A16, A16, 4, 24, 4, A16, None) == SHAPE
    assert d(None, None, None, 0, 32, 1, None, None) == OK
    assert d(A16, None, A16, 4, 32, 4, A16, None) == INVALID
    assert d(A16, A16, A16, 4, 32, 4, A16 + 8, None) == ALIGN
    assert d(A16 + 4, A16, A16, 4, 32, 4, A16, None) == ALIGN      # codes: 8-byte aligned, as the quantize requires
