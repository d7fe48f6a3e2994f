"""Python binding of the fp8blk C ABI (include/fp8blk.h).

Argument marshalling only: every function here forwards torch tensors'
device pointers, sizes and the current HIP stream to the native entry point
of the same name in ``libfp8blk.so``; all arithmetic runs in the library's
HIP kernels.  PyTorch supplies device memory and streams.  There is no CPU
fallback: if the library is missing, every call raises.

Block kinds, E8M0 rules and output types mirror the C enums.
"""

import ctypes
import os
import re

import torch

__all__ = [
    "FP8_BLOCK_1x32_E8M0", "FP8_BLOCK_1x128_F32", "FP8_BLOCK_128x128_F32",
    "FP8_E8M0_CEIL", "FP8_E8M0_FLOOR", "FP8_OUT_BF16", "FP8_OUT_F32",
    "Fp8Error", "library", "library_path",
    "fp8_block_quantize", "fp8_block_quantize_batch", "fp8_block_dequantize", "fp8_fake_quant_merge", "fp8_block_scaled_gemm",
    "fp8_grouped_gemm", "fp8_grouped_gemm_gather", "fp8_lora_backward", "fp8_lora_backward_workspace",
    "fp8_lora_backward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "fp8_nvfp4_quantize", "fp8_nvfp4_dequantize",
    "fp8_status_string", "fp8_abi_version",
    "quantize", "dequantize", "fake_quant_merge", "block_scaled_gemm", "grouped_gemm", "lora_backward", "nvfp4_quantize", "nvfp4_dequantize",
    "scale_shape",
    "is_routed_expert_weight", "quantize_state_dict",
]

FP8_OK = 0
FP8_BLOCK_1x32_E8M0, FP8_BLOCK_1x128_F32, FP8_BLOCK_128x128_F32 = 0, 1, 2
FP8_E8M0_CEIL, FP8_E8M0_FLOOR = 0, 1
FP8_OUT_BF16, FP8_OUT_F32 = 0, 1
ABI_VERSION = 6
NOALLOC_SCRATCH_BYTES = 40 << 20    # fixed scratch of fp8_lora_backward_noalloc (per device)

_KIND_NAMES = {"1x32": FP8_BLOCK_1x32_E8M0, "1x128": FP8_BLOCK_1x128_F32, "128x128": FP8_BLOCK_128x128_F32}
_RULE_NAMES = {"ceil": FP8_E8M0_CEIL, "floor": FP8_E8M0_FLOOR}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8blk.so")

_lib = None


class QuantizeJob(ctypes.Structure):
    """Mirror of fp8_quantize_job (include/fp8blk.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("kind", ctypes.c_int), ("rule", ctypes.c_int), ("q", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("xdq", ctypes.c_void_p)]


class Fp8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: fp8blk status {status} ({_status_text(status)})")


def library():
    """The loaded ctypes library (loads it on first use; raises if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is not built; run `python -m block_scaled_fp8_amax_amd._build`")
        lib = ctypes.CDLL(library_path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.fp8_block_quantize.argtypes = [vp, i64, i64, ci, ci, vp, vp, vp, vp]
        lib.fp8_block_quantize.restype = ci
        lib.fp8_block_quantize_batch.argtypes = [ctypes.POINTER(QuantizeJob), ci, vp]
        lib.fp8_block_quantize_batch.restype = ci
        lib.fp8_block_dequantize.argtypes = [vp, vp, i64, i64, ci, vp, vp]
        lib.fp8_block_dequantize.restype = ci
        lib.fp8_fake_quant_merge.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp]
        lib.fp8_fake_quant_merge.restype = ci
        lib.fp8_block_scaled_gemm.argtypes = [vp, vp, ci, vp, vp, ci, i64, i64, i64, vp, ci, vp]
        lib.fp8_block_scaled_gemm.restype = ci
        lib.fp8_grouped_gemm.argtypes = [vp, vp, ci, vp, vp, ci, vp, i64, i64, i64, i64, vp, ci, vp]
        lib.fp8_grouped_gemm.restype = ci
        lib.fp8_grouped_gemm_gather.argtypes = [vp, vp, ci, i64, vp, vp, vp, ci, vp, i64, i64, i64, i64, vp, ci, vp]
        lib.fp8_grouped_gemm_gather.restype = ci
        lib.fp8_lora_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, ctypes.c_size_t, vp, vp, ci, vp]
        lib.fp8_lora_backward.restype = ci
        lib.fp8_lora_backward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, ci, vp]
        lib.fp8_lora_backward_noalloc.restype = ci
        lib.fp8_lora_backward_workspace.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.fp8_lora_backward_workspace.restype = ci
        lib.fp8_nvfp4_quantize.argtypes = [vp, i64, i64, i64, vp, ci, vp, vp, vp, vp, vp]
        lib.fp8_nvfp4_quantize.restype = ci
        lib.fp8_nvfp4_dequantize.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp]
        lib.fp8_nvfp4_dequantize.restype = ci
        lib.fp8_status_string.argtypes = [ci]
        lib.fp8_status_string.restype = ctypes.c_char_p
        lib.fp8_abi_version.argtypes = []
        lib.fp8_abi_version.restype = ci
        if lib.fp8_abi_version() != ABI_VERSION:
            raise ImportError("libfp8blk.so ABI version mismatch")
        _lib = lib
    return _lib


def _status_text(status):
    try:
        return library().fp8_status_string(int(status)).decode()
    except Exception:  # noqa: BLE001 - only used for error text
        return "?"


def fp8_status_string(status):
    return library().fp8_status_string(int(status)).decode()


def fp8_abi_version():
    return library().fp8_abi_version()


def _kind(k):
    return _KIND_NAMES[k] if isinstance(k, str) else int(k)


def _rule(r):
    return _RULE_NAMES[r] if isinstance(r, str) else int(r)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    for t in tensors:
        if t is not None and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status, where):
    if status != FP8_OK:
        raise Fp8Error(status, where)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("fp8blk expects contiguous tensors")


# The library takes raw device pointers and sizes and cannot see the
# tensors behind them, so the binding checks what it can before a kernel
# runs: every tensor on one GPU, the documented dtypes, and each buffer at
# least as large as the sizes passed with it (floor-divided block counts:
# shapes the library rejects never reach a kernel).
_CODES = (torch.uint8, torch.float8_e4m3fn)
_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_U8 = (torch.uint8,)
_OUT = (torch.bfloat16, torch.float32)


def _same_gpu(where, *ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{where}: every tensor must be on a GPU, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{where}: tensors on different devices ({dev} and {t.device})")


def _expect(where, name, t, dtypes, numel):
    if t is None:
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{where}: {name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.numel() < numel:
        raise ValueError(f"{where}: {name} holds {t.numel()} elements, needs at least {numel}")


def _expect_dims(where, name, t, shape):
    """A tensor with as many dimensions as ``shape`` must have exactly that
    shape: the library reads it with the strides the sizes imply, so a
    wider row would be read wrongly.  A buffer given with another number of
    dimensions (for example flat) is checked by size only."""
    if t is None or t.dim() != len(shape):
        return
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(int(d) for d in shape)}")


def _scale_dims(rows, cols, kind):
    kind = _kind(kind)
    if kind == FP8_BLOCK_1x32_E8M0:
        return (rows, cols // 32)
    if kind == FP8_BLOCK_1x128_F32:
        return (rows, cols // 128)
    return (rows // 128, cols // 128)


def _scale_numel(rows, cols, kind):
    kind = _kind(kind)
    if kind == FP8_BLOCK_1x32_E8M0:
        return rows * (cols // 32), _U8
    if kind == FP8_BLOCK_1x128_F32:
        return rows * (cols // 128), _F32
    return (rows // 128) * (cols // 128), _F32


def _check_quantize_job(where, x, kind, q, scale, xdq):
    if x.dim() != 2:
        raise ValueError(f"{where}: x must be 2-D, got shape {tuple(x.shape)}")
    rows, cols = x.shape
    _expect(where, "x", x, _BF16, 0)
    _expect(where, "q", q, _CODES, rows * cols)
    sn, sdt = _scale_numel(rows, cols, kind)
    _expect(where, "scale", scale, sdt, sn)
    _expect(where, "xdq", xdq, _BF16, rows * cols)
    _expect_dims(where, "q", q, (rows, cols))
    _expect_dims(where, "scale", scale, _scale_dims(rows, cols, kind))
    _expect_dims(where, "xdq", xdq, (rows, cols))
    _same_gpu(where, x, q, scale, xdq)


# ------------------------------------------------------------- entry points

def fp8_block_quantize(x, kind, rule, q, scale, xdq=None, stream=None):
    """x: bf16 [rows, cols]; q: uint8/float8_e4m3fn [rows, cols]; scale: uint8
    (1x32) or float32 of the kind's shape; xdq: optional bf16 [rows, cols]."""
    _contig(x, q, scale, xdq)
    _check_quantize_job("fp8_block_quantize", x, kind, q, scale, xdq)
    rows, cols = x.shape
    st = library().fp8_block_quantize(_ptr(x), rows, cols, _kind(kind), _rule(rule), _ptr(q), _ptr(scale),
                                      _ptr(xdq), _stream(stream, x))
    _check(st, "fp8_block_quantize")


def fp8_block_quantize_batch(jobs, stream=None):
    """jobs: list of (x, kind, rule, q, scale[, xdq]) tuples, each exactly the
    arguments of fp8_block_quantize; all of them run in one launch."""
    if not jobs:
        return
    arr = (QuantizeJob * len(jobs))()
    for i, job in enumerate(jobs):
        x, kind, rule, q, scale = job[:5]
        xdq = job[5] if len(job) > 5 else None
        _contig(x, q, scale, xdq)
        _check_quantize_job(f"fp8_block_quantize_batch job {i}", x, kind, q, scale, xdq)
        if i and x.device != jobs[0][0].device:
            raise ValueError("fp8_block_quantize_batch: jobs on different devices")
        rows, cols = x.shape
        arr[i] = QuantizeJob(_ptr(x), rows, cols, _kind(kind), _rule(rule), _ptr(q), _ptr(scale), _ptr(xdq))
    st = library().fp8_block_quantize_batch(arr, len(jobs), _stream(stream, jobs[0][0]))
    _check(st, "fp8_block_quantize_batch")


def fp8_block_dequantize(q, scale, kind, x, stream=None):
    """q: uint8/float8_e4m3fn [rows, cols]; scale as written by
    fp8_block_quantize for ``kind``; x: bf16 [rows, cols] output."""
    _contig(q, scale, x)
    where = "fp8_block_dequantize"
    rows, cols = q.shape
    _expect(where, "q", q, _CODES, 0)
    sn, sdt = _scale_numel(rows, cols, kind)
    _expect(where, "scale", scale, sdt, sn)
    _expect(where, "x", x, _BF16, rows * cols)
    _expect_dims(where, "scale", scale, _scale_dims(rows, cols, kind))
    _expect_dims(where, "x", x, (rows, cols))
    _same_gpu(where, q, scale, x)
    st = library().fp8_block_dequantize(_ptr(q), _ptr(scale), rows, cols, _kind(kind), _ptr(x), _stream(stream, q))
    _check(st, "fp8_block_dequantize")


def fp8_fake_quant_merge(w, lora_b, lora_a, q, scale, wdq=None, stream=None):
    """w: bf16 [n, k]; lora_b bf16 [n, r]; lora_a bf16 [r, k]; q [n, k];
    scale float32 [n/128, k/128]; wdq optional bf16 [n, k]."""
    _contig(w, lora_b, lora_a, q, scale, wdq)
    where = "fp8_fake_quant_merge"
    n, k = w.shape
    r = lora_a.shape[0]
    _expect(where, "w", w, _BF16, 0)
    _expect(where, "lora_b", lora_b, _BF16, n * r)
    _expect(where, "lora_a", lora_a, _BF16, r * k)
    _expect(where, "q", q, _CODES, n * k)
    _expect(where, "scale", scale, _F32, (n // 128) * (k // 128))
    _expect(where, "wdq", wdq, _BF16, n * k)
    if lora_b.dim() != 2 or tuple(lora_b.shape) != (n, r) or lora_a.dim() != 2 or lora_a.shape[1] != k:
        raise ValueError(f"{where}: lora_b {tuple(lora_b.shape)} and lora_a {tuple(lora_a.shape)} do not match "
                         f"w {tuple(w.shape)} (expected ({n}, r) and (r, {k}))")
    _expect_dims(where, "q", q, (n, k))
    _expect_dims(where, "scale", scale, (n // 128, k // 128))
    _expect_dims(where, "wdq", wdq, (n, k))
    _same_gpu(where, w, lora_b, lora_a, q, scale, wdq)
    st = library().fp8_fake_quant_merge(_ptr(w), _ptr(lora_b), _ptr(lora_a), n, k, r, _ptr(q), _ptr(scale),
                                        _ptr(wdq), _stream(stream, w))
    _check(st, "fp8_fake_quant_merge")


def fp8_block_scaled_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, y, stream=None):
    """Y[m, n] = deq(A) . deq(B)^T; y is bf16 or float32 [m, n]."""
    _contig(a_q, a_scale, b_q, b_scale, y)
    where = "fp8_block_scaled_gemm"
    m, k = a_q.shape
    n = b_q.shape[0]
    _expect(where, "a_q", a_q, _CODES, 0)
    _expect(where, "b_q", b_q, _CODES, n * k)
    sn, sdt = _scale_numel(m, k, a_kind)
    _expect(where, "a_scale", a_scale, sdt, sn)
    sn, sdt = _scale_numel(n, k, b_kind)
    _expect(where, "b_scale", b_scale, sdt, sn)
    _expect(where, "y", y, _OUT, m * n)
    if b_q.dim() != 2 or b_q.shape[1] != k:
        raise ValueError(f"{where}: b_q has shape {tuple(b_q.shape)}, expected (n, {k}) to match a_q {tuple(a_q.shape)}")
    _expect_dims(where, "a_scale", a_scale, _scale_dims(m, k, a_kind))
    _expect_dims(where, "b_scale", b_scale, _scale_dims(n, k, b_kind))
    _expect_dims(where, "y", y, (m, n))
    y_type = FP8_OUT_F32 if y.dtype == torch.float32 else FP8_OUT_BF16
    _same_gpu(where, a_q, a_scale, b_q, b_scale, y)
    st = library().fp8_block_scaled_gemm(_ptr(a_q), _ptr(a_scale), _kind(a_kind), _ptr(b_q), _ptr(b_scale),
                                         _kind(b_kind), m, n, k, _ptr(y), y_type, _stream(stream, a_q))
    _check(st, "fp8_block_scaled_gemm")


def _check_grouped(where, a_q, a_scale, a_kind, a_rows, b_q, b_scale, b_kind, groups, n, k, offsets, y, total_m):
    _expect(where, "a_q", a_q, _CODES, 0)
    sn, sdt = _scale_numel(a_rows, k, a_kind)
    _expect(where, "a_scale", a_scale, sdt, sn)
    _expect(where, "b_q", b_q, _CODES, groups * n * k)
    sn, sdt = _scale_numel(n, k, b_kind)
    _expect(where, "b_scale", b_scale, sdt, groups * sn)
    _expect(where, "group_offsets", offsets, _I32, groups + 1)
    _expect(where, "y", y, _OUT, total_m * n)
    if b_q.dim() != 3 or b_q.shape[2] != k:
        raise ValueError(f"{where}: b_q has shape {tuple(b_q.shape)}, expected (groups, n, {k}) to match a_q "
                         f"{tuple(a_q.shape)}")
    _expect_dims(where, "a_scale", a_scale, _scale_dims(a_rows, k, a_kind))
    _expect_dims(where, "b_scale", b_scale, (groups,) + _scale_dims(n, k, b_kind))
    _expect_dims(where, "y", y, (total_m, n))


def fp8_grouped_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, group_offsets, y, stream=None):
    """a_q [total_m, k]; b_q [groups, n, k]; group_offsets int32 [groups+1]
    on the device; y bf16/float32 [total_m, n]."""
    _contig(a_q, a_scale, b_q, b_scale, group_offsets, y)
    where = "fp8_grouped_gemm"
    total_m, k = a_q.shape
    groups, n = b_q.shape[0], b_q.shape[1]
    if group_offsets.dtype != torch.int32:
        raise ValueError("group_offsets must be int32")
    _check_grouped(where, a_q, a_scale, a_kind, total_m, b_q, b_scale, b_kind, groups, n, k, group_offsets, y, total_m)
    y_type = FP8_OUT_F32 if y.dtype == torch.float32 else FP8_OUT_BF16
    _same_gpu(where, a_q, a_scale, b_q, b_scale, group_offsets, y)
    st = library().fp8_grouped_gemm(_ptr(a_q), _ptr(a_scale), _kind(a_kind), _ptr(b_q), _ptr(b_scale),
                                    _kind(b_kind), _ptr(group_offsets), groups, total_m, n, k, _ptr(y), y_type,
                                    _stream(stream, a_q))
    _check(st, "fp8_grouped_gemm")


def fp8_grouped_gemm_gather(a_q, a_scale, a_kind, row_index, b_q, b_scale, b_kind, group_offsets, y, stream=None):
    """a_q [a_rows, k]; row_index int32 [total_m] on the device (A row of each
    grouped row); b_q [groups, n, k]; group_offsets int32 [groups+1];
    y bf16/float32 [total_m, n]."""
    _contig(a_q, a_scale, row_index, b_q, b_scale, group_offsets, y)
    where = "fp8_grouped_gemm_gather"
    a_rows, k = a_q.shape
    groups, n = b_q.shape[0], b_q.shape[1]
    if group_offsets.dtype != torch.int32 or row_index.dtype != torch.int32:
        raise ValueError("group_offsets and row_index must be int32")
    total_m = row_index.numel()
    _check_grouped(where, a_q, a_scale, a_kind, a_rows, b_q, b_scale, b_kind, groups, n, k, group_offsets, y, total_m)
    y_type = FP8_OUT_F32 if y.dtype == torch.float32 else FP8_OUT_BF16
    _same_gpu(where, a_q, a_scale, row_index, b_q, b_scale, group_offsets, y)
    st = library().fp8_grouped_gemm_gather(_ptr(a_q), _ptr(a_scale), _kind(a_kind), a_rows, _ptr(row_index),
                                           _ptr(b_q), _ptr(b_scale), _kind(b_kind), _ptr(group_offsets), groups,
                                           total_m, n, k, _ptr(y), y_type, _stream(stream, a_q))
    _check(st, "fp8_grouped_gemm_gather")


def fp8_lora_backward_workspace(m, n, k, r):
    """Workspace bytes fp8_lora_backward needs for these sizes."""
    out = ctypes.c_size_t(0)
    _check(library().fp8_lora_backward_workspace(m, n, k, r, ctypes.byref(out)), "fp8_lora_backward_workspace")
    return out.value


def fp8_lora_backward(dy, x, lora_b, lora_a, workspace, d_lora_b, d_lora_a, stream=None):
    """dy bf16 [m, n]; x bf16 [m, k] (the fake-quantized activations);
    lora_b bf16 [n, r]; lora_a bf16 [r, k]; workspace uint8 device tensor of
    at least fp8_lora_backward_workspace(m, n, k, r) bytes; d_lora_b [n, r]
    and d_lora_a [r, k] outputs, both bf16 or both float32."""
    _contig(dy, x, lora_b, lora_a, workspace, d_lora_b, d_lora_a)
    m, n = dy.shape
    k = x.shape[1]
    r = lora_a.shape[0]
    if x.shape[0] != m or lora_b.shape != (n, r) or lora_a.shape != (r, k):
        raise ValueError("fp8_lora_backward: inconsistent shapes")
    if d_lora_b.dtype != d_lora_a.dtype:
        raise ValueError("fp8_lora_backward: both gradients must have one dtype")
    where = "fp8_lora_backward"
    for name, t in (("dy", dy), ("x", x), ("lora_b", lora_b), ("lora_a", lora_a)):
        _expect(where, name, t, _BF16, 0)
    _expect(where, "d_lora_b", d_lora_b, _OUT, n * r)
    _expect(where, "d_lora_a", d_lora_a, _OUT, r * k)
    out_type = FP8_OUT_F32 if d_lora_b.dtype == torch.float32 else FP8_OUT_BF16
    _same_gpu(where, dy, x, lora_b, lora_a, workspace, d_lora_b, d_lora_a)
    st = library().fp8_lora_backward(_ptr(dy), _ptr(x), _ptr(lora_b), _ptr(lora_a), m, n, k, r, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _ptr(d_lora_b), _ptr(d_lora_a),
                                     out_type, _stream(stream, dy))
    _check(st, "fp8_lora_backward")


def fp8_lora_backward_noalloc(dy, x, lora_b, lora_a, d_lora_b, d_lora_a, stream=None):
    """fp8_lora_backward without a workspace: the library's fixed per-device
    scratch (NOALLOC_SCRATCH_BYTES) stands in for it and nothing is
    allocated.  Calls that may overlap on one device must be serialized by
    the caller; problems whose workspace exceeds the scratch raise
    (status FP8_ERR_TOO_LARGE)."""
    _contig(dy, x, lora_b, lora_a, d_lora_b, d_lora_a)
    m, n = dy.shape
    k = x.shape[1]
    r = lora_a.shape[0]
    if x.shape[0] != m or lora_b.shape != (n, r) or lora_a.shape != (r, k):
        raise ValueError("fp8_lora_backward_noalloc: inconsistent shapes")
    if d_lora_b.dtype != d_lora_a.dtype:
        raise ValueError("fp8_lora_backward_noalloc: both gradients must have one dtype")
    where = "fp8_lora_backward_noalloc"
    for name, t in (("dy", dy), ("x", x), ("lora_b", lora_b), ("lora_a", lora_a)):
        _expect(where, name, t, _BF16, 0)
    _expect(where, "d_lora_b", d_lora_b, _OUT, n * r)
    _expect(where, "d_lora_a", d_lora_a, _OUT, r * k)
    out_type = FP8_OUT_F32 if d_lora_b.dtype == torch.float32 else FP8_OUT_BF16
    _same_gpu(where, dy, x, lora_b, lora_a, d_lora_b, d_lora_a)
    st = library().fp8_lora_backward_noalloc(_ptr(dy), _ptr(x), _ptr(lora_b), _ptr(lora_a), m, n, k, r,
                                             _ptr(d_lora_b), _ptr(d_lora_a), out_type, _stream(stream, dy))
    _check(st, where)


def fp8_nvfp4_quantize(x, rows_per_tensor, q, block_scale, global_scale, tensor_amax, xdq=None, amax_given=False,
                       stream=None):
    """x bf16 [rows, cols] (rows_per_tensor rows per stacked tensor); q uint8
    [rows, cols/2]; block_scale uint8 / float8_e4m3fn [rows, cols/16];
    global_scale, tensor_amax float32 [rows/rows_per_tensor] (tensor_amax is
    read instead of written when amax_given); xdq optional bf16 [rows, cols]."""
    _contig(x, q, block_scale, global_scale, tensor_amax, xdq)
    where = "fp8_nvfp4_quantize"
    rows, cols = x.shape
    tensors = rows // rows_per_tensor if rows_per_tensor > 0 else 0
    _expect(where, "x", x, _BF16, 0)
    _expect(where, "q", q, _U8, rows * (cols // 2))
    _expect(where, "block_scale", block_scale, _CODES, rows * (cols // 16))
    _expect(where, "global_scale", global_scale, _F32, tensors)
    _expect(where, "tensor_amax", tensor_amax, _F32, tensors)
    _expect(where, "xdq", xdq, _BF16, rows * cols)
    _expect_dims(where, "q", q, (rows, cols // 2))
    _expect_dims(where, "block_scale", block_scale, (rows, cols // 16))
    _expect_dims(where, "xdq", xdq, (rows, cols))
    _same_gpu(where, x, q, block_scale, global_scale, tensor_amax, xdq)
    st = library().fp8_nvfp4_quantize(_ptr(x), rows, cols, rows_per_tensor, _ptr(tensor_amax), 1 if amax_given else 0,
                                      _ptr(q), _ptr(block_scale), _ptr(global_scale), _ptr(xdq), _stream(stream, x))
    _check(st, "fp8_nvfp4_quantize")


def fp8_nvfp4_dequantize(q, block_scale, global_scale, rows_per_tensor, x, stream=None):
    """q uint8 [rows, cols/2], block_scale [rows, cols/16], global_scale
    float32 [tensors]; x bf16 [rows, cols] output."""
    _contig(q, block_scale, global_scale, x)
    where = "fp8_nvfp4_dequantize"
    rows, cols = x.shape
    tensors = rows // rows_per_tensor if rows_per_tensor > 0 else 0
    _expect(where, "q", q, _U8, rows * (cols // 2))
    _expect(where, "block_scale", block_scale, _CODES, rows * (cols // 16))
    _expect(where, "global_scale", global_scale, _F32, tensors)
    _expect(where, "x", x, _BF16, rows * cols)
    _expect_dims(where, "q", q, (rows, cols // 2))
    _expect_dims(where, "block_scale", block_scale, (rows, cols // 16))
    _same_gpu(where, q, block_scale, global_scale, x)
    st = library().fp8_nvfp4_dequantize(_ptr(q), _ptr(block_scale), _ptr(global_scale), rows, cols, rows_per_tensor,
                                        _ptr(x), _stream(stream, q))
    _check(st, "fp8_nvfp4_dequantize")


# --------------------------------------------- allocating conveniences (torch)

def scale_shape(rows, cols, kind):
    kind = _kind(kind)
    if kind == FP8_BLOCK_1x32_E8M0:
        return (rows, cols // 32), torch.uint8
    if kind == FP8_BLOCK_1x128_F32:
        return (rows, cols // 128), torch.float32
    return (rows // 128, cols // 128), torch.float32


def quantize(x, block="1x128", rule="ceil", dequant=False, stream=None):
    """Allocate outputs and run fp8_block_quantize: returns (q, scale[, xdq])
    with q viewed as torch.float8_e4m3fn."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    shp, dt = scale_shape(rows, cols, block)
    scale = torch.empty(shp, dtype=dt, device=x.device)
    xdq = torch.empty_like(x) if dequant else None
    fp8_block_quantize(x, block, rule, q, scale, xdq, stream)
    q = q.view(torch.float8_e4m3fn)
    return (q, scale, xdq) if dequant else (q, scale)


def fake_quant_merge(w, lora_b, lora_a, dequant=False, stream=None):
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n // 128, k // 128), dtype=torch.float32, device=w.device)
    wdq = torch.empty_like(w) if dequant else None
    fp8_fake_quant_merge(w, lora_b, lora_a, q, scale, wdq, stream)
    q = q.view(torch.float8_e4m3fn)
    return (q, scale, wdq) if dequant else (q, scale)


def block_scaled_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, out_dtype=torch.bfloat16, stream=None):
    y = torch.empty((a_q.shape[0], b_q.shape[0]), dtype=out_dtype, device=a_q.device)
    fp8_block_scaled_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, y, stream)
    return y


def grouped_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, group_offsets, out_dtype=torch.bfloat16, stream=None,
                 row_index=None):
    """Grouped GEMM; with ``row_index`` the A rows are gathered
    (fp8_grouped_gemm_gather) and the output has row_index.numel() rows."""
    rows = a_q.shape[0] if row_index is None else row_index.numel()
    y = torch.empty((rows, b_q.shape[1]), dtype=out_dtype, device=a_q.device)
    if row_index is None:
        fp8_grouped_gemm(a_q, a_scale, a_kind, b_q, b_scale, b_kind, group_offsets, y, stream)
    else:
        fp8_grouped_gemm_gather(a_q, a_scale, a_kind, row_index, b_q, b_scale, b_kind, group_offsets, y, stream)
    return y


def lora_backward(dy, x, lora_b, lora_a, out_dtype=torch.bfloat16, workspace=None, stream=None):
    """Allocate (dB, dA) and, unless given, the workspace, and run
    fp8_lora_backward: returns (d_lora_b [n, r], d_lora_a [r, k])."""
    m, n = dy.shape
    k = x.shape[1]
    r = lora_a.shape[0]
    if workspace is None:
        workspace = torch.empty(fp8_lora_backward_workspace(m, n, k, r), dtype=torch.uint8, device=dy.device)
    db = torch.empty((n, r), dtype=out_dtype, device=dy.device)
    da = torch.empty((r, k), dtype=out_dtype, device=dy.device)
    fp8_lora_backward(dy, x, lora_b, lora_a, workspace, db, da, stream)
    return db, da


def nvfp4_quantize(x, rows_per_tensor=None, dequant=False, amax=None, stream=None):
    """Allocate outputs and run fp8_nvfp4_quantize: returns (q uint8
    [rows, cols/2], block_scale float8_e4m3fn [rows, cols/16], global_scale
    float32 [T], tensor_amax float32 [T][, xdq]).  ``amax`` (float32 [T] on the
    device) replaces the measured tensor amax."""
    rows, cols = x.shape
    rpt = rows if rows_per_tensor is None else rows_per_tensor
    t = rows // max(rpt, 1)
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    bs = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    gs = torch.empty((t,), dtype=torch.float32, device=x.device)
    am = amax.to(torch.float32).contiguous() if amax is not None else torch.empty((t,), dtype=torch.float32,
                                                                                  device=x.device)
    xdq = torch.empty_like(x) if dequant else None
    fp8_nvfp4_quantize(x, max(rpt, 1), q, bs, gs, am, xdq, amax_given=amax is not None, stream=stream)
    bs = bs.view(torch.float8_e4m3fn)
    return (q, bs, gs, am, xdq) if dequant else (q, bs, gs, am)


def nvfp4_dequantize(q, block_scale, global_scale, rows_per_tensor=None, stream=None):
    """Allocate the bf16 output and run fp8_nvfp4_dequantize."""
    rows = q.shape[0]
    x = torch.empty((rows, q.shape[1] * 2), dtype=torch.bfloat16, device=q.device)
    bs = block_scale.view(torch.uint8) if block_scale.dtype != torch.uint8 else block_scale
    fp8_nvfp4_dequantize(q, bs, global_scale, rows if rows_per_tensor is None else rows_per_tensor, x, stream)
    return x


def dequantize(q, scale, block, stream=None):
    """Allocate the bf16 output and run fp8_block_dequantize."""
    x = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    fp8_block_dequantize(q, scale, block, x, stream)
    return x


# ------------------------------------ MXFP8 / NVFP4 prequantization of experts

# Routed MoE expert projections, prefix-tolerant ("fireworks-prequant 0.1.0",
# "Formats": model.layers.*.mlp.experts.*.{gate,up,down}_proj.weight); dense,
# attention, router and shared-expert weights do not match.
_ROUTED_EXPERT = re.compile(r"(^|\.)layers\.\d+\.mlp\.experts\.\d+\.(gate|up|down)_proj\.weight$")


def is_routed_expert_weight(name):
    return _ROUTED_EXPERT.search(name) is not None


def quantize_state_dict(state, fmt="mxfp8", device="cuda", rule="ceil", out_device=None):
    """Prequantize the routed expert weights of a state dict to MXFP8 or NVFP4.

    Every tensor whose name is a routed expert projection weight (bf16,
    [rows, cols]) is quantized on ``device`` ("fireworks-prequant 0.1.0",
    "Quick start", "Formats"):
      * fmt="mxfp8" (cols % 32 == 0): fp8_block_quantize with 1x32 blocks and
        E8M0 scales; ``{..}.weight`` becomes the float8_e4m3fn codes and
        ``{..}.weight_scale_inv`` the uint8 E8M0 scale codes [rows, cols/32];
      * fmt="nvfp4" (cols % 16 == 0): fp8_nvfp4_quantize, one tensor;
        ``{..}.weight`` becomes the packed E2M1 codes (uint8 [rows, cols/2]),
        ``{..}.weight_scale_inv`` the float8_e4m3fn 1x16 block scales
        [rows, cols/16] and ``{..}.weight_global_scale`` the float32 tensor
        scale g (shape [1]).
    Other tensors pass through unchanged (the same objects).  Quantized
    outputs stay on ``device`` unless ``out_device`` is given.
    """
    if fmt not in ("mxfp8", "nvfp4"):
        raise ValueError(f"unsupported prequant format {fmt!r} (only 'mxfp8' and 'nvfp4')")
    out = {}
    for name, t in state.items():
        if not is_routed_expert_weight(name):
            out[name] = t
            continue
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise ValueError(f"{name}: expected a 2-D bf16 tensor, got {t.dtype} {tuple(t.shape)}")
        x = t.to(device).contiguous()
        stem = name[: -len("weight")]
        if fmt == "mxfp8":
            q, s = quantize(x, "1x32", rule)
            extra = {}
        else:
            q, s, g, _ = nvfp4_quantize(x)
            extra = {stem + "weight_global_scale": g}
        if out_device is not None:
            q, s = q.to(out_device), s.to(out_device)
            extra = {k: v.to(out_device) for k, v in extra.items()}
        out[name] = q
        out[stem + "weight_scale_inv"] = s
        out.update(extra)
    return out
