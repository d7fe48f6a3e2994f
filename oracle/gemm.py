"""Block-scaled FP8 GEMM and grouped (MoE expert) GEMM references (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages: FP8 values are multiplied on the matrix units while intermediate
results are promoted to a higher precision before the final accumulation
([DSV3-Blog5] "Hardware Optimization: Leveraging NVIDIA Tensor Cores for
FP8"); matmul accumulation is one of the places that must not stay in low
precision ([FP8-DSV3-ru] "Какие операции нельзя бездумно переводить в FP8");
the serving stack runs FP8 matrix multiplication on block-quantized
weights and activations ([FP8-DSV3-ru] "Инференс с FP8"); routed MoE
experts are the tensors served in MXFP8 ([prequant] "Formats" and the
routed-expert rule below it).

What the GEMM computes (a reading of the pages): Y = A_hat . B_hat^T
with both operands stored K-contiguous ([M, K] and [N, K]), where
A_hat = RN32(decode(qa) * sa) and B_hat = RN32(decode(qb) * sb) are the
dequantized fp32 operands (exact for E8M0 scales).  The reference result is
the fp32-accumulated product of those dequantized operands, written out as
its plain definition: for every output, the fp32 sum of the rounded
products RN32(A_hat[m, k] * B_hat[n, k]) taken in the order k = 0..K-1,
starting from 0 (no blocking, no fused multiply-add).  A float64 product
of the same operands (a library matmul: its rounding is far below the
tolerance) is the near-exact value it is compared with.  The grouped GEMM
is the dense GEMM applied per group: group g owns rows [off[g], off[g+1])
of A and the expert matrix B[g].
"""

import numpy as np

from .quant import dequantize_f32


def dequant_operand(q, scale, kind):
    """The dequantized fp32 operand RN32(decode(q) * scale)."""
    return dequantize_f32(np.asarray(q, dtype=np.uint8), scale, kind)


def sum_k_ordered(a_hat, b_hat):
    """Y[m, n] = (((0 + p_0) + p_1) + ...) + p_{K-1} in float32, with
    p_k = RN32(a_hat[m, k] * b_hat[n, k]).  Each step is one numpy float32
    operation (rounded on its own); rows are taken 64 at a time only to keep
    the running sums small, which does not change any sum."""
    a = np.asarray(a_hat, dtype=np.float32)
    b = np.asarray(b_hat, dtype=np.float32)
    m, k = a.shape
    n = b.shape[0]
    bt = np.ascontiguousarray(b.T)                 # [K, N]: row k holds b_hat[:, k]
    out = np.empty((m, n), dtype=np.float32)
    for r0 in range(0, m, 64):
        at = np.ascontiguousarray(a[r0:r0 + 64].T)  # [K, rows]
        acc = np.zeros((at.shape[1], n), dtype=np.float32)
        for t in range(k):
            acc += np.multiply.outer(at[t], bt[t])
        out[r0:r0 + 64] = acc
    return out


def gemm_ref32(a_q, a_scale, a_kind, b_q, b_scale, b_kind):
    """fp32-accumulated Y[M, N] = A_hat . B_hat^T, k-ordered (sum_k_ordered)."""
    a = dequant_operand(a_q, a_scale, a_kind)
    b = dequant_operand(b_q, b_scale, b_kind)
    return sum_k_ordered(a, b)


def gemm_ref64(a_q, a_scale, a_kind, b_q, b_scale, b_kind):
    """The same product accumulated in float64 (library matmul; rounding
    about 2^-53 per term, so it stands for the exact product here)."""
    a = dequant_operand(a_q, a_scale, a_kind).astype(np.float64)
    b = dequant_operand(b_q, b_scale, b_kind).astype(np.float64)
    return np.matmul(a, b.T)


def gemm_entries(a_hat, b_hat, rows, cols):
    """Selected outputs Y[rows[i], cols[i]], each an fp64 dot product of
    dequantized rows (for checks at sizes where the whole product is not
    formed)."""
    a = np.asarray(a_hat, dtype=np.float64)[rows]
    b = np.asarray(b_hat, dtype=np.float64)[cols]
    return np.einsum("ik,ik->i", a, b)


def grouped_gemm_ref(a_q, a_scale, a_kind, b_q, b_scale, b_kind, offsets,
                     groups=None, acc64=False):
    """Per-group dense reference.

    a_q [total_m, K] with its scales; b_q [G, N, K] with per-expert scales
    b_scale[g]; offsets int [G+1].  Returns {g: Y_g [M_g, N]} for the
    requested groups (all by default).  Empty groups map to [0, N] arrays.
    """
    if a_kind not in ("1x32", "1x128"):
        raise ValueError("grouped GEMM: A must use per-row (1x32 / 1x128) blocks")
    off = np.asarray(offsets, dtype=np.int64)
    g_count = len(off) - 1
    if groups is None:
        groups = range(g_count)
    out = {}
    for g in groups:
        lo, hi = int(off[g]), int(off[g + 1])
        b = dequant_operand(b_q[g], b_scale[g], b_kind)
        a = dequant_operand(a_q[lo:hi], a_scale[lo:hi], a_kind)
        if acc64:
            out[g] = np.matmul(a.astype(np.float64), b.astype(np.float64).T)
        else:
            out[g] = sum_k_ordered(a, b)
    return out


def normwise_rel_err(y, ref):
    """max |y - ref| / max |ref| (the GEMM tolerance metric); 0 for empty."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(y - ref))
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)
