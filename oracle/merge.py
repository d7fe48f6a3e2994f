"""QAT forward: LoRA merge W + B.A in bf16, then 128x128 fake-quant (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages: the QAT forward pass fake-quantizes the *merged* weights (and the
activations) so that it follows FP8 numerics, while the LoRA factors stay in
bf16; at inference LoRA is merged into the base weights and the merged
weight is converted to block-wise FP8 ([Fireworks-QAT] "Synopsis",
"Interpretation").  The block-wise FP8 format of DeepSeek-V3 weights is the
128x128 block with an fp32 scale inverse ([FP8-DSV3-ru] "Почему обычное
округление не подходит").

Reading of "merge W + B.A in bf16" (the pages print no formula): the bf16
product B.A is a rank-r sum accumulated in fp32 in the
order r = 0, 1, ..., R-1, each step one correctly rounded fp32
multiply-add of an exact bf16 x bf16 product,
    acc_0 = 0,   acc_{r+1} = RN32(acc_r + B[n, r] * A[r, k]),
rounded once to bf16, delta = RN_bf16(acc_R); the bf16 add is an fp32 add
rounded to bf16, W' = RN_bf16(RN32(W + delta)).  No LoRA alpha/r factor
appears on the pages; a caller folds it into B.

Arithmetic of the fp32 step: the exact product of two bf16 values has at
most 16 significant bits, so it is exact in float64; float64 has more than
2*24+1 bits, so rounding acc + product to float64 first and then to float32
equals rounding the exact sum to float32 once (double rounding through a
format of at least 2p+1 bits is innocuous for a sum of two p-bit numbers).
A test checks this formulation against exact rational arithmetic.
"""

import numpy as np

from .codec import bf16_to_f32, f32_to_bf16
from .quant import quantize


def lora_delta(b_bits, a_bits):
    """delta = RN_bf16(sequential fp32 sum over r of B[n, r] * A[r, k]), bf16 bits [N, K]."""
    bf = bf16_to_f32(b_bits).astype(np.float64)    # [N, R]
    af = bf16_to_f32(a_bits).astype(np.float64)    # [R, K]
    n, r_dim = bf.shape
    r2, k = af.shape
    if r_dim != r2:
        raise ValueError("LoRA rank mismatch")
    acc = np.zeros((n, k), dtype=np.float32)
    for r in range(r_dim):
        exact = acc.astype(np.float64) + bf[:, r:r + 1] * af[r:r + 1, :]
        acc = exact.astype(np.float32)             # RN32 of the exact sum
    return f32_to_bf16(acc)


def merge_weights(w_bits, b_bits, a_bits):
    """W' = RN_bf16(RN32(W + delta)) as bf16 bits [N, K]."""
    delta = bf16_to_f32(lora_delta(b_bits, a_bits))
    w = bf16_to_f32(w_bits)
    return f32_to_bf16((w + delta).astype(np.float32))


def fake_quant_merge(w_bits, b_bits, a_bits):
    """Merge, then 128x128 fp32-scale quantize: (q, scale [N/128, K/128], W'dq)."""
    return quantize(merge_weights(w_bits, b_bits, a_bits), "128x128")
