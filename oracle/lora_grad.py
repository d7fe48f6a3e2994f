"""QAT backward for the LoRA factors (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages: in QAT the merged weights (and activations) are fake-quantized
in the forward pass, while the LoRA factors and their gradients stay in
bfloat16 ([Fireworks-QAT] Synopsis, Interpretation).  The forward GEMM is
Y = X_hat . W_hat^T with W_hat = fakequant(W + B.A) and X_hat the
fake-quantized activations.

Reading (the pages name no gradient rule): the
fake-quant is passed straight through in the backward pass (its Jacobian
is taken as the identity), so with dY = dL/dY

    dW = dY^T . X_hat                       [N x K]
    dB = dW . A^T                           [N x r]
    dA = B^T . dW                           [r x K]

evaluated here in float64 from the exact bf16 inputs, exactly as written
(dW formed).  A kernel's bf16 results are compared with these float64
values within a tolerance (fp32 accumulation, one bf16 rounding).
"""

import numpy as np

from .codec import bf16_to_f32


def lora_grads(dy_bits, x_bits, b_bits, a_bits):
    """(dB, dA) in float64 from bf16 bits dY [M, N], X_hat [M, K],
    B [N, r], A [r, K]."""
    dy = bf16_to_f32(dy_bits).astype(np.float64)
    x = bf16_to_f32(x_bits).astype(np.float64)
    b = bf16_to_f32(b_bits).astype(np.float64)
    a = bf16_to_f32(a_bits).astype(np.float64)
    dw = dy.T @ x
    return dw @ a.T, b.T @ dw


def lora_grads_columns(dy_bits, x_bits, b_bits, a_bits, n_rows, k_cols):
    """Selected rows of dB (rows ``n_rows``) and columns of dA (columns
    ``k_cols``) without forming the whole dW: dW[n_rows, :] and
    dW[:, k_cols] are the needed slices of the same product."""
    dy = bf16_to_f32(dy_bits).astype(np.float64)
    x = bf16_to_f32(x_bits).astype(np.float64)
    b = bf16_to_f32(b_bits).astype(np.float64)
    a = bf16_to_f32(a_bits).astype(np.float64)
    dw_rows = dy[:, n_rows].T @ x              # [|n_rows| x K]
    dw_cols = dy.T @ x[:, k_cols]              # [N x |k_cols|]
    return dw_rows @ a.T, b.T @ dw_cols

