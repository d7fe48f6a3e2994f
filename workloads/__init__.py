"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``; it holds
none of the method's arithmetic (no quantization, no scales, no GEMM): only
random bf16 tensors, outlier placement, MoE routing and row grouping.

Shapes follow DeepSeek-V3 projections (hidden 7168, routed-expert
intermediate 2048, 256 routed experts, top-8 routing); the pages describe
the model (671B parameters, about 37B active per token) and its MXFP8
routed-expert checkpoints but ship no tensors, so every input is drawn here.

Recipe:
  * values: torch.randn(float32) with a ``torch.Generator`` seeded per tensor
    on the target device, times sigma, times the outlier factor, then
    rounded to bf16 (RNE, torch ``.to(bfloat16)``);
  * outliers: exactly round(p * count) distinct positions (elements, or whole
    K-columns for "channels"), chosen by a seeded permutation;
  * the CPU and GPU generators produce different streams: a parity test
    always feeds the *same* tensor to both sides.
"""

import math

import numpy as np
import torch

HIDDEN = 7168
EXPERT_INTER = 2048
N_EXPERTS = 256
TOP_K = 8


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, sigma, seed, device="cpu", outlier_frac=0.0, outlier_mult=1.0,
                outlier_channels=False):
    """bf16 tensor N(0, sigma^2) with optional element or channel outliers."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma
    if outlier_frac > 0:
        if outlier_channels:
            cols = shape[-1]
            cnt = int(round(outlier_frac * cols))
            idx = torch.randperm(cols, generator=g, device=device)[:cnt]
            x[..., idx] *= outlier_mult
        else:
            n = x.numel()
            cnt = int(round(outlier_frac * n))
            idx = torch.randperm(n, generator=g, device=device)[:cnt]
            x.view(-1)[idx] *= outlier_mult
    return x.to(torch.bfloat16)


def bf16_bits(t):
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------- the configs

def mx_small(device="cpu"):
    """MXFP8 parity case: W 256x512 and X 64x512, N(0,1), 0.1% outliers x100."""
    w = normal_bf16((256, 512), 1.0, 0, device, 0.001, 100.0)
    x = normal_bf16((64, 512), 1.0, 1, device, 0.001, 100.0)
    return {"w": w, "x": x}


def dense_projection(device="cpu", m=4096, n=2048, k=HIDDEN, seeds=(200, 201)):
    """DeepSeek-V3-shaped dense projection: W [n, k] N(0, 0.02);
    X [m, k] N(0, 1) with 1% of the K channels scaled x50."""
    w = normal_bf16((n, k), 0.02, seeds[0], device)
    x = normal_bf16((m, k), 1.0, seeds[1], device, 0.01, 50.0, outlier_channels=True)
    return {"w": w, "x": x}


def qat_forward(device="cpu", m=8192, n=HIDDEN, k=HIDDEN, r=16, seed=300):
    """QAT fake-quant forward: base W [n, k] N(0, 0.02), LoRA A [r, k] and
    B [n, r] N(0, 0.01), activations X [m, k] as the dense projection
    (seeds seed .. seed+3)."""
    w = normal_bf16((n, k), 0.02, seed, device)
    a = normal_bf16((r, k), 0.01, seed + 1, device)
    b = normal_bf16((n, r), 0.01, seed + 2, device)
    x = normal_bf16((m, k), 1.0, seed + 3, device, 0.01, 50.0, outlier_channels=True)
    return {"w": w, "lora_a": a, "lora_b": b, "x": x}


def qat_backward(device="cpu", m=8192, n=HIDDEN, k=HIDDEN, r=16, seed=310):
    """QAT backward for the LoRA factors: output gradient dY [m, n]
    N(0, 1e-3^2); activations X [m, k] as the dense projection (the caller
    fake-quantizes them when it wants X_hat); LoRA A [r, k], B [n, r]
    N(0, 0.01^2)."""
    dy = normal_bf16((m, n), 1e-3, seed, device)
    x = normal_bf16((m, k), 1.0, seed + 1, device, 0.01, 50.0, outlier_channels=True)
    a = normal_bf16((r, k), 0.01, seed + 2, device)
    b = normal_bf16((n, r), 0.01, seed + 3, device)
    return {"dy": dy, "x": x, "lora_a": a, "lora_b": b}


def expert_factors(n_experts=N_EXPERTS):
    """Per-expert scale c_e drawn log-uniform in [0.5, 2] (seed 400, float64)."""
    rng = np.random.default_rng(400)
    return np.exp(rng.uniform(math.log(0.5), math.log(2.0), size=n_experts))


def expert_weights(e, device="cpu", factors=None, inter=EXPERT_INTER, hidden=HIDDEN):
    """Expert e's gate [inter, hidden], up [inter, hidden], down [hidden, inter],
    N(0, (0.02 c_e)^2), drawn in that order from one generator seeded 4000+e."""
    if factors is None:
        factors = expert_factors()
    sigma = 0.02 * float(factors[e])
    g = _gen(4000 + e, device)
    out = []
    for shape in ((inter, hidden), (inter, hidden), (hidden, inter)):
        out.append((torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma)
                   .to(torch.bfloat16))
    return out


def zipf_routing(tokens=16384, n_experts=N_EXPERTS, top_k=TOP_K, s=1.1, seed=501):
    """Top-k routing with Zipf(s) expert popularity p_e ~ (e+1)^-s.

    Gumbel-top-k sampling (distinct experts per token) on the CPU in float64.
    Returns (token_ids int64 [tokens*top_k] grouped by expert, rows within a
    group ordered by token id; offsets int32 [n_experts+1])."""
    g = _gen(seed, "cpu")
    logp = -s * torch.log(torch.arange(1, n_experts + 1, dtype=torch.float64))
    u = torch.rand((tokens, n_experts), generator=g, dtype=torch.float64).clamp_(1e-300, 1.0)
    gumbel = -torch.log(-torch.log(u))
    experts = torch.topk(logp[None, :] + gumbel, top_k, dim=1).indices      # [tokens, k]
    tok = torch.arange(tokens).repeat_interleave(top_k)
    exp_flat = experts.reshape(-1)
    order = torch.argsort(exp_flat * tokens + tok)                          # by expert, then token
    counts = torch.bincount(exp_flat, minlength=n_experts)
    offsets = torch.zeros(n_experts + 1, dtype=torch.int64)
    offsets[1:] = torch.cumsum(counts, 0)
    return tok[order], offsets.to(torch.int32)


def moe_tokens(device="cpu", tokens=16384, seed=500):
    """MoE activations X [tokens, 7168] N(0,1) with 1% channels x50."""
    return normal_bf16((tokens, HIDDEN), 1.0, seed, device, 0.01, 50.0, outlier_channels=True)
