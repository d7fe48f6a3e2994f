"""Benchmark of the block-scaled FP8 hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input.  The
default workload is the largest one-GPU configuration, the grouped MoE
expert GEMM: 16384 tokens of hidden 7168 quantized per token in 1x128 tiles,
then the gate||up projection of their top-8 routed copies (Zipf(1.1) over
256 experts, sum M 131072, N 4096, K 7168) against MXFP8 expert weights,
fp32 accumulation, bf16 out:
    fp8_block_quantize(X 16384x7168, 1x128)
    -> fp8_grouped_gemm(A = routed rows, B = 256 experts' gate||up codes)
(the routed rows are gathered into expert order once, outside the timed
region).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  ``value`` is the step's throughput in GEMM TFLOP/s
(2*sum(M)*N*K per step over the measured step time).  ``roofline``
describes the dominant kernel (the GEMM): its average duration comes from HIP events on
the stream the kernel runs on, around a back-to-back loop of it run right
after the timed region (its time between per-launch events inside whole
steps, from the untimed pass below, is reported beside it).  ``components``
gives, for every kernel of the step, its time alone (``us``: the kernel run
back to back on the rotating inputs between one event pair, like the
dominant call) with the GB/s and roofline fraction that follow from it, and
its time inside whole steps (``us_in_step``: an untimed pass with an event
pair around each launch; such markers read several microseconds high for a
short kernel).  ``device_copy`` is the runtime's plain 512 MiB device-to-device
copy timed the same way after everything else, and each bandwidth-bound
component also gives its fraction of that copy's rate (``copy_frac``): a
second reference beside the 8 TB/s peak (the runtime's copy itself streams
well below the quantize kernels, so the fraction can exceed 1).

Other workloads (``--config``) print the same kind of line for their own
path: dense (the DeepSeek-V3-shaped dense projection: W 2048x7168 quantized
in 128x128 blocks and X 4096x7168 in 1x128 tiles in one batched launch,
GEMM 4096x2048x7168 with per-128-K promotion), mx (MXFP8 quantize of W
256x512 and X 64x512, MX x MX GEMM), qat
(LoRA merge + 128x128 fake-quant of W 7168x7168, 1x128 fake-quant of X
8192x7168, GEMM 8192x7168x7168), prequant (MXFP8 quantization of one MoE
layer's 256 routed experts), moe (the default, above), moe_gather
(the same with the routed rows read through row_index), moe_down (the
experts' down projection, K 2048, N 7168), dequant (the MXFP8 MoE layer
back to bf16), qat_backward (the QAT backward for the LoRA factors of the
qat step: dB and dA from dY 8192x7168 and the fake-quantized X 8192x7168,
rank 16) and prequant_nvfp4 (NVFP4 prequantization of the MoE layer's 256
routed experts, one fp32 scale per expert projection).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, TFLOP/s
MALL_BYTES = 256 << 20
HERE = os.path.dirname(os.path.abspath(__file__))
METRIC = "FP8 block-scaled GEMM TFLOPS + quantize GB/s, % of MI355X roofline"


def _lib():
    import block_scaled_fp8_amax_amd as fb
    fb.library()          # raises if the HIP library is missing: no fallback
    return fb


def _sets_for(bytes_per_set):
    """Number of rotating input sets so that a step never reads inputs that
    the previous two steps left in the Infinity Cache."""
    return max(2, int(np.ceil(2 * MALL_BYTES / bytes_per_set)) + 1)


class Events:
    """HIP event pairs on the current stream (the stream the library's
    launches go to), grouped by kernel name."""

    def __init__(self):
        self.ev = {}

    def around(self, name, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.ev.setdefault(name, []).append((s, e))

    def mean_ms(self):
        return {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.ev.items()}


class Workload:
    """A step is a list of (name, launch) pairs; ``bytes``/``flops`` hold
    each kernel's algorithmic work per launch."""

    def __init__(self, launches, dominant, bound, step_flops, step_bytes, kbytes, kflops, cfg, unit, dtype="fp8"):
        self.launches = launches          # i -> [(name, fn)]
        self.dominant = dominant
        self.bound = bound                # "mfma" or "hbm"
        self.step_flops = step_flops
        self.step_bytes = step_bytes
        self.kbytes = kbytes
        self.kflops = kflops
        self.cfg = cfg
        self.unit = unit                  # unit of ``value``
        self.dtype = dtype                # arithmetic type of the path


# ----------------------------------------------------------------- workloads

def dense_workload(fb, dev):
    import workloads
    M, N, K = 4096, 2048, 7168
    nsets = _sets_for((M * K + N * K) * 2)
    sets = []
    for i in range(nsets):
        d = workloads.dense_projection(dev, seeds=(200 + 2 * i, 201 + 2 * i))
        sets.append((d["w"], d["x"]))
    wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def launches(i):
        w, x = sets[i % nsets]
        # W (128x128 blocks) and X (1x128 tiles) quantized in one launch
        return [("quantize_w_x_batch",
                 lambda: fb.fp8_block_quantize_batch([(w, "128x128", "ceil", wq, ws), (x, "1x128", "ceil", xq, xs)])),
                ("gemm", lambda: fb.fp8_block_scaled_gemm(xq, xs, "1x128", wq, ws, "128x128", y))]

    flops = 2.0 * M * N * K
    kbytes = {
        # algorithmic bytes: read bf16, write codes + scales (W and X)
        "quantize_w_x_batch": N * K * 2 + N * K + (N // 128) * (K // 128) * 4 + M * K * 2 + M * K + M * (K // 128) * 4,
        # GEMM operand/result bytes (reported, not the bound)
        "gemm": M * K + N * K + M * (K // 128) * 4 + (N // 128) * (K // 128) * 4 + M * N * 2,
    }
    cfg = {"workload": "dense projection: quantize W 2048x7168 (128x128, fp32 scales) and X 4096x7168 "
                       "(1x128, fp32 scales) in one batched launch, block-scaled FP8 GEMM M4096 N2048 K7168, "
                       "bf16 out",
           "m": M, "n": N, "k": K, "input_sets": nsets}
    return Workload(launches, "gemm", "mfma", flops, sum(kbytes.values()), kbytes, {"gemm": flops}, cfg, "TFLOP/s")


def mx_workload(fb, dev):
    import workloads
    d = workloads.mx_small(dev)
    w, x = d["w"], d["x"]
    wq = torch.empty((256, 512), dtype=torch.uint8, device=dev)
    ws = torch.empty((256, 16), dtype=torch.uint8, device=dev)
    xq = torch.empty((64, 512), dtype=torch.uint8, device=dev)
    xs = torch.empty((64, 16), dtype=torch.uint8, device=dev)
    y = torch.empty((64, 256), dtype=torch.bfloat16, device=dev)

    # W and X are quantized in one batched launch (the same bytes as two
    # separate calls), then the MX x MX GEMM
    def launches(i):
        return [("quantize_w_x_1x32", lambda: fb.fp8_block_quantize_batch([(w, "1x32", "ceil", wq, ws),
                                                                           (x, "1x32", "ceil", xq, xs)])),
                ("gemm_mx", lambda: fb.fp8_block_scaled_gemm(xq, xs, "1x32", wq, ws, "1x32", y))]

    flops = 2.0 * 64 * 256 * 512
    kbytes = {"quantize_w_x_1x32": (256 + 64) * 512 * 3 + (256 + 64) * 16,
              "gemm_mx": 64 * 512 + 256 * 512 + 64 * 16 + 256 * 16 + 64 * 256 * 2}
    cfg = {"workload": "MXFP8 small case: quantize W 256x512 and X 64x512 (1x32, E8M0) in one batched launch, "
                       "GEMM 64x256x512, bf16 out (launch-latency bound, not roofline-meaningful)",
           "m": 64, "n": 256, "k": 512}
    return Workload(launches, "gemm_mx", "mfma", flops, sum(kbytes.values()), kbytes, {"gemm_mx": flops}, cfg,
                    "TFLOP/s")


def qat_workload(fb, dev):
    import workloads
    M, N, K, R = 8192, 7168, 7168, 16
    # two input sets (2 x 220 MB of W and X, more than the Infinity Cache)
    sets = [workloads.qat_forward(dev), workloads.qat_forward(dev, seed=350)]
    wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    wdq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    xdq = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def launches(i):
        d = sets[i % 2]
        w, la, lb, x = d["w"], d["lora_a"], d["lora_b"], d["x"]
        return [("merge_fake_quant_w", lambda: fb.fp8_fake_quant_merge(w, lb, la, wq, ws, wdq)),
                ("fake_quant_x_1x128", lambda: fb.fp8_block_quantize(x, "1x128", "ceil", xq, xs, xdq)),
                ("gemm", lambda: fb.fp8_block_scaled_gemm(xq, xs, "1x128", wq, ws, "128x128", y))]

    flops = 2.0 * M * N * K
    kbytes = {"merge_fake_quant_w": N * K * 2 + (N * R + R * K) * 2 + N * K + (N // 128) * (K // 128) * 4 + N * K * 2,
              "fake_quant_x_1x128": M * K * 2 + M * K + M * (K // 128) * 4 + M * K * 2,
              "gemm": M * K + N * K + M * (K // 128) * 4 + (N // 128) * (K // 128) * 4 + M * N * 2}
    cfg = {"workload": "QAT fake-quant forward: merge W 7168x7168 + B.A (rank 16) and fake-quantize "
                       "(128x128), fake-quantize X 8192x7168 (1x128), GEMM M8192 N7168 K7168, bf16 out",
           "m": M, "n": N, "k": K, "rank": R}
    return Workload(launches, "gemm", "mfma", flops, sum(kbytes.values()), kbytes, {"gemm": flops}, cfg, "TFLOP/s")


def prequant_workload(fb, dev):
    import workloads
    E, I, H = 256, 2048, 7168
    fac = workloads.expert_factors()
    # experts stacked per matrix shape: [gate; up] rows of every expert, then
    # every expert's down projection, so that one launch covers each shape
    gu = torch.empty((E * 2 * I, H), dtype=torch.bfloat16, device=dev)
    dn = torch.empty((E * H, I), dtype=torch.bfloat16, device=dev)
    for e in range(E):
        gate, up, down = workloads.expert_weights(e, dev, fac)
        gu[e * 2 * I:e * 2 * I + I].copy_(gate)
        gu[e * 2 * I + I:(e + 1) * 2 * I].copy_(up)
        dn[e * H:(e + 1) * H].copy_(down)
        del gate, up, down
    guq = torch.empty(gu.shape, dtype=torch.uint8, device=dev)
    gus = torch.empty((gu.shape[0], H // 32), dtype=torch.uint8, device=dev)
    dnq = torch.empty(dn.shape, dtype=torch.uint8, device=dev)
    dns = torch.empty((dn.shape[0], I // 32), dtype=torch.uint8, device=dev)

    def launches(i):
        return [("quantize_gate_up_1x32", lambda: fb.fp8_block_quantize(gu, "1x32", "ceil", guq, gus)),
                ("quantize_down_1x32", lambda: fb.fp8_block_quantize(dn, "1x32", "ceil", dnq, dns))]

    n_gu, n_dn = gu.numel(), dn.numel()
    kbytes = {"quantize_gate_up_1x32": n_gu * 3 + n_gu // 32, "quantize_down_1x32": n_dn * 3 + n_dn // 32}
    cfg = {"workload": "MXFP8 prequant of one MoE layer: 256 experts x {gate, up 2048x7168; down 7168x2048} bf16 "
                       "(22.5 GB) -> e4m3fn codes + uint8 E8M0 scales per 1x32 block; experts stacked per shape, "
                       "one launch per shape",
           "experts": E, "elements": n_gu + n_dn}
    return Workload(launches, "quantize_gate_up_1x32", "hbm", 0.0, sum(kbytes.values()), kbytes, {}, cfg, "GB/s")


def dequant_workload(fb, dev):
    """MXFP8 MoE layer back to bf16: the codes and E8M0 scales of the
    prequant workload (quantized while setting up) are dequantized."""
    import workloads
    E, I, H = 256, 2048, 7168
    fac = workloads.expert_factors()
    guq = torch.empty((E * 2 * I, H), dtype=torch.uint8, device=dev)
    gus = torch.empty((E * 2 * I, H // 32), dtype=torch.uint8, device=dev)
    dnq = torch.empty((E * H, I), dtype=torch.uint8, device=dev)
    dns = torch.empty((E * H, I // 32), dtype=torch.uint8, device=dev)
    for e in range(E):
        gate, up, down = workloads.expert_weights(e, dev, fac)
        fb.fp8_block_quantize(torch.cat([gate, up], 0), "1x32", "ceil", guq[e * 2 * I:(e + 1) * 2 * I],
                              gus[e * 2 * I:(e + 1) * 2 * I])
        fb.fp8_block_quantize(down, "1x32", "ceil", dnq[e * H:(e + 1) * H], dns[e * H:(e + 1) * H])
        del gate, up, down
    gux = torch.empty(guq.shape, dtype=torch.bfloat16, device=dev)
    dnx = torch.empty(dnq.shape, dtype=torch.bfloat16, device=dev)

    def launches(i):
        return [("dequantize_gate_up_1x32", lambda: fb.fp8_block_dequantize(guq, gus, "1x32", gux)),
                ("dequantize_down_1x32", lambda: fb.fp8_block_dequantize(dnq, dns, "1x32", dnx))]

    n_gu, n_dn = guq.numel(), dnq.numel()
    kbytes = {"dequantize_gate_up_1x32": n_gu * 3 + n_gu // 32, "dequantize_down_1x32": n_dn * 3 + n_dn // 32}
    cfg = {"workload": "MXFP8 MoE layer to bf16: 256 experts x {gate, up 2048x7168; down 7168x2048} e4m3fn codes "
                       "+ uint8 E8M0 scales per 1x32 block -> bf16 (22.5 GB written), one launch per shape",
           "experts": E, "elements": n_gu + n_dn}
    return Workload(launches, "dequantize_gate_up_1x32", "hbm", 0.0, sum(kbytes.values()), kbytes, {}, cfg, "GB/s")


def moe_workload(fb, dev):
    import workloads
    T, E, N, K = 16384, 256, 4096, 7168
    tok, off = workloads.zipf_routing()
    # two activation sets (2 x 235 MB, more than the 256 MB Infinity Cache)
    # rotate through the per-token quantize
    xsets = [workloads.moe_tokens(dev), workloads.moe_tokens(dev, seed=502)]
    xq = torch.empty((T, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, K // 128), dtype=torch.float32, device=dev)
    fb.fp8_block_quantize(xsets[0], "1x128", "ceil", xq, xs)
    idx = tok.to(dev)
    aq = xq.index_select(0, idx).contiguous()     # rows grouped by expert (gathered outside the timed region)
    sa = xs.index_select(0, idx).contiguous()
    bq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    fac = workloads.expert_factors()
    for e in range(E):
        gate, up, _ = workloads.expert_weights(e, dev, fac)
        fb.fp8_block_quantize(torch.cat([gate, up], 0), "1x32", "ceil", bq[e], sb[e])
    offt = off.to(dev)
    total_m = int(off[-1])
    y = torch.empty((total_m, N), dtype=torch.bfloat16, device=dev)

    def launches(i):
        x = xsets[i % 2]
        return [("quantize_x_1x128", lambda: fb.fp8_block_quantize(x, "1x128", "ceil", xq, xs)),
                ("grouped_gemm", lambda: fb.fp8_grouped_gemm(aq, sa, "1x128", bq, sb, "1x32", offt, y))]

    flops = 2.0 * total_m * N * K
    kbytes = {"quantize_x_1x128": T * K * 3 + T * (K // 128) * 4,
              "grouped_gemm": total_m * K + total_m * (K // 128) * 4 + E * N * K + E * N * (K // 32) +
                              total_m * N * 2 + (E + 1) * 4}
    sizes = (off[1:] - off[:-1]).numpy()
    cfg = {"workload": "MoE gate||up: quantize X 16384x7168 (1x128), grouped block-scaled FP8 GEMM over 256 "
                       "experts (Zipf(1.1) top-8, sum M 131072, N 4096, K 7168, MXFP8 weights), bf16 out",
           "total_m": total_m, "n": N, "k": K, "groups": E,
           "group_m_max": int(sizes.max()), "group_m_min": int(sizes.min()), "group_m_median": float(np.median(sizes))}
    return Workload(launches, "grouped_gemm", "mfma", flops, sum(kbytes.values()), kbytes, {"grouped_gemm": flops},
                    cfg, "TFLOP/s")


def moe_gather_workload(fb, dev):
    """The MoE gate||up step without the permuted copy: per-token quantize of
    X, then the grouped GEMM reads each routed row through row_index."""
    import workloads
    T, E, N, K = 16384, 256, 4096, 7168
    tok, off = workloads.zipf_routing()
    xsets = [workloads.moe_tokens(dev), workloads.moe_tokens(dev, seed=502)]   # rotated, as in the moe step
    xq = torch.empty((T, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((T, K // 128), dtype=torch.float32, device=dev)
    idx = tok.to(torch.int32).to(dev)
    bq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    fac = workloads.expert_factors()
    for e in range(E):
        gate, up, _ = workloads.expert_weights(e, dev, fac)
        fb.fp8_block_quantize(torch.cat([gate, up], 0), "1x32", "ceil", bq[e], sb[e])
    offt = off.to(dev)
    total_m = int(off[-1])
    y = torch.empty((total_m, N), dtype=torch.bfloat16, device=dev)

    def launches(i):
        x = xsets[i % 2]
        return [("quantize_x_1x128", lambda: fb.fp8_block_quantize(x, "1x128", "ceil", xq, xs)),
                ("grouped_gemm_gather",
                 lambda: fb.fp8_grouped_gemm_gather(xq, xs, "1x128", idx, bq, sb, "1x32", offt, y))]

    flops = 2.0 * total_m * N * K
    kbytes = {"quantize_x_1x128": T * K * 3 + T * (K // 128) * 4,
              "grouped_gemm_gather": T * K + T * (K // 128) * 4 + total_m * 4 + E * N * K + E * N * (K // 32) +
                                     total_m * N * 2 + (E + 1) * 4}
    cfg = {"workload": "MoE gate||up with gathered rows: quantize X 16384x7168 (1x128), grouped FP8 GEMM reading "
                       "the 131072 routed rows through row_index (Zipf(1.1) top-8, 256 experts, N 4096, K 7168, "
                       "MXFP8 weights), bf16 out",
           "tokens": T, "total_m": total_m, "n": N, "k": K, "groups": E}
    return Workload(launches, "grouped_gemm_gather", "mfma", flops, sum(kbytes.values()), kbytes,
                    {"grouped_gemm_gather": flops}, cfg, "TFLOP/s")


def moe_down_workload(fb, dev):
    """The MoE down projection: per-row quantize of the routed intermediate
    activations (131072 x 2048), grouped GEMM against the experts' MXFP8
    down weights (N 7168, K 2048)."""
    import workloads
    E, N, K = 256, 7168, 2048
    tok, off = workloads.zipf_routing()
    total_m = int(off[-1])
    h = workloads.normal_bf16((total_m, K), 1.0, 510, dev)
    hq = torch.empty((total_m, K), dtype=torch.uint8, device=dev)
    hs = torch.empty((total_m, K // 128), dtype=torch.float32, device=dev)
    bq = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    fac = workloads.expert_factors()
    for e in range(E):
        _, _, down = workloads.expert_weights(e, dev, fac)
        fb.fp8_block_quantize(down, "1x32", "ceil", bq[e], sb[e])
    offt = off.to(dev)
    y = torch.empty((total_m, N), dtype=torch.bfloat16, device=dev)

    def launches(i):
        return [("quantize_h_1x128", lambda: fb.fp8_block_quantize(h, "1x128", "ceil", hq, hs)),
                ("grouped_gemm_down", lambda: fb.fp8_grouped_gemm(hq, hs, "1x128", bq, sb, "1x32", offt, y))]

    flops = 2.0 * total_m * N * K
    kbytes = {"quantize_h_1x128": total_m * K * 3 + total_m * (K // 128) * 4,
              "grouped_gemm_down": total_m * K + total_m * (K // 128) * 4 + E * N * K + E * N * (K // 32) +
                                   total_m * N * 2 + (E + 1) * 4}
    cfg = {"workload": "MoE down projection: quantize the routed intermediate 131072x2048 (1x128), grouped FP8 GEMM "
                       "over 256 experts (Zipf(1.1) top-8, N 7168, K 2048, MXFP8 down weights), bf16 out",
           "total_m": total_m, "n": N, "k": K, "groups": E}
    return Workload(launches, "grouped_gemm_down", "mfma", flops, sum(kbytes.values()), kbytes,
                    {"grouped_gemm_down": flops}, cfg, "TFLOP/s")


def prequant_nvfp4_workload(fb, dev):
    """NVFP4 prequant of one MoE layer's 256 routed experts, stacked per
    shape as for MXFP8; every expert projection (gate, up, down) is its own
    tensor with its own amax and fp32 scale."""
    import workloads
    E, I, H = 256, 2048, 7168
    fac = workloads.expert_factors()
    gu = torch.empty((E * 2 * I, H), dtype=torch.bfloat16, device=dev)
    dn = torch.empty((E * H, I), dtype=torch.bfloat16, device=dev)
    for e in range(E):
        gate, up, down = workloads.expert_weights(e, dev, fac)
        gu[e * 2 * I:e * 2 * I + I].copy_(gate)
        gu[e * 2 * I + I:(e + 1) * 2 * I].copy_(up)
        dn[e * H:(e + 1) * H].copy_(down)
        del gate, up, down
    guq = torch.empty((gu.shape[0], H // 2), dtype=torch.uint8, device=dev)
    gus = torch.empty((gu.shape[0], H // 16), dtype=torch.uint8, device=dev)
    gug = torch.empty((2 * E,), dtype=torch.float32, device=dev)
    gua = torch.empty((2 * E,), dtype=torch.float32, device=dev)
    dnq = torch.empty((dn.shape[0], I // 2), dtype=torch.uint8, device=dev)
    dns = torch.empty((dn.shape[0], I // 16), dtype=torch.uint8, device=dev)
    dng = torch.empty((E,), dtype=torch.float32, device=dev)
    dna = torch.empty((E,), dtype=torch.float32, device=dev)

    def launches(i):
        return [("nvfp4_gate_up", lambda: fb.fp8_nvfp4_quantize(gu, I, guq, gus, gug, gua)),
                ("nvfp4_down", lambda: fb.fp8_nvfp4_quantize(dn, H, dnq, dns, dng, dna))]

    # algorithmic bytes: bf16 read once, packed codes (1/2 B) and block scales
    # (1/16 B) written, per element; the per-tensor amax is a second read of
    # each tensor that the algorithm's two-level scale needs
    n_gu, n_dn = gu.numel(), dn.numel()
    kbytes = {"nvfp4_gate_up": n_gu * 2 + n_gu // 2 + n_gu // 16 + 2 * E * 8,
              "nvfp4_down": n_dn * 2 + n_dn // 2 + n_dn // 16 + E * 8}
    cfg = {"workload": "NVFP4 prequant of one MoE layer: 256 experts x {gate, up 2048x7168; down 7168x2048} bf16 "
                       "(22.5 GB) -> packed E2M1 codes + e4m3 1x16 block scales + one fp32 scale per expert "
                       "projection (768 tensors); experts stacked per shape, one call per shape",
           "experts": E, "elements": n_gu + n_dn, "tensors": 3 * E}
    return Workload(launches, "nvfp4_gate_up", "hbm", 0.0, sum(kbytes.values()), kbytes, {}, cfg, "GB/s",
                    dtype="fp4")


def dequant_nvfp4_workload(fb, dev):
    """NVFP4 MoE layer back to bf16: the packed codes, e4m3 block scales and
    per-tensor scales of the NVFP4 prequant workload (quantized while
    setting up) are dequantized, one call per stacked shape."""
    import workloads
    E, I, H = 256, 2048, 7168
    fac = workloads.expert_factors()
    guq = torch.empty((E * 2 * I, H // 2), dtype=torch.uint8, device=dev)
    gus = torch.empty((E * 2 * I, H // 16), dtype=torch.uint8, device=dev)
    gug = torch.empty((2 * E,), dtype=torch.float32, device=dev)
    dnq = torch.empty((E * H, I // 2), dtype=torch.uint8, device=dev)
    dns = torch.empty((E * H, I // 16), dtype=torch.uint8, device=dev)
    dng = torch.empty((E,), dtype=torch.float32, device=dev)
    amax = torch.empty((2,), dtype=torch.float32, device=dev)
    for e in range(E):
        gate, up, down = workloads.expert_weights(e, dev, fac)
        for j, wt in enumerate((gate, up)):
            r0 = e * 2 * I + j * I
            fb.fp8_nvfp4_quantize(wt, I, guq[r0:r0 + I], gus[r0:r0 + I], gug[2 * e + j:2 * e + j + 1], amax[:1])
        fb.fp8_nvfp4_quantize(down, H, dnq[e * H:(e + 1) * H], dns[e * H:(e + 1) * H], dng[e:e + 1], amax[1:])
        del gate, up, down
    gux = torch.empty((E * 2 * I, H), dtype=torch.bfloat16, device=dev)
    dnx = torch.empty((E * H, I), dtype=torch.bfloat16, device=dev)

    def launches(i):
        return [("nvfp4_dequantize_gate_up", lambda: fb.fp8_nvfp4_dequantize(guq, gus, gug, I, gux)),
                ("nvfp4_dequantize_down", lambda: fb.fp8_nvfp4_dequantize(dnq, dns, dng, H, dnx))]

    # algorithmic bytes: packed codes (1/2 B) and block scales (1/16 B) read,
    # bf16 written, per element
    n_gu, n_dn = gux.numel(), dnx.numel()
    kbytes = {"nvfp4_dequantize_gate_up": n_gu * 2 + n_gu // 2 + n_gu // 16 + 2 * E * 4,
              "nvfp4_dequantize_down": n_dn * 2 + n_dn // 2 + n_dn // 16 + E * 4}
    cfg = {"workload": "NVFP4 MoE layer to bf16: 256 experts x {gate, up 2048x7168; down 7168x2048} packed E2M1 "
                       "codes + e4m3 1x16 block scales + one fp32 scale per expert projection -> bf16 (22.5 GB "
                       "written); experts stacked per shape, one call per shape",
           "experts": E, "elements": n_gu + n_dn, "tensors": 3 * E}
    return Workload(launches, "nvfp4_dequantize_gate_up", "hbm", 0.0, sum(kbytes.values()), kbytes, {}, cfg,
                    "GB/s", dtype="fp4")


def qat_backward_workload(fb, dev):
    """QAT backward for the LoRA factors of the qat step: dB [7168 x 16] and
    dA [16 x 7168] from the output gradient dY 8192x7168 and the
    fake-quantized activations X_hat 8192x7168 (the 1x128 fake-quant output
    of the forward), bf16 in and out, fp32 accumulation."""
    import workloads
    M, N, K, R = 8192, 7168, 7168, 16
    nsets = _sets_for((M * N + M * K) * 2)
    sets = []
    for i in range(nsets):
        d = workloads.qat_backward(dev, M, N, K, R, seed=310 + 10 * i)
        _, _, xdq = fb.quantize(d["x"], "1x128", dequant=True)
        sets.append((d["dy"], xdq, d["lora_b"], d["lora_a"]))
        del d
    ws = torch.empty(fb.fp8_lora_backward_workspace(M, N, K, R), dtype=torch.uint8, device=dev)
    db = torch.empty((N, R), dtype=torch.bfloat16, device=dev)
    da = torch.empty((R, K), dtype=torch.bfloat16, device=dev)

    def launches(i):
        dy, x, b, a = sets[i % nsets]
        return [("lora_backward", lambda: fb.fp8_lora_backward(dy, x, b, a, ws, db, da))]

    # algorithmic bytes: dY and X_hat once, the factors, the two gradients
    kbytes = {"lora_backward": (M * N + M * K) * 2 + 2 * (N * R + R * K) * 2}
    flops = 4.0 * M * R * (N + K)       # P, Q, dB and dA: 2*M*R*K + 2*M*R*N + 2*M*R*N + 2*M*R*K
    cfg = {"workload": "QAT backward for the LoRA factors: dB = dY^T (X_hat A^T), dA = (dY B)^T X_hat with dY "
                       "8192x7168, X_hat 8192x7168 (1x128 fake-quant of X), rank 16, bf16 in/out, fp32 accumulation",
           "m": M, "n": N, "k": K, "rank": R, "input_sets": nsets,
           "workspace_bytes": int(ws.numel())}
    return Workload(launches, "lora_backward", "hbm", flops, sum(kbytes.values()), kbytes, {}, cfg, "GB/s",
                    dtype="bf16")


WORKLOADS = {"dense": dense_workload, "mx": mx_workload, "qat": qat_workload, "prequant": prequant_workload,
             "moe": moe_workload, "moe_gather": moe_gather_workload, "moe_down": moe_down_workload,
             "dequant": dequant_workload, "qat_backward": qat_backward_workload,
             "prequant_nvfp4": prequant_nvfp4_workload, "dequant_nvfp4": dequant_nvfp4_workload}


# ------------------------------------------------------------ traffic record

# Sources that determine each workload's dominant call; a committed counter
# summary is used only while these hash to the value recorded with it.
_TRAFFIC_SOURCES = {
    "dense": ("gemm.hip", "device.h"), "mx": ("gemm.hip", "device.h"), "qat": ("gemm.hip", "device.h"),
    "moe": ("gemm.hip", "device.h"), "moe_gather": ("gemm.hip", "device.h"), "moe_down": ("gemm.hip", "device.h"),
    "prequant": ("quantize.hip", "device.h"), "dequant": ("dequant.hip", "device.h"),
    "qat_backward": ("lora_bwd.hip", "device.h"), "prequant_nvfp4": ("nvfp4.hip", "device.h"),
    "dequant_nvfp4": ("nvfp4.hip", "device.h"),
}


def _kernel_source_hash(config):
    h = hashlib.sha256()
    for f in _TRAFFIC_SOURCES[config]:
        with open(os.path.join(HERE, "block_scaled_fp8_amax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(config):
    """HBM bytes per launch of the dominant call from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE of its kernels, each
    scaled by the factor a plain copy of known size gives).  None when there
    is no summary for this workload or its kernel sources changed since."""
    path = os.path.join(HERE, "profiles", f"traffic_{config}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256") != _kernel_source_hash(config):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------- cpu baseline

def _oracle_threads():
    """Threads the oracle runs on: its arithmetic is numpy elementwise work
    (one thread), and any BLAS call it makes is pinned to one thread while
    the baseline is timed (``_one_thread``)."""
    return 1


class _one_thread:
    """Limit BLAS / OpenMP pools to one thread while the oracle is timed."""

    def __enter__(self):
        self._ctl = None
        try:
            import threadpoolctl
            self._ctl = threadpoolctl.threadpool_limits(1)
        except Exception:  # noqa: BLE001
            pass
        return self

    def __exit__(self, *exc):
        if self._ctl is not None:
            self._ctl.restore_original_limits()
        return False


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_dense(sample_rows=256):
    """The oracle on a 1/16 row slice of the same step (256 of the 4096
    activation rows, 128 of the 2048 weight rows, and the GEMM of the 256
    rows against all 2048 weight rows), timed on this host's cores."""
    import workloads
    from oracle import gemm as ogemm, quant as oquant
    d = workloads.dense_projection("cpu", m=sample_rows, n=2048)
    wb = workloads.bf16_bits(d["w"])
    xb = workloads.bf16_bits(d["x"])
    t0 = time.perf_counter()
    oquant.quantize(wb[:128], "128x128")                  # 1/16 of the weight quantization
    t1 = time.perf_counter()
    xq, xs, _ = oquant.quantize(xb, "1x128")
    t2 = time.perf_counter()
    wq_full, ws_full, _ = oquant.quantize(wb, "128x128")   # operands for the GEMM (not timed)
    t3 = time.perf_counter()
    ogemm.gemm_ref32(xq, xs, "1x128", wq_full, ws_full, "128x128")
    t4 = time.perf_counter()
    secs = (t1 - t0) + (t2 - t1) + (t4 - t3)
    flops = 2.0 * sample_rows * 2048 * 7168
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"1/16 row slice of the step: quantize W rows 0..127 (128x128), quantize X "
                      f"{sample_rows}x7168 (1x128), GEMM {sample_rows}x2048x7168 fp32-accumulated; "
                      f"{secs:.2f} s on the host"}


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def cpu_baseline_mx():
    """The oracle on the whole MXFP8 small step (it is small)."""
    import workloads
    from oracle import gemm as ogemm, quant as oquant
    d = workloads.mx_small("cpu")
    wb, xb = workloads.bf16_bits(d["w"]), workloads.bf16_bits(d["x"])
    (w, dt1) = _timed(lambda: oquant.quantize(wb, "1x32"))
    (x, dt2) = _timed(lambda: oquant.quantize(xb, "1x32"))
    (_, dt3) = _timed(lambda: ogemm.gemm_ref32(x[0], x[1], "1x32", w[0], w[1], "1x32"))
    secs = dt1 + dt2 + dt3
    return {"value": 2.0 * 64 * 256 * 512 / secs / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"the whole step (quantize W and X 1x32, GEMM 64x256x512); {secs:.3f} s"}


def cpu_baseline_qat(rows=128):
    """The oracle on a row slice of the QAT step: merge + fake-quant of 128
    of the 7168 weight rows, fake-quant of 128 of the 8192 activation rows,
    and their GEMM against the full merged weight."""
    import workloads
    from oracle import gemm as ogemm, merge as omerge, quant as oquant
    d = workloads.qat_forward("cpu", m=rows)
    wb, ab, bb, xb = (workloads.bf16_bits(d[k]) for k in ("w", "lora_a", "lora_b", "x"))
    (_, dt1) = _timed(lambda: omerge.fake_quant_merge(wb[:rows], bb[:rows], ab))
    (x, dt2) = _timed(lambda: oquant.quantize(xb, "1x128"))
    wq, ws, _ = oquant.quantize(wb, "128x128")             # GEMM operand (not timed)
    (_, dt3) = _timed(lambda: ogemm.gemm_ref32(x[0], x[1], "1x128", wq, ws, "128x128"))
    secs = dt1 + dt2 + dt3
    return {"value": 2.0 * rows * 7168 * 7168 / secs / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"merge + fake-quant of W rows 0..{rows - 1}, fake-quant of X {rows}x7168, "
                                        f"GEMM {rows}x7168x7168 (about 1/60 of the step); {secs:.2f} s"}


def cpu_baseline_quant_expert(dequant=False):
    """The oracle on one expert's gate projection (2048x7168, 1x32), about
    1/770 of the MoE layer's elements."""
    import workloads
    from oracle import quant as oquant
    gate, _, _ = workloads.expert_weights(0, "cpu")
    gb = workloads.bf16_bits(gate)
    n = gb.size
    if dequant:
        q, sc, _ = oquant.quantize(gb, "1x32")
        (_, secs) = _timed(lambda: oquant.dequantize(q, sc, "1x32"))
        what = "dequantize"
    else:
        (_, secs) = _timed(lambda: oquant.quantize(gb, "1x32"))
        what = "quantize"
    return {"value": (n * 3 + n / 32) / secs / 1e9, "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"{what} of expert 0's gate projection 2048x7168 (1x32, E8M0); {secs:.2f} s"}


def cpu_baseline_grouped(n=4096, k=7168, rows=1024, down=False):
    """The oracle on one routed slice of the grouped step: quantize ``rows``
    activation rows (1x128) and their GEMM against one expert's weights."""
    import workloads
    from oracle import gemm as ogemm, quant as oquant
    x = workloads.normal_bf16((rows, k), 1.0, 520, "cpu", 0.01, 50.0, outlier_channels=True)
    gate, up, dn = workloads.expert_weights(0, "cpu")
    w = dn if down else torch.cat([gate, up], 0)
    wq, ws, _ = oquant.quantize(workloads.bf16_bits(w), "1x32")   # expert weights (not timed)
    (xq, dt1) = _timed(lambda: oquant.quantize(workloads.bf16_bits(x), "1x128"))
    (_, dt2) = _timed(lambda: ogemm.grouped_gemm_ref(xq[0], xq[1], "1x128", wq[None], ws[None], "1x32",
                                                      [0, rows]))
    secs = dt1 + dt2
    return {"value": 2.0 * rows * n * k / secs / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"quantize {rows}x{k} (1x128) and one expert's GEMM {rows}x{n}x{k}; "
                                        f"{secs:.2f} s"}


def cpu_baseline_qat_backward(rows=2048):
    """The oracle on a token slice of the QAT backward: dB and dA from 2048
    of the 8192 token rows of dY and X_hat (every column)."""
    import workloads
    from oracle import lora_grad
    d = workloads.qat_backward("cpu", m=rows)
    bits = [workloads.bf16_bits(d[k]) for k in ("dy", "x", "lora_b", "lora_a")]
    (_, secs) = _timed(lambda: lora_grad.lora_grads(*bits))
    nbytes = rows * (7168 + 7168) * 2 + 2 * (7168 * 16 + 16 * 7168) * 2
    return {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"dB, dA from {rows} of the 8192 token rows (1/{8192 // rows} of the step), float64 with dW "
                      f"formed; {secs:.2f} s"}


def cpu_baseline_nvfp4(dequant=False):
    """The oracle on one expert's gate projection (2048x7168), about 1/768
    of the MoE layer's elements."""
    import workloads
    from oracle import nvfp4 as onv
    gate, _, _ = workloads.expert_weights(0, "cpu")
    gb = workloads.bf16_bits(gate)
    n = gb.size
    if dequant:
        packed, bs, g, _, _ = onv.quantize(gb)
        (_, secs) = _timed(lambda: onv.dequantize(packed, bs, g, gb.shape[0]))
        what = "dequantize"
    else:
        (_, secs) = _timed(lambda: onv.quantize(gb))
        what = "quantize"
    return {"value": (n * 2 + n / 2 + n / 16) / secs / 1e9, "unit": "GB/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"NVFP4 {what} of expert 0's gate projection 2048x7168; {secs:.2f} s"}


CPU_BASELINES = {
    "dense": lambda: cpu_baseline_dense(),
    "mx": cpu_baseline_mx,
    "qat": lambda: cpu_baseline_qat(),
    "prequant": lambda: cpu_baseline_quant_expert(False),
    "dequant": lambda: cpu_baseline_quant_expert(True),
    "moe": lambda: cpu_baseline_grouped(),
    "moe_gather": lambda: cpu_baseline_grouped(),
    "moe_down": lambda: cpu_baseline_grouped(n=7168, k=2048, down=True),
    "qat_backward": lambda: cpu_baseline_qat_backward(),
    "prequant_nvfp4": lambda: cpu_baseline_nvfp4(False),
    "dequant_nvfp4": lambda: cpu_baseline_nvfp4(True),
}


# ---------------------------------------------------------------------- main

_SPIN_PER_MS = None


def _spin_ms(ms):
    """Queue a device spin of about ``ms`` milliseconds on the current stream
    (torch's sleep kernel, calibrated once with events)."""
    global _SPIN_PER_MS
    if _SPIN_PER_MS is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_PER_MS = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(min(ms, 2000.0) * _SPIN_PER_MS))


def device_copy_gbs(nbytes=1 << 29, reps=5):
    """Read + write bytes per second of a plain device-to-device copy of
    nbytes (twice the Infinity Cache, so it streams from HBM), on the
    current stream between one event pair."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def run(args):
    fb = _lib()
    dev = "cuda"
    wl = WORKLOADS[args.config](fb, dev)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        for _, fn in wl.launches(i):
            fn()
    torch.cuda.synchronize()

    # host cost of enqueueing one step (the GPU runs behind the host here)
    h0 = time.perf_counter()
    for i in range(max(1, args.warmup)):
        for _, fn in wl.launches(i):
            fn()
    host_ms = (time.perf_counter() - h0) * 1e3 / max(1, args.warmup)
    torch.cuda.synchronize()

    # timed region: K whole steps between one event pair, nothing else on
    # the stream.  A spin kernel queued first keeps the GPU busy while the
    # host enqueues the steps, so the GPU-side timestamps see back-to-back
    # device work and not the host's launch overhead.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _spin_ms(1.5 * host_ms * args.steps + 2.0)
    t_start.record()
    for i in range(args.steps):
        for name, fn in wl.launches(args.warmup + i):
            fn()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # the dominant call alone, back to back on the same stream, between one
    # event pair: its average duration per launch without the per-launch
    # event markers (which add several microseconds to a short kernel)
    nd = max(args.steps, 20)
    dom_fns = [fn for i in range(nd) for name, fn in wl.launches(args.warmup + args.steps + i) if name == wl.dominant]
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _spin_ms(1.5 * host_ms * nd + 2.0)
    d0.record()
    for fn in dom_fns:
        fn()
    d1.record()
    torch.cuda.synchronize()
    dom_ms = d0.elapsed_time(d1) / len(dom_fns)

    # untimed pass: every kernel on its own
    comp = Events()
    torch.cuda.synchronize()
    nc = max(1, min(args.steps, 10))
    _spin_ms(1.5 * host_ms * nc + 2.0)
    for i in range(nc):
        for name, fn in wl.launches(i):
            comp.around(name, fn)
    torch.cuda.synchronize()
    in_step = comp.mean_ms()

    # every other kernel alone as well, back to back on the step's rotating
    # inputs between one event pair, as the dominant call above: a marker
    # pair around a single short launch reads several microseconds high
    alone = {wl.dominant: dom_ms}
    base = args.warmup + args.steps + nd
    for name in in_step:
        if name in alone:
            continue
        fns = [fn for i in range(nd) for n2, fn in wl.launches(base + i) if n2 == name]
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        _spin_ms(1.5 * host_ms * nd + 2.0)
        a0.record()
        for fn in fns:
            fn()
        a1.record()
        torch.cuda.synchronize()
        alone[name] = a0.elapsed_time(a1) / len(fns)

    components = {}
    for name, ms_step in in_step.items():
        ms = alone[name]
        c = {"us": ms * 1e3, "us_in_step": ms_step * 1e3}
        if name in wl.kbytes:
            c["GB/s"] = wl.kbytes[name] / (ms * 1e-3) / 1e9
            c["hbm_frac"] = c["GB/s"] / HBM_PEAK_GBS
        if name in wl.kflops:
            c["TFLOP/s"] = wl.kflops[name] / (ms * 1e-3) / 1e12
            c["mfma_frac"] = c["TFLOP/s"] / FP8_PEAK_TFLOPS
        components[name] = c
    copy_gbs = device_copy_gbs()
    for name, c in components.items():
        if "GB/s" in c and name not in wl.kflops:
            c["copy_frac"] = c["GB/s"] / copy_gbs

    if wl.bound == "mfma":
        achieved = wl.kflops[wl.dominant] / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / FP8_PEAK_TFLOPS}
    else:
        achieved = wl.kbytes[wl.dominant] / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    roof["traffic"] = recorded_traffic(args.config)
    roof["kernel"] = wl.dominant
    roof["kernel_us"] = dom_ms * 1e3
    roof["kernel_us_in_step"] = components[wl.dominant]["us_in_step"]
    roof["host_enqueue_us_per_step"] = host_ms * 1e3

    if wl.unit == "TFLOP/s":
        value = wl.step_flops / (ms_per_step * 1e-3) / 1e12
    else:
        value = wl.step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": value,
        "unit": wl.unit,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic, seeded: N(0,0.02) weights (routed experts scaled log-uniform in [0.5,2]), N(0,1) "
                "activations with 1% of channels x50, Zipf(1.1) top-8 routing over 256 experts",
        "config": wl.cfg,
        "components": components,
        "roofline": roof,
        "device_copy": {"GB/s": copy_gbs, "bytes_per_copy": 2 * (1 << 29)},
    }
    if not args.no_cpu_baseline:
        with _one_thread():
            cb = CPU_BASELINES[args.config]()
        cb["cpu_model"] = _cpu_model()
        cb["host_cpus"] = os.cpu_count()
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


def copy_calibration(args):
    """Plain device copies of a known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(max(1, args.steps)):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": max(1, args.steps)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="moe", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 1 GiB device copies (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(a sharded deployment would run one independent copy per GPU)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
