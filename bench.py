"""Benchmark of the block-scaled FP8 hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input of the
DeepSeek-V3-shaped dense projection (weights bf16 2048x7168 quantized in
128x128 blocks, activations bf16 4096x7168 quantized per token in 1x128
tiles, block-scaled FP8 GEMM M=4096 N=2048 K=7168, bf16 out):
    fp8_block_quantize(W, 128x128) -> fp8_block_quantize(X, 1x128)
    -> fp8_block_scaled_gemm(A=X codes, B=W codes)
Inputs are resident in HBM before timing starts; several input sets rotate
so that no step finds its inputs in the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is the whole step's throughput in GEMM
TFLOP/s (2*M*N*K per step over the step time); per-kernel times, GB/s and
roofline fractions are in ``components``; ``roofline`` is the dominant
kernel (the GEMM) timed with HIP events on the stream it runs on.

Other workloads (``--config``) print the same kind of line for their own
path: mx (the MXFP8 small case), qat (merge + fake-quant + GEMM), prequant
(MXFP8 quantization of one MoE layer's 256 routed experts), moe (per-token
quantize + grouped expert GEMM).
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA, TFLOP/s
MALL_BYTES = 256 << 20


def _lib():
    import block_scaled_fp8_amax_amd as fb
    fb.library()          # raises if the HIP library is missing: no fallback
    return fb


class KernelTimer:
    """HIP events on the current stream around every launch of each kernel."""

    def __init__(self):
        self.ev = {}

    def __call__(self, name, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.ev.setdefault(name, []).append((s, e))

    def mean_ms(self):
        return {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.ev.items()}


# ----------------------------------------------------------------- workloads

def dense_workload(fb, dev):
    import workloads
    M, N, K = 4096, 2048, 7168
    per_set = (M * K + N * K) * 2
    nsets = max(2, int(np.ceil(2 * MALL_BYTES / per_set)) + 1)
    sets = []
    for i in range(nsets):
        d = workloads.dense_projection(dev, seeds=(200 + 2 * i, 201 + 2 * i))
        sets.append((d["w"], d["x"]))
    wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(i, timer):
        w, x = sets[i % nsets]
        timer("quantize_w_128x128", lambda: fb.fp8_block_quantize(w, "128x128", "ceil", wq, ws))
        timer("quantize_x_1x128", lambda: fb.fp8_block_quantize(x, "1x128", "ceil", xq, xs))
        timer("gemm", lambda: fb.fp8_block_scaled_gemm(xq, xs, "1x128", wq, ws, "128x128", y))

    flops = 2.0 * M * N * K
    comp_bytes = {
        # algorithmic bytes: read bf16, write codes + scales
        "quantize_w_128x128": N * K * 2 + N * K + (N // 128) * (K // 128) * 4,
        "quantize_x_1x128": M * K * 2 + M * K + M * (K // 128) * 4,
        # GEMM operand/result bytes (reported, not the bound)
        "gemm": M * K + N * K + M * (K // 128) * 4 + (N // 128) * (K // 128) * 4 + M * N * 2,
    }
    comp_flops = {"gemm": flops}
    cfg = {"workload": "dense projection W 2048x7168 (128x128) + X 4096x7168 (1x128) + GEMM M4096 N2048 K7168",
           "m": M, "n": N, "k": K, "input_sets": nsets}
    return step, flops, comp_bytes, comp_flops, cfg, "gemm", sets[0]


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
    threads = torch.get_num_threads()
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:  # noqa: BLE001
        pass
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"1/16 row slice of the step: quantize W rows 0..127 (128x128), quantize X "
                      f"{sample_rows}x7168 (1x128), GEMM {sample_rows}x2048x7168 fp32-accumulated; "
                      f"{secs:.2f} s on the host"}


# ---------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dense", choices=["dense"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(a sharded deployment would run one independent copy per GPU)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fb = _lib()
    dev = "cuda"
    step, flops, comp_bytes, comp_flops, cfg, dominant, _ = dense_workload(fb, dev)
    torch.cuda.synchronize()
    warm = KernelTimer()
    for i in range(args.warmup):
        step(i, warm)
    torch.cuda.synchronize()
    timer = KernelTimer()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(args.warmup + i, timer)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    kms = timer.mean_ms()
    components = {}
    for name, ms in kms.items():
        c = {"us": ms * 1e3}
        if name in comp_bytes:
            c["GB/s"] = comp_bytes[name] / (ms * 1e-3) / 1e9
            c["hbm_frac"] = c["GB/s"] / HBM_PEAK_GBS
        if name in comp_flops:
            c["TFLOP/s"] = comp_flops[name] / (ms * 1e-3) / 1e12
            c["mfma_frac"] = c["TFLOP/s"] / FP8_PEAK_TFLOPS
        components[name] = c
    dom_ms = kms[dominant]
    achieved = comp_flops[dominant] / (dom_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / FP8_PEAK_TFLOPS, "traffic": None, "kernel": "gemm_kernel<kF32xF32,bf16>"}
    out = {
        "metric": "FP8 block-scaled GEMM TFLOPS + quantize GB/s, % of MI355X roofline",
        "value": flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3fn x fp8_e4m3fn -> fp32 accumulate, bf16 out",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations with 1% channels x50)",
        "config": cfg,
        "components": components,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_dense()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
