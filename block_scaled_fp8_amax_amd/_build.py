"""Builds libfp8blk.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m block_scaled_fp8_amax_amd._build``; ``__graft_entry__.build``
calls :func:`build`.  Objects go to ``_build/`` at the repository root and the
shared library into this package directory, next to the Python binding.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libfp8blk.so")

SOURCES = ["quantize.hip", "dequant.hip", "merge.hip", "gemm.hip", "lora_bwd.hip", "nvfp4.hip", "abi.cpp"]

# -ffp-contract=off: every fused multiply-add in the kernels is written out
# explicitly, so rounding follows the source exactly.  Packed fp32 vector
# ops are disabled for all device code.
DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the fp8blk library needs ROCm's hipcc")


def build(verbose=False, save_temps=False):
    hipcc = _hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".", "_") + ".o")
        cmd = [hipcc, *DEVICE_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd.insert(1, "--save-temps")
        res = subprocess.run(cmd, cwd=bdir, capture_output=True, text=True)
        errs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                         if "is not a recognized feature for this target" not in ln)
        return src, obj, cmd, res.returncode, errs

    # the sources compile independently, so they go to hipcc side by side
    workers = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(compile_one, SOURCES))
    objs = []
    for src, obj, cmd, rc, errs in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if verbose and errs.strip():
            print(errs)
        objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))
