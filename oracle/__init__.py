"""Plain CPU oracle for block-scaled FP8 quantization and block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, no
headers, no tables, no helpers) and is written for a reader checking it
against the pages by eye, not for speed: numpy for vectorised element work,
exact integer / Fraction arithmetic where a rounding decision is defined,
and a library fp32 matmul as the GEMM step.

Pages (titles as they appear in the source text):
  [Fireworks-QAT]  "DeepSeek R1 and V3 get quantization-aware fine-tuning on
                   Fireworks ..." (news item), sections Synopsis, Interpretation.
  [DSV3-Blog5]     "DeepSeek-V3 Blog 5: Low-Precision Training - The FP8
                   Revolution in Large-Scale AI", sections "The Solution:
                   Block-Wise Quantization", "Hardware Optimization".
  [FP8-DSV3-ru]    "FP8 в DeepSeek V3: как низкая точность ускоряет обучение и
                   инференс", sections "Как FP8 встроен в DeepSeek V3",
                   "Почему обычное округление не подходит",
                   "Почему FP8 требует scale factors".
  [prequant]       "fireworks-prequant 0.1.0" (PyPI page), sections
                   "Quick start", "Formats".

Numeric facts the pages only name (the e4m3fn layout, E8M0, the E2M1 FP4
element) come from the public OCP 8-bit floating point and Microscaling (MX)
specifications.

Modules
  codec   e4m3fn / E8M0 / bf16 encode and decode
  quant   block amax, scale rules, quantize, dequantize (fake-quant output)
  merge   LoRA merge W + B.A in bf16 followed by 128x128 fake-quant
  gemm    block-scaled GEMM and grouped GEMM references, error metric
  lora_grad  QAT backward for the LoRA factors (straight-through fake-quant)
  nvfp4   NVFP4 prequant: E2M1 codes, e4m3 1x16 block scales, per-tensor fp32 scale

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, torch's own dtype casts or exact
rational arithmetic; none is "parity unpinned".
"""

from . import codec, quant, merge, gemm, lora_grad, nvfp4  # noqa: F401
