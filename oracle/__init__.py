"""CPU oracle for the weight-only NVFP4 fused MoE layer -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct numpy implementation of what the
GPU path computes.  It exists to check the HIP kernels; it is never a fallback.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library or its Python
binding and imports nothing from them.

Modules
  nvfp4  -- E2M1 / E4M3 codecs, the NVFP4 quantizer used to build test weights,
            dequantization, and the two global-scale conventions.
  mxfp4  -- E8M0 block scales per 32 elements: codec, quantizer, dequantization
            (the second weight format, section 6.4 of the Guide).
  moe    -- router, top-k, permutation, expert FFN, combine, whole-layer forward
            (float64 arithmetic on the exact values of the bf16/NVFP4 inputs).
  w4a4   -- the W4A4 variant: MXFP4 weights and MXFP4-quantized activations
            (x before gate/up, bf16-rounded h before down).
  brute  -- an independent scalar float64 per-token loop for tiny layers, used to
            pin ``moe`` and ``w4a4`` themselves.

Sources (the pages these follow):
  * "vLLM on the NVIDIA DGX Spark: A Complete Technical Guide", section 6.1
    (NVFP4 format) and section 7.1 (modular fused-MoE stages).
  * "Serving Solar Open 2 on DGX Spark", sections "Solar Open 2 in brief"
    (320 routed + 1 shared expert, top-8) and "Supporting real NVFP4 checkpoints"
    (E4M3 block scales clamped to 448; fused gate/up ordering).
  * "GLM-5.3-Flash-NVFP4 deployment blocked on SM121" (discussion), the
    compressed-tensors follow-up (weight recipe g16 / symmetric / E4M3 block
    scales; ModelOpt vs compressed-tensors global-scale reciprocal with a worked
    example) and the MoE fault analysis (a missing activation scale must never
    zero an expert).

Parity status: every function is pinned by a ``-m "not gpu"`` test against
closed forms, library routines (torch float8_e4m3fn), the worked example of the
discussion page, brute force or invariants.  The end-to-end layer output has no
printed value on the pages; it is pinned only through ``brute`` (an independent
scalar implementation of the same definition).
"""

from . import nvfp4, mxfp4, moe, w4a4, brute  # noqa: F401
