"""CPU oracle for the NVFP4 paged KV-cache path (TEST INFRASTRUCTURE ONLY).

Plain, slow, float64 numpy implementations of what the GPU library
computes, written from the pages:

  * "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache"
    (papercache summary of the LMSYS / SGLang / Qwen / NVIDIA blog,
    2026-09-16): section A3 (the NVFP4 format: E2M1 values, one FP8 E4M3
    scale per 16 values, one FP32 tensor scale), section A2 (the paged
    cache and its three attention paths; the decode kernel that unpacks
    E2M1 pairs in registers and applies the E4M3 block scale, Fig. 3; the
    storage-ratio equation (8 + 1) / 16).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never calls it and
shares no code, table or helper with it.

Modules:
  formats    E2M1 and E4M3 value sets from their bit layouts; round-to-
             nearest-even encoders.
  nvfp4      NVFP4 block encode / decode and the paged cache layout.
  fp8        FP8-E4M3 per-tensor-scaled KV cache (the comparison baseline).
  attention  float64 softmax decode attention over a paged cache, and the
             dequantize-to-workspace of the extend path.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, library cross-checks, brute force, invariants). Decode
output values have no printed example on the pages; they are pinned by the
reduction to torch's scaled_dot_product_attention on the dequantized cache
and by the closed-form special cases in that test file.
"""
from . import formats, nvfp4, fp8, attention  # noqa: F401
