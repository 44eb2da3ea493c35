"""FP8-E4M3 KV cache with a per-tensor FP32 scale (the comparison baseline).

Source: "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
sections A3 and A4 (the baseline is SGLang's fp8_e4m3 KV cache; only the KV
data type differs between the two arms).

Reading: byte = E4M3(fl32(x / s)) rounded to nearest even and saturated to
+-448, dequantized as e4m3 * s. fl32 is IEEE single-precision division; with
s = 1.0 (every workload here) it is exact. Cache layout:
[page][kv_head][slot][head_dim] uint8.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_VALUES, e4m3_encode
from .nvfp4 import bf16_to_f64


def quantize_rows(x_bits: np.ndarray, scale: float = 1.0) -> np.ndarray:
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    q = (x32 / np.float32(scale)).astype(np.float64)
    return e4m3_encode(q)


def write_cache(cache: np.ndarray, x_bits: np.ndarray, slot_mapping: np.ndarray,
                scale: float = 1.0) -> None:
    """Token row i goes to physical slot slot_mapping[i]; a slot below 0 or past
    the pool (>= pages * page_size) skips the token."""
    P = cache.shape[2]
    rows = quantize_rows(x_bits, scale)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    keep = (sm >= 0) & (sm < cache.shape[0] * P)
    cache[sm[keep] // P, :, sm[keep] % P, :] = rows[keep]


def dequant_cache(cache: np.ndarray, scale: float = 1.0) -> np.ndarray:
    return E4M3_VALUES[cache.astype(np.int64)] * scale
