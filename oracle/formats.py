"""E2M1 and E4M3 number formats, written out from their bit layouts.

Source: "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
section A3 (NVFP4 stores 4-bit E2M1 values with one FP8 E4M3 scale per block
of 16 values and one FP32 tensor scale). The pages name the formats only; the
layouts used here are the standard ones those names denote:

  E2M1  1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field
        0 is subnormal (value = mantissa * 0.5). No Inf, no NaN.
        Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  E4M3  (OCP "E4M3FN") 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
        bits; exponent field 0 is subnormal (value = mantissa * 2^-9);
        S.1111.111 is NaN; no Inf. Largest finite 448, smallest 2^-9.

Rounding (a reading of the pages, which do not state it): round to nearest,
ties to the even code; values beyond the largest finite magnitude saturate
to it.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# value tables from the bit layouts
# ---------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (sign bit 3, exponent bits 2..1, mantissa bit 0)."""
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = man * 0.5
    else:
        mag = math.ldexp(1.0 + man * 0.5, exp - 1)
    return -mag if sign else mag


def e4m3_value(byte: int) -> float:
    """Value of an OCP E4M3FN byte."""
    sign = (byte >> 7) & 1
    exp = (byte >> 3) & 0xF
    man = byte & 7
    if exp == 0xF and man == 7:
        return math.nan
    if exp == 0:
        mag = math.ldexp(man, -9)
    else:
        mag = math.ldexp(1.0 + man / 8.0, exp - 7)
    return -mag if sign else mag


E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_VALUES = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)

# non-negative finite grids, indexed by code (both are increasing in the code)
_E2M1_GRID = E2M1_VALUES[:8]
_E4M3_GRID = E4M3_VALUES[:127]          # bytes 0x00 .. 0x7E
E4M3_MAX = float(_E4M3_GRID[-1])        # 448
E2M1_MAX = float(_E2M1_GRID[-1])        # 6


def _rne_on_grid(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value to each x >= 0; ties go to the even index.

    ``grid`` is increasing and starts at 0. Values above the last grid value
    map to the last index (saturation).
    """
    x = np.asarray(x, dtype=np.float64)
    assert not np.any(np.isnan(x)), "NaN has no code in this encoder"
    assert np.all(x >= 0)
    hi = np.searchsorted(grid, x, side="left")          # grid[hi-1] < x <= grid[hi]
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = x - grid[lo]
    d_hi = grid[hi] - x
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(x >= grid[-1], len(grid) - 1, idx)    # saturate
    idx = np.where(x == 0, 0, idx)
    return idx.astype(np.int64)


def e2m1_magnitude_code(r: np.ndarray) -> np.ndarray:
    """Magnitude code 0..7 of r = |x| / scale: nearest E2M1 value, ties to even, saturate at 6."""
    return _rne_on_grid(r, _E2M1_GRID)


def e4m3_encode_nonneg(x: np.ndarray) -> np.ndarray:
    """E4M3 byte (0x00..0x7E) of x >= 0: nearest finite value, ties to even, saturate at 448."""
    return _rne_on_grid(x, _E4M3_GRID).astype(np.uint8)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Signed E4M3 byte with saturation to +-448 (the sign of zero is kept)."""
    x = np.asarray(x, dtype=np.float64)
    mag = e4m3_encode_nonneg(np.abs(x))
    sign = np.signbit(x).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(b, dtype=np.int64)]


def e2m1_decode(nib: np.ndarray) -> np.ndarray:
    return E2M1_VALUES[np.asarray(nib, dtype=np.int64)]
