"""NVFP4 encode / decode of K/V and the paged cache layout (float64 reference).

Source: "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache":
  * section A3: E2M1 values, one E4M3 block scale per 16 values, one FP32
    tensor-level scale (fixed to 1.0 in every experiment, section A7);
  * section A2, storage-ratio equation: 16 values take 8 bytes of packed
    data plus 1 scale byte, (8 + 1) / 16 = 0.5625 of an FP8 cache;
  * section A2, paths 1 and 2: new K/V are quantized and appended to the
    persistent paged NVFP4 pool.

Readings where the pages are silent (each listed in the design notes):
  * block scale S = E4M3(amax / (6 * gs)): the block maximum maps onto the
    largest E2M1 magnitude, 6; rounding to nearest even, saturating at 448;
  * each element is quantized as the nearest E2M1 value to |x| / (S * gs),
    ties to the even code, saturating at 6; S == 0 gives magnitude code 0;
  * the sign bit is kept (-0.0 and negatives that round to 0 give 0x8);
  * a block is 16 consecutive channels of one token's one-head vector;
  * element 2i goes to the low nibble of byte i;
  * paged layout: data  [page][kv_head][slot][head_dim / 2]  (uint8)
                  scale [page][kv_head][slot][head_dim / 16] (uint8, E4M3)
    slot = token position within the page; a token's physical slot number
    is page * page_size + slot.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_VALUES, E4M3_VALUES, e2m1_magnitude_code, e4m3_encode,
                      e4m3_encode_nonneg)

BLOCK = 16


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def encode_blocks(x: np.ndarray, gs: float = 1.0):
    """Encode blocks of 16 values.

    x: float64 [..., 16]. Returns (codes uint8 [..., 16] with sign in bit 3,
    scale bytes uint8 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == BLOCK
    amax = np.max(np.abs(x), axis=-1)
    s_byte = e4m3_encode_nonneg(amax / (6.0 * gs))
    s_eff = E4M3_VALUES[s_byte] * gs
    s_b = s_eff[..., None]
    safe = np.where(s_b > 0, s_b, 1.0)
    r = np.abs(x) / safe
    mag = np.where(s_b > 0, e2m1_magnitude_code(r.reshape(-1)).reshape(x.shape), 0)
    sign = np.signbit(x).astype(np.int64)
    codes = (sign << 3) | mag
    return codes.astype(np.uint8), s_byte


# E2M1 magnitude midpoints, and whether a value exactly on one rounds up
# (the upper neighbour has the even code: 0.75 -> 1, 1.75 -> 2, 3.5 -> 4)
MIDPOINTS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False))


def is_power_of_two(gs: float) -> bool:
    m, _ = np.frexp(np.float64(gs))
    return bool(gs > 0 and m == 0.5)


def encode_blocks_fp32(x: np.ndarray, gs: float):
    """Encode with a calibrated global scale, in FP32 arithmetic. The NVFP4
    page (section A3) fixes only that the tensor scale is FP32; where it
    leaves the arithmetic open, each step below is one FP32 operation:

      S     = E4M3(fl32(amax / fl32(6 * gs)))        nearest even, saturating
      S_eff = fl32(S * gs)
      code  = number of E2M1 midpoints m with |x| > fl32(m * S_eff), counting
              |x| == fl32(m * S_eff) as passing where a tie rounds up
              (S_eff == 0: code 0)

    For a power-of-two gs every product and quotient is exact and this is
    encode_blocks (pinned by the tests). x: float64 [..., 16] of bf16 values.
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == BLOCK
    a = np.abs(x).astype(np.float32)                     # exact: bf16 or FP32 values
    amax = np.fmax.reduce(a, axis=-1, initial=np.float32(0.0))   # NaN elements ignored
    g = np.float32(gs)
    s_byte = e4m3_encode_nonneg((amax / (np.float32(6.0) * g)).astype(np.float64))
    s_eff = (E4M3_VALUES[s_byte].astype(np.float32) * g)[..., None]
    mag = np.zeros(x.shape, dtype=np.int64)
    for m, tie_up in MIDPOINTS:
        t = np.float32(m) * s_eff
        mag += (a > t) | ((a == t) & tie_up)
    mag = np.where(s_eff > 0, mag, 0)
    sign = np.signbit(x).astype(np.int64)
    return ((sign << 3) | mag).astype(np.uint8), s_byte


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) of float32 values, rounded to nearest even (finite values)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def workspace_bits(data: np.ndarray, scale: np.ndarray, gs: float = 1.0) -> np.ndarray:
    """bf16 bits of dequantized values as a bf16 workspace holds them:
    bf16(fl32(e2m1 * fl32(S * gs))). For a power-of-two gs both roundings are
    exact (every E2M1 x E4M3 product is a bf16 value), so this is the exact value."""
    codes = unpack_nibbles(data)
    vals = E2M1_VALUES[codes.astype(np.int64)].astype(np.float32)
    s = E4M3_VALUES[np.asarray(scale, dtype=np.int64)].astype(np.float32) * np.float32(gs)
    d = vals.shape[-1]
    prod = vals.reshape(vals.shape[:-1] + (d // BLOCK, BLOCK)) * s[..., None]
    return f32_to_bf16_rne(prod.reshape(vals.shape))


def quantize_rows_fp8(x_bytes: np.ndarray, src_scale: float = 1.0, gs: float = 1.0):
    """Quantize FP8-E4M3 token rows [T][H][d] (bytes) to NVFP4 (the pages' source
    type, section A2 paths 1-2): element value fl32(e4m3 * src_scale), then the
    FP32 recipe (for src_scale = 1 and a power-of-two gs every step is exact)."""
    x = (E4M3_VALUES[np.asarray(x_bytes, dtype=np.int64)].astype(np.float32) * np.float32(src_scale))
    T, H, d = x.shape
    codes, s = encode_blocks_fp32(x.astype(np.float64).reshape(T, H, d // BLOCK, BLOCK), gs)
    return pack_nibbles(codes.reshape(T, H, d)), s.reshape(T, H, d // BLOCK)


def workspace_fp8_bytes(data: np.ndarray, scale: np.ndarray, gs: float = 1.0, ws_scale: float = 1.0) -> np.ndarray:
    """E4M3 bytes of dequantized values in the pages' FP8 workspace (section A2,
    path 2): E4M3(fl32(fl32(e2m1 * fl32(S * gs)) / ws_scale)), nearest even,
    saturating at +-448, sign kept. Lossy: some products are not E4M3 values."""
    codes = unpack_nibbles(data)
    vals = E2M1_VALUES[codes.astype(np.int64)].astype(np.float32)
    s = E4M3_VALUES[np.asarray(scale, dtype=np.int64)].astype(np.float32) * np.float32(gs)
    d = vals.shape[-1]
    prod = (vals.reshape(vals.shape[:-1] + (d // BLOCK, BLOCK)) * s[..., None]).reshape(vals.shape)
    return e4m3_encode((prod / np.float32(ws_scale)).astype(np.float64))


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit codes -> [..., n] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(data: np.ndarray) -> np.ndarray:
    d = np.asarray(data, dtype=np.uint8)
    out = np.empty(d.shape[:-1] + (2 * d.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = d & 0xF
    out[..., 1::2] = d >> 4
    return out


def quantize_rows(x_bits: np.ndarray, gs: float = 1.0):
    """Quantize token rows [T][H][d] (bf16 bits) to (data [T][H][d/2], scale [T][H][d/16]).
    Power-of-two gs: the real-number encode; any other gs: its FP32 recipe."""
    x = bf16_to_f64(x_bits)
    T, H, d = x.shape
    assert d % BLOCK == 0
    enc = encode_blocks if is_power_of_two(gs) else encode_blocks_fp32
    codes, s = enc(x.reshape(T, H, d // BLOCK, BLOCK), gs)
    data = pack_nibbles(codes.reshape(T, H, d))
    return data, s.reshape(T, H, d // BLOCK)


def dequant_rows(data: np.ndarray, scale: np.ndarray, gs: float = 1.0) -> np.ndarray:
    """data [..., d/2], scale [..., d/16] -> float64 [..., d] = e2m1 * S * gs."""
    codes = unpack_nibbles(data)
    vals = E2M1_VALUES[codes.astype(np.int64)]
    s = E4M3_VALUES[np.asarray(scale, dtype=np.int64)] * gs
    d = vals.shape[-1]
    vals = vals.reshape(vals.shape[:-1] + (d // BLOCK, BLOCK)) * s[..., None]
    return vals.reshape(vals.shape[:-2] + (d,))


def empty_cache(num_pages: int, num_kv_heads: int, page_size: int, head_dim: int, fill: int = 0):
    data = np.full((num_pages, num_kv_heads, page_size, head_dim // 2), fill, dtype=np.uint8)
    scale = np.full((num_pages, num_kv_heads, page_size, head_dim // BLOCK), fill, dtype=np.uint8)
    return data, scale


def write_cache(data: np.ndarray, scale: np.ndarray, x_bits: np.ndarray,
                slot_mapping: np.ndarray, gs: float = 1.0) -> None:
    """Quantize-on-write: token row i goes to physical slot slot_mapping[i]; a slot
    below 0 or past the pool (>= pages * page_size) skips the token."""
    P = data.shape[2]
    rd, rs = quantize_rows(x_bits, gs)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    keep = (sm >= 0) & (sm < data.shape[0] * P)
    page, off = sm[keep] // P, sm[keep] % P
    data[page, :, off, :] = rd[keep]
    scale[page, :, off, :] = rs[keep]


def dequant_cache(data: np.ndarray, scale: np.ndarray, gs: float = 1.0) -> np.ndarray:
    """Whole paged cache -> float64 [page][kv_head][slot][head_dim]."""
    return dequant_rows(data, scale, gs)


def storage_bytes(num_tokens: int, num_kv_heads: int, head_dim: int) -> int:
    """Bytes of packed data plus block scales for one of K or V."""
    return num_tokens * num_kv_heads * (head_dim // 2 + head_dim // BLOCK)
