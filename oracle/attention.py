"""Decode attention over a paged KV cache, and the extend-path workspace (float64).

Source: "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
section A2:
  * path 3 (decode): the kernel reads the packed cache, dequantizes it
    on the fly and runs attention of one BF16 query per head over the
    whole cached context; the tensor-level K/V scales act as scaling
    parameters of the two attention products;
  * path 2 (chunked prefill / extend): the cached prefix is gathered from
    the paged pool, dequantized and written into a workspace that the
    extend attention then reads together with the current chunk.

This is the plain definition: softmax(sm_scale * q . k_t) over the
dequantized tokens t < seq_len, then the weighted sum of dequantized v_t.
Splitting the context and merging partial results by log-sum-exp (what the
GPU does) reaches the same value algebraically, so the oracle never splits.

Readings: query head h uses KV head h // (Hq / Hkv); sm_scale = 1/sqrt(d) in
every workload; a sequence of length 0 gives an all-zero output.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import bf16_to_f64


def gather_tokens(cache_hat: np.ndarray, block_table: np.ndarray, length: int) -> np.ndarray:
    """Logical tokens [0, length) of one sequence -> float64 [length][Hkv][d]."""
    P = cache_hat.shape[2]
    t = np.arange(length, dtype=np.int64)
    pages = np.asarray(block_table, dtype=np.int64)[t // P]
    return cache_hat[pages, :, t % P, :]


def decode_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Attention of query heads q [Hq][d] over tokens k, v [L][Hkv][d] (float64).

    Returns (out [Hq][d], mass [Hq][d]) where mass = sum_t p_t |v_t| is the
    natural magnitude of each output element (used to normalise errors).
    """
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    if L == 0:
        z = np.zeros((Hq, d))
        return z, z.copy()
    G = Hq // Hkv
    qg = q.reshape(Hkv, G, d)
    kt = np.transpose(k, (1, 0, 2))                      # [Hkv][L][d]
    vt = np.transpose(v, (1, 0, 2))
    logits = np.einsum("hgd,htd->hgt", qg, kt) * sm_scale
    m = logits.max(axis=-1, keepdims=True)
    w = np.exp(logits - m)
    denom = w.sum(axis=-1, keepdims=True)
    p = w / denom
    out = np.einsum("hgt,htd->hgd", p, vt)
    mass = np.einsum("hgt,htd->hgd", p, np.abs(vt))
    return out.reshape(Hq, d), mass.reshape(Hq, d)


def paged_decode(q_bits: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                 block_tables: np.ndarray, seq_lens: np.ndarray, sm_scale: float):
    """Decode attention for a batch.

    q_bits: bf16 bits [B][Hq][d]; k_hat, v_hat: dequantized caches
    [page][Hkv][slot][d] float64. Returns (out, mass), each [B][Hq][d].
    """
    q = bf16_to_f64(q_bits)
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    mass = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        k = gather_tokens(k_hat, block_tables[b], L)
        v = gather_tokens(v_hat, block_tables[b], L)
        out[b], mass[b] = decode_heads(q[b], k, v, sm_scale)
    return out, mass


def f64_to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """bf16 bits of values that bf16 represents exactly (asserted, never rounded)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x), "value not exact in float32"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def dequant_workspace(cache_hat: np.ndarray, block_tables: np.ndarray,
                      prefix_lens: np.ndarray, ws_row_offsets: np.ndarray,
                      rows: int, fill: int = 0, cache_bits: np.ndarray = None) -> np.ndarray:
    """Extend-path workspace: rows [off_b, off_b + prefix_len_b) hold the
    dequantized tokens [0, prefix_len_b) of sequence b as bf16 bits
    [rows][Hkv][d]; other rows keep ``fill``. The values are cache_hat
    (exact in bf16), or, when given, the bf16 bits ``cache_bits`` of every
    cache element (a calibrated global scale rounds them)."""
    _, Hkv, _, d = cache_hat.shape
    ws = np.full((rows, Hkv, d), fill, dtype=np.uint16)
    for b in range(len(prefix_lens)):
        n = int(prefix_lens[b])
        off = int(ws_row_offsets[b])
        if cache_bits is None:
            ws[off:off + n] = f64_to_bf16_exact(gather_tokens(cache_hat, block_tables[b], n))
        else:
            ws[off:off + n] = gather_tokens(cache_bits, block_tables[b], n)
    return ws


def extend_attention(q: np.ndarray, k_ws: np.ndarray, v_ws: np.ndarray, q_row_offsets: np.ndarray,
                     ws_row_offsets: np.ndarray, prefix_lens: np.ndarray, sm_scale: float):
    """Extend (chunked-prefill) attention, "Accelerating Long-Context and Agentic
    Inference with NVFP4 KV Cache" section A2 path 2: the chunk's queries
    attend to the cached prefix and causally to the chunk. Query i of sequence
    b (q row q_row_offsets[b] + i) sits at position prefix_lens[b] + i and sees
    workspace rows ws_row_offsets[b] + j for j <= prefix_lens[b] + i.

    q [rows][Hq][d], k_ws / v_ws [rows][Hkv][d] (float64). Returns (out, mass)
    shaped like q: the plain softmax attention per query and the tolerance
    weight sum_t p_t |v_t| (decode_heads per query)."""
    out = np.zeros(q.shape, dtype=np.float64)
    mass = np.zeros(q.shape, dtype=np.float64)
    for b in range(len(prefix_lens)):
        L, w0 = int(prefix_lens[b]), int(ws_row_offsets[b])
        for r in range(int(q_row_offsets[b]), int(q_row_offsets[b + 1])):
            i = r - int(q_row_offsets[b])
            keys = slice(w0, w0 + L + i + 1)
            out[r], mass[r] = decode_heads(q[r], k_ws[keys], v_ws[keys], sm_scale)
    return out, mass
