"""Seeded synthetic inputs for the NVFP4 paged-KV decode path.

This module is shared by the oracle-side tests and the GPU-side tests and
benchmark. It holds input generation only: workload shapes, random K/V/q
values rounded to bf16, page permutations, block tables and slot mappings.
It contains none of the quantization or attention arithmetic.

Workload shapes follow the pages:
  * the synthetic long-context benchmark of "Accelerating Long-Context and
    Agentic Inference with NVFP4 KV Cache" (section A4, experimental setup:
    input lengths 32K and 1M, random inputs, prefix cache off) and its
    iso-concurrency / iso-capacity decode results (Figs. 6 and 7: batch 44
    at 32K, batch 2 at 1M);
  * the multi-turn prefix-reuse table of "Jetson edge agent 6.4x speed-up:
    NVFP4 quantization and KV reuse in practice" (section 2.2: a shared
    ~2,800-token prefix, ~500 new tokens per turn, totals 3,200-10,000).

Every value array is produced from a float32 normal draw, optionally with
outlier channels multiplied by 20, then rounded to bf16 (round to nearest
even). bf16 tensors are carried as uint16 bit patterns on the host.

Two generators exist. ``host_*`` functions use numpy's PCG64 and are used for
sizes the CPU oracle handles whole. ``device_*`` functions draw the same
distributions with torch's generator on the GPU for the full-size workloads
(gigabytes of K/V); their parity checks download sampled slices and give
those to the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BASE_SEED = 20260826  # the serving benchmark's fixed random seed (page A6 appendix)
OUTLIER_FRACTION = 0.02
OUTLIER_GAIN = 20.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload: shapes only."""

    index: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    context: int  # uniform context length (0 for the agentic workload)
    outliers: bool
    num_splits: int  # 0 = library heuristic
    # agentic prefix-reuse workload only
    len_min: int = 0
    len_max: int = 0
    shared_prefix: int = 0
    chunk: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    1: Workload(1, "tiny", 1, 4, 1, 64, 16, 256, False, 1),
    2: Workload(2, "moderate-batch", 8, 32, 8, 128, 16, 4096, True, 0),
    3: Workload(3, "long-context-32k", 44, 40, 8, 128, 64, 32768, True, 32),
    4: Workload(4, "extreme-context-1m", 2, 40, 8, 128, 64, 1048576, False, 256),
    5: Workload(5, "agentic-prefix-reuse", 64, 32, 8, 128, 16, 0, False, 0,
                len_min=3200, len_max=10000, shared_prefix=2800, chunk=500),
    # the third context length of the synthetic benchmark (section A3, 160K), N(0,1) values
    6: Workload(6, "long-context-160k", 10, 40, 8, 128, 64, 163840, False, 0),
}

# Decode batch sizes of the NVFP4 page's decode figures, per context length:
# iso-concurrency (Fig. 6: the same batch for both caches) and iso-capacity
# (Fig. 7: the batch each cache fits in the same memory).
ISO_CONCURRENCY = {"32k": (3, 44), "160k": (6, 10), "1m": (4, 1)}
ISO_CAPACITY = {"32k": (3, {"fp8": 44, "nvfp4": 70}), "160k": (6, {"fp8": 10, "nvfp4": 15}),
                "1m": (4, {"fp8": 1, "nvfp4": 2})}


# ---------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# host (numpy PCG64) generators
# ---------------------------------------------------------------------------

def outlier_mask(rng: np.random.Generator, num_kv_heads: int, head_dim: int) -> np.ndarray:
    """Per-(head, channel) gain: 2% of the pairs scaled by 20, the rest 1."""
    n = num_kv_heads * head_dim
    k = int(round(OUTLIER_FRACTION * n))
    gain = np.ones(n, dtype=np.float32)
    gain[rng.choice(n, size=k, replace=False)] = OUTLIER_GAIN
    return gain.reshape(num_kv_heads, head_dim)


def host_values(rng: np.random.Generator, shape, gain: Optional[np.ndarray] = None) -> np.ndarray:
    """float32 N(0,1) draw, optional per-(head, channel) gain, rounded to bf16 bits."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if gain is not None:
        x = x * gain
    return f32_to_bf16_bits(x)


@dataclasses.dataclass
class PagedInputs:
    """Host copy of one paged decode problem (all integer / bf16-bit arrays)."""

    wl: Workload
    num_pages: int
    k: np.ndarray            # uint16 [T][Hkv][d] bf16 bits, tokens in slot order below
    v: np.ndarray            # uint16 [T][Hkv][d]
    slot_mapping: np.ndarray  # int64 [T]: physical slot (page * P + offset) of token row i
    q: np.ndarray            # uint16 [B][Hq][d]
    block_tables: np.ndarray  # int32 [B][max_pages]
    seq_lens: np.ndarray     # int32 [B]
    max_pages: int


def host_uniform_decode(wl: Workload, context: Optional[int] = None,
                        batch: Optional[int] = None, seed: Optional[int] = None) -> PagedInputs:
    """Uniform-length decode problem: every sequence has ``context`` cached tokens.

    Draw order: outlier gains (K then V, if any), K, V, q, page permutation.
    Physical pages are a seeded permutation of all pages, assigned in
    (sequence, logical page) order.
    """
    L = wl.context if context is None else context
    B = wl.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    H, d, P = wl.num_kv_heads, wl.head_dim, wl.page_size
    gk = outlier_mask(rng, H, d) if wl.outliers else None
    gv = outlier_mask(rng, H, d) if wl.outliers else None
    T = B * L
    k = host_values(rng, (T, H, d), gk)
    v = host_values(rng, (T, H, d), gv)
    q = host_values(rng, (B, wl.num_q_heads, d))
    pages_per_seq = max(1, -(-L // P))
    num_pages = B * pages_per_seq
    perm = rng.permutation(num_pages).astype(np.int32)
    block_tables = perm.reshape(B, pages_per_seq)
    t = np.arange(L, dtype=np.int64)
    slots = []
    for b in range(B):
        slots.append(block_tables[b, t // P].astype(np.int64) * P + (t % P))
    slot_mapping = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    seq_lens = np.full(B, L, dtype=np.int32)
    return PagedInputs(wl, num_pages, k, v, slot_mapping, q, block_tables,
                       seq_lens, pages_per_seq)


@dataclasses.dataclass
class AgenticInputs:
    """Host copy of the prefix-reuse step (see ``host_agentic``)."""

    wl: Workload
    num_pages: int
    cached_lens: np.ndarray      # int32 [B]  L_b: tokens cached before the step
    seq_lens: np.ndarray         # int32 [B]  L_b + chunk: decode length after the step
    block_tables: np.ndarray     # int32 [B][max_pages]; first prefix/P pages shared
    max_pages: int
    shared_pages: np.ndarray     # int32 [prefix/P]
    # cached tokens: K/V rows and their slots (shared prefix once + private parts)
    k_cached: np.ndarray
    v_cached: np.ndarray
    slot_cached: np.ndarray
    # the step's new chunk: chunk tokens per sequence, concatenated
    k_chunk: np.ndarray
    v_chunk: np.ndarray
    slot_chunk: np.ndarray
    q: np.ndarray                # uint16 [B][Hq][d]
    ws_row_offsets: np.ndarray   # int64 [B+1]: workspace rows = prefix + chunk per sequence


def host_agentic(wl: Workload, batch: Optional[int] = None,
                 len_min: Optional[int] = None, len_max: Optional[int] = None,
                 shared_prefix: Optional[int] = None, chunk: Optional[int] = None,
                 seed: Optional[int] = None) -> AgenticInputs:
    """Prefix-reuse step with a ref-counted shared prefix.

    L_b ~ U[len_min, len_max] is the cached length before the step; the
    first ``shared_prefix`` tokens of every sequence live on the same
    physical pages. The step writes a new ``chunk``-token chunk at
    [L_b, L_b + chunk), dequantizes the prefix [0, L_b) into a workspace
    laid out per sequence as prefix rows then chunk rows, and decodes at
    length L_b + chunk. Draw order: lengths, shared K, shared V, private
    K/V per sequence, chunk K/V per sequence, q, page permutation.
    """
    B = wl.batch if batch is None else batch
    lo = wl.len_min if len_min is None else len_min
    hi = wl.len_max if len_max is None else len_max
    S = wl.shared_prefix if shared_prefix is None else shared_prefix
    C = wl.chunk if chunk is None else chunk
    H, d, P = wl.num_kv_heads, wl.head_dim, wl.page_size
    assert S % P == 0 and lo >= S
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    cached = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    total = cached.astype(np.int64) + C
    ks = host_values(rng, (S, H, d))
    vs = host_values(rng, (S, H, d))
    kp, vp, kc, vc = [], [], [], []
    for b in range(B):
        n = int(cached[b]) - S
        kp.append(host_values(rng, (n, H, d)))
        vp.append(host_values(rng, (n, H, d)))
    for b in range(B):
        kc.append(host_values(rng, (C, H, d)))
        vc.append(host_values(rng, (C, H, d)))
    q = host_values(rng, (B, wl.num_q_heads, d))
    n_shared = S // P
    private = [-(-(int(total[b]) - S) // P) for b in range(B)]
    num_pages = n_shared + sum(private)
    perm = rng.permutation(num_pages).astype(np.int32)
    shared_pages = perm[:n_shared]
    max_pages = n_shared + max(private)
    block_tables = np.zeros((B, max_pages), dtype=np.int32)
    pos = n_shared
    for b in range(B):
        block_tables[b, :n_shared] = shared_pages
        block_tables[b, n_shared:n_shared + private[b]] = perm[pos:pos + private[b]]
        pos += private[b]

    def slots_of(b, t0, t1):
        t = np.arange(t0, t1, dtype=np.int64)
        return block_tables[b, t // P].astype(np.int64) * P + (t % P)

    slot_cached = [slots_of(0, 0, S)] + [slots_of(b, S, int(cached[b])) for b in range(B)]
    slot_chunk = [slots_of(b, int(cached[b]), int(total[b])) for b in range(B)]
    offs = np.zeros(B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(total)
    return AgenticInputs(
        wl, num_pages, cached, total.astype(np.int32), block_tables, max_pages, shared_pages,
        np.concatenate([ks] + kp), np.concatenate([vs] + vp), np.concatenate(slot_cached),
        np.concatenate(kc), np.concatenate(vc), np.concatenate(slot_chunk), q, offs)


# ---------------------------------------------------------------------------
# device (torch generator) recipe for full-size workloads
# ---------------------------------------------------------------------------

def device_generator(seed: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_values(gen, shape, gain=None, device="cuda"):
    """float32 N(0,1) on the device, optional per-(head, channel) gain, rounded to bf16."""
    import torch
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if gain is not None:
        x.mul_(gain)
    return x.to(torch.bfloat16)


def device_outlier_gain(gen, num_kv_heads, head_dim, device="cuda"):
    import torch
    n = num_kv_heads * head_dim
    k = int(round(OUTLIER_FRACTION * n))
    idx = torch.randperm(n, generator=gen, device=device)[:k]
    gain = torch.ones(n, device=device, dtype=torch.float32)
    gain[idx] = OUTLIER_GAIN
    return gain.view(num_kv_heads, head_dim)


def page_layout(num_seqs: int, context: int, page_size: int, seed: int):
    """Seeded page permutation and block table for uniform contexts (host, int32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pages_per_seq = max(1, -(-context // page_size))
    perm = rng.permutation(num_seqs * pages_per_seq).astype(np.int32)
    return perm.reshape(num_seqs, pages_per_seq)


# ---------------------------------------------------------------------------
# host -> device plumbing (no arithmetic)
# ---------------------------------------------------------------------------

def to_device_bf16(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor (same bits)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_device(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_tensor_bits(t) -> np.ndarray:
    """torch bf16 tensor (any device) -> uint16 bit patterns on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
