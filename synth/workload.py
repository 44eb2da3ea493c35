"""Full-size decode workloads built on the device.

Draws K, V and q with torch's generator on the GPU (the device recipe of
``synth``), lays out a seeded page permutation, and writes the cache through
the library's own quantize-on-write entry points. Used by the benchmark and
by the sampled full-size parity tests. No quantization arithmetic here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import Workload, device_generator, device_outlier_gain, device_values, page_layout


@dataclasses.dataclass
class DeviceWorkload:
    wl: Workload
    q: torch.Tensor                 # [B][Hq][d] bf16
    bt: torch.Tensor                # [B][pages_per_seq] int32
    sl: torch.Tensor                # [B] int32
    kp: object                      # NVFP4Pool
    vp: object
    num_pages: int
    k_bf16: Optional[torch.Tensor] = None   # [B][L][Hkv][d] when kept
    v_bf16: Optional[torch.Tensor] = None
    slots: Optional[torch.Tensor] = None    # [B*L] int64


def build_uniform_workload(nk, wl: Workload, keep_bf16: bool = False, fp8: bool = False,
                           batch: Optional[int] = None) -> DeviceWorkload:
    """Uniform-context workload with an NVFP4 (or FP8) cache filled by the library."""
    B = wl.batch if batch is None else batch
    L, H, d, P = wl.context, wl.num_kv_heads, wl.head_dim, wl.page_size
    gen = device_generator(wl.seed)
    gk = device_outlier_gain(gen, H, d) if wl.outliers else None
    gv = device_outlier_gain(gen, H, d) if wl.outliers else None
    bt_host = page_layout(B, L, P, wl.seed)
    pages_per_seq = bt_host.shape[1]
    num_pages = B * pages_per_seq
    bt = torch.from_numpy(bt_host).cuda()
    if fp8:
        kp = nk.FP8Pool.empty(num_pages, H, P, d)
        vp = nk.FP8Pool.empty(num_pages, H, P, d)
        quant = nk.fp8_kv_quantize
    else:
        kp = nk.NVFP4Pool.empty(num_pages, H, P, d)
        vp = nk.NVFP4Pool.empty(num_pages, H, P, d)
        quant = nk.nvfp4_kv_quantize
    t = torch.arange(L, device="cuda", dtype=torch.int64)
    keep_k, keep_v, keep_s = [], [], []
    for b in range(B):
        k = device_values(gen, (L, H, d), gk)
        v = device_values(gen, (L, H, d), gv)
        slots = bt[b, t // P].to(torch.int64) * P + t % P
        quant(k, v, slots, kp, vp)
        if keep_bf16:
            keep_k.append(k)
            keep_v.append(v)
            keep_s.append(slots)
    q = device_values(gen, (B, wl.num_q_heads, d))
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    w = DeviceWorkload(wl, q, bt, sl, kp, vp, num_pages)
    if keep_bf16:
        w.k_bf16 = torch.stack(keep_k)
        w.v_bf16 = torch.stack(keep_v)
        w.slots = torch.cat(keep_s)
    return w


@dataclasses.dataclass
class DeviceAgentic:
    """The prefix-reuse step at full size, resident on the device.

    Cached tokens [0, L_b) are already in the pool (the first
    ``shared_prefix`` tokens on pages every row references); the step writes
    the new chunk [L_b, L_b + chunk), dequantizes [0, L_b) into the
    workspace rows ws_row_offsets[b] .., and decodes at L_b + chunk.
    """
    wl: Workload
    kp: object
    vp: object
    num_pages: int
    bt: torch.Tensor            # [B][max_pages] int32
    cached_lens: torch.Tensor   # [B] int32 (L_b)
    seq_lens: torch.Tensor      # [B] int32 (L_b + chunk)
    k_chunk: torch.Tensor       # [B*chunk][Hkv][d] bf16
    v_chunk: torch.Tensor
    slot_chunk: torch.Tensor    # [B*chunk] int64
    ws_row_offsets: torch.Tensor  # [B+1] int64
    k_ws: torch.Tensor          # [rows][Hkv][d] bf16
    v_ws: torch.Tensor
    q: torch.Tensor             # [B][Hq][d] bf16
    shared_pages: np.ndarray
    host_cached_lens: np.ndarray
    host_bt: np.ndarray
    k_shared: Optional[torch.Tensor] = None   # kept bf16 inputs (for sampled parity)
    v_shared: Optional[torch.Tensor] = None
    k_private: Optional[list] = None
    v_private: Optional[list] = None


def build_agentic_workload(nk, wl: Workload, keep_bf16: bool = False) -> DeviceAgentic:
    """Agentic prefix-reuse workload at full size (lengths and pages from the
    host PCG64 generator, values from torch's generator on the device)."""
    B, H, d, P = wl.batch, wl.num_kv_heads, wl.head_dim, wl.page_size
    S, C = wl.shared_prefix, wl.chunk
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    cached = rng.integers(wl.len_min, wl.len_max, size=B, endpoint=True).astype(np.int32)
    total = cached.astype(np.int64) + C
    n_shared = S // P
    private = [-(-(int(total[b]) - S) // P) for b in range(B)]
    num_pages = n_shared + sum(private)
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = n_shared + max(private)
    bt = np.zeros((B, max_pages), dtype=np.int32)
    pos = n_shared
    for b in range(B):
        bt[b, :n_shared] = perm[:n_shared]
        bt[b, n_shared:n_shared + private[b]] = perm[pos:pos + private[b]]
        pos += private[b]
    bt_d = torch.from_numpy(bt).cuda()

    def slots(b, t0, t1):
        t = torch.arange(t0, t1, device="cuda", dtype=torch.int64)
        return bt_d[b, t // P].to(torch.int64) * P + t % P

    gen = device_generator(wl.seed)
    kp = nk.NVFP4Pool.empty(num_pages, H, P, d)
    vp = nk.NVFP4Pool.empty(num_pages, H, P, d)
    ks = device_values(gen, (S, H, d))
    vs = device_values(gen, (S, H, d))
    nk.nvfp4_kv_quantize(ks, vs, slots(0, 0, S), kp, vp)
    kpriv, vpriv = [], []
    for b in range(B):
        k = device_values(gen, (int(cached[b]) - S, H, d))
        v = device_values(gen, (int(cached[b]) - S, H, d))
        nk.nvfp4_kv_quantize(k, v, slots(b, S, int(cached[b])), kp, vp)
        if keep_bf16:
            kpriv.append(k)
            vpriv.append(v)
    kc = device_values(gen, (B * C, H, d))
    vc = device_values(gen, (B * C, H, d))
    sc = torch.cat([slots(b, int(cached[b]), int(total[b])) for b in range(B)])
    q = device_values(gen, (B, wl.num_q_heads, d))
    offs = np.zeros(B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(total)
    rows = int(offs[-1])
    kws = torch.empty((rows, H, d), dtype=torch.bfloat16, device="cuda")
    vws = torch.empty((rows, H, d), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    w = DeviceAgentic(wl, kp, vp, num_pages, bt_d, torch.from_numpy(cached).cuda(),
                      torch.from_numpy(total.astype(np.int32)).cuda(), kc, vc, sc,
                      torch.from_numpy(offs).cuda(), kws, vws, q, perm[:n_shared], cached, bt)
    if keep_bf16:
        w.k_shared, w.v_shared, w.k_private, w.v_private = ks, vs, kpriv, vpriv
    return w


def agentic_bytes(w: DeviceAgentic):
    """Logical and unique bytes of the three kernels of one agentic step."""
    wl = w.wl
    H, d, P = wl.num_kv_heads, wl.head_dim, wl.page_size
    per_tok = H * (d // 2 + d // 16)            # NVFP4 bytes per token, one of K or V
    B, C, S = wl.batch, wl.chunk, wl.shared_prefix
    cached = w.host_cached_lens.astype(np.int64)
    n_chunk = B * C
    quant_read = 2 * n_chunk * H * d * 2
    quant_write = 2 * n_chunk * per_tok
    dq_logical = 2 * int(cached.sum()) * per_tok
    dq_unique = 2 * (S + int((cached - S).sum())) * per_tok
    dq_write = 2 * int(cached.sum()) * H * d * 2
    dec_logical = 2 * int((cached + C).sum()) * per_tok
    dec_unique = 2 * (S + int((cached + C - S).sum())) * per_tok
    io = 2 * B * wl.num_q_heads * d * 2
    return dict(quant_read=quant_read, quant_write=quant_write, dequant_read_logical=dq_logical,
                dequant_read_unique=dq_unique, dequant_write=dq_write, decode_read_logical=dec_logical,
                decode_read_unique=dec_unique, decode_io=io)
