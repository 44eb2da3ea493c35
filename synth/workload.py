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
