#!/usr/bin/env python3
"""Benchmark of the NVFP4 paged decode path on one MI355X.

Workload (default): batch 44, 40 query / 8 KV heads, head_dim 128, context
32,768, page 64, 32 splits, K/V ~ N(0,1) bf16 with 2% of channels x20 --
the iso-concurrency long-context point of "Accelerating Long-Context and
Agentic Inference with NVFP4 KV Cache" (section A4, Fig. 6), with the same
layer also run over an FP8-E4M3 cache.

One step = quantize-on-write of the step's new token of every sequence into
the NVFP4 pool (it overwrites the last slot, so the shape stays fixed) +
split-KV decode partials + log-sum-exp merge. Inputs are resident in HBM
before timing. Prints ONE JSON line on stdout; diagnostics go to stderr.

  value           KV GB/s of the step: (packed + scale bytes) / step time
  roofline        dominant kernel (decode partial): algorithmic bytes per
                  launch / mean launch time (HIP events on the launch stream);
                  also as a fraction of the measured read bandwidth
  hbm_read_probe  read bandwidth of the library's plain streaming-read kernel
                  over 4 GiB (best of a few launch shapes)
  cpu_baseline    the CPU oracle (dequantize + fp64 attention) on a bounded
                  sample of (sequence, KV head) slices of the same workload
  fp8, extreme_context_1m, agentic_prefix_reuse
                  the same step over the FP8 pool, the 1M batch-2 step, and
                  the agentic prefix-reuse step with per-kernel times
  decode_figures  decode tokens/s of NVFP4 and FP8 at the batch sizes of the
                  page's decode figures (Fig. 6 iso-concurrency: 44 / 10 / 1
                  at 32K / 160K / 1M; Fig. 7 iso-capacity: NVFP4 70 / 15 / 2
                  against FP8 44 / 10 / 1)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "NVFP4 paged decode attn: KV GB/s + % HBM roofline; steps/s vs FP8-KV kernel"
DECODE_SOURCES = ["nvfp4_quantized_paged_amd/csrc/decode_mfma.hip",
                  "nvfp4_quantized_paged_amd/csrc/common.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes(wl, fp8=False):
    per = wl.head_dim if fp8 else wl.head_dim // 2 + wl.head_dim // 16
    return 2 * wl.batch * wl.context * wl.num_kv_heads * per


def io_bytes(wl):
    return 2 * wl.batch * wl.num_q_heads * wl.head_dim * 2      # q read + out written (bf16)


def partial_bytes(wl, splits):
    return wl.batch * wl.num_q_heads * splits * (wl.head_dim + 2) * 4


def source_digest():
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current decode kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


RAMP_S = 0.5


def ramp(fn, seconds=RAMP_S):
    """Untimed calls for `seconds` of wall time before the counted warm-up:
    the first few hundred microseconds of a burst run measurably slower
    (clocks and caches coming up), which a handful of sub-millisecond warm-up
    steps does not cover."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


class Bench:
    def __init__(self, nk, wl, fp8, variant, batch=None):
        import torch
        from synth.workload import build_uniform_workload
        self.torch = torch
        self.nk, self.wl, self.fp8, self.variant = nk, wl, fp8, variant
        self.batch = B = wl.batch if batch is None else batch
        t = time.time()
        self.w = build_uniform_workload(nk, wl, fp8=fp8, batch=B)
        log(f"[bench] built {'fp8' if fp8 else 'nvfp4'} {wl.name} batch {B} in {time.time() - t:.1f}s")
        H, d, P, L = wl.num_kv_heads, wl.head_dim, wl.page_size, wl.context
        g = torch.Generator(device="cuda")
        g.manual_seed(wl.seed + 1000)
        self.k_new = torch.randn((B, H, d), generator=g, device="cuda").to(torch.bfloat16)
        self.v_new = torch.randn((B, H, d), generator=g, device="cuda").to(torch.bfloat16)
        last = L - 1
        self.slots_new = (self.w.bt[:, last // P].to(torch.int64) * P + last % P).contiguous()
        self.S = wl.num_splits or nk.nvfp4_paged_decode_num_splits(B, H, self.w.bt.shape[1], P)
        self.ws = nk.decode_workspace(B, wl.num_q_heads, d, self.S)
        self.out = torch.empty_like(self.w.q)

    def quantize(self):
        f = self.nk.fp8_kv_quantize if self.fp8 else self.nk.nvfp4_kv_quantize
        f(self.k_new, self.v_new, self.slots_new, self.w.kp, self.w.vp)

    def partial(self):
        f = self.nk.fp8_paged_decode_partial if self.fp8 else self.nk.nvfp4_paged_decode_partial
        f(self.w.q, self.w.kp, self.w.vp, self.w.bt, self.w.sl, self.wl.sm_scale, self.S,
          variant=self.variant, workspace=self.ws)

    def merge(self):
        scale = self.w.vp.scale if self.fp8 else self.w.vp.global_scale
        self.nk.nvfp4kv_lse_merge(self.ws, self.batch, self.wl.num_q_heads, self.wl.head_dim, self.S,
                                  scale, self.out)

    def step(self):
        self.quantize()
        self.partial()
        self.merge()

    def time_steps(self, steps, warmup):
        torch = self.torch
        ramp(self.step)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def time_partial(self, launches):
        """Mean duration of the decode-partial kernel, HIP events on its stream."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        self.partial()
        for a, b in ev:
            a.record(stream)
            self.partial()
            b.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        return sum(ms) / len(ms) / 1e3, min(ms) / 1e3

    def free(self):
        del self.w, self.ws, self.out
        self.torch.cuda.empty_cache()


def decode_figures(nk, variant, steps, warmup, measured):
    """Kernel-level decode throughput at the batch sizes of the NVFP4 page's
    decode figures: iso-concurrency (Fig. 6, both caches at the same batch)
    and iso-capacity (Fig. 7, each cache at the batch it fits in the same
    memory), at 32K, 160K and 1M context. One step = quantize the new token
    + decode partial + merge; decode tokens/s = batch / step time. Steps
    already timed by the main benchmark are reused from `measured`."""
    import synth

    def run(idx, batch, fp8):
        key = (idx, batch, fp8)
        if key not in measured:
            b = Bench(nk, synth.WORKLOADS[idx], fp8, variant, batch=batch)
            measured[key] = (b.time_steps(steps, warmup), b.S)
            b.free()
        t, S = measured[key]
        wl = synth.WORKLOADS[idx]
        kv = 2 * batch * wl.context * wl.num_kv_heads * (wl.head_dim if fp8 else wl.head_dim // 2 + wl.head_dim // 16)
        return {"batch": batch, "num_splits": S, "ms_per_step": round(t * 1e3, 4),
                "decode_tokens_per_s": round(batch / t, 1), "kv_gbs": round(kv / t / 1e9, 1)}
    out = {"iso_concurrency": {}, "iso_capacity": {}}
    for name, (idx, batch) in synth.ISO_CONCURRENCY.items():
        nv, f8 = run(idx, batch, False), run(idx, batch, True)
        out["iso_concurrency"][name] = {"nvfp4": nv, "fp8": f8,
                                        "nvfp4_over_fp8": round(nv["decode_tokens_per_s"] / f8["decode_tokens_per_s"], 3)}
    for name, (idx, batches) in synth.ISO_CAPACITY.items():
        nv, f8 = run(idx, batches["nvfp4"], False), run(idx, batches["fp8"], True)
        out["iso_capacity"][name] = {"nvfp4": nv, "fp8": f8,
                                     "nvfp4_over_fp8": round(nv["decode_tokens_per_s"] / f8["decode_tokens_per_s"], 3)}
    log("[bench] decode figures: " + ", ".join(
        f"{k} {n} x{v['nvfp4_over_fp8']}" for k in out for n, v in out[k].items()))
    return out


def time_calls(calls, steps, warmup):
    """Whole-sequence time of `calls` per step (wall clock, synchronised) and each
    call's mean duration from HIP events on the launch stream."""
    import torch
    ramp(lambda: [f() for _, f in calls], seconds=0.2)
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    stream = torch.cuda.current_stream()
    per = {}
    for name, f in calls:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            f()
            b.record(stream)
        torch.cuda.synchronize()
        per[name] = sum(a.elapsed_time(b) for a, b in ev) / steps / 1e3
    return t_step, per


def agentic(nk, wl, steps, warmup):
    """The prefix-reuse step (quantize the new chunk, dequantize every cached
    prefix into the workspace, decode all sequences): whole-step time and
    each kernel's mean duration from HIP events on the launch stream. Run
    twice: with bf16 chunk and workspace (the workload definition) and with
    the pages' FP8 types (FP8 chunk quantized to NVFP4 and copied into an FP8
    workspace in one pass, FP8 workspace)."""
    import numpy as np
    import torch
    from synth.workload import agentic_bytes, build_agentic_workload
    t = time.time()
    w = build_agentic_workload(nk, wl)
    log(f"[bench] built agentic workload in {time.time() - t:.1f}s")
    B, Hq, d, H, C = wl.batch, wl.num_q_heads, wl.head_dim, wl.num_kv_heads, wl.chunk
    S = nk.nvfp4_paged_decode_num_splits(B, H, w.bt.shape[1], wl.page_size)
    ws = nk.decode_workspace(B, Hq, d, S)
    out = torch.empty_like(w.q)
    decode = ("decode", lambda: nk.nvfp4_paged_decode_attn(w.q, w.kp, w.vp, w.bt, w.seq_lens, wl.sm_scale,
                                                           num_splits=S, workspace=ws, out=out))
    calls = [
        ("quantize", lambda: nk.nvfp4_kv_quantize(w.k_chunk, w.v_chunk, w.slot_chunk, w.kp, w.vp)),
        ("dequant_workspace", lambda: nk.nvfp4_kv_dequant_workspace(w.kp, w.vp, w.bt, w.cached_lens,
                                                                    w.ws_row_offsets, w.k_ws, w.v_ws)),
        decode,
    ]
    t_step, per = time_calls(calls, steps, warmup)
    by = agentic_bytes(w)
    res = {
        "ms_per_step": round(t_step * 1e3, 4), "steps_per_s": round(1.0 / t_step, 2), "num_splits": S,
        "quantize": {"ms": round(per["quantize"] * 1e3, 4),
                     "gbs": round((by["quant_read"] + by["quant_write"]) / per["quantize"] / 1e9, 1)},
        "dequant_workspace": {"ms": round(per["dequant_workspace"] * 1e3, 4),
                              "gbs_unique": round((by["dequant_read_unique"] + by["dequant_write"])
                                                  / per["dequant_workspace"] / 1e9, 1),
                              "write_gbs": round(by["dequant_write"] / per["dequant_workspace"] / 1e9, 1)},
        "decode": {"ms": round(per["decode"] * 1e3, 4),
                   "kv_gbs_logical": round(by["decode_read_logical"] / per["decode"] / 1e9, 1),
                   "kv_gbs_unique": round(by["decode_read_unique"] / per["decode"] / 1e9, 1)},
        "bytes": by,
    }
    log(f"[bench] agentic step {t_step * 1e3:.3f} ms: " + ", ".join(f"{k} {v * 1e3:.3f} ms" for k, v in per.items()))

    # the pages' path-2 types: FP8 chunk and FP8 workspace
    k8 = w.k_chunk.to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = w.v_chunk.to(torch.float8_e4m3fn).view(torch.uint8)
    rows = int(w.ws_row_offsets[-1].item())
    kws8 = torch.empty((rows, H, d), dtype=torch.uint8, device="cuda")
    vws8 = torch.empty((rows, H, d), dtype=torch.uint8, device="cuda")
    offs = w.ws_row_offsets.cpu().numpy()
    chunk_rows = np.concatenate([offs[b] + w.host_cached_lens[b] + np.arange(C) for b in range(B)]).astype(np.int64)
    ws_rows = torch.from_numpy(chunk_rows).cuda()
    calls8 = [
        ("quantize", lambda: nk.nvfp4_kv_quantize_fp8(k8, v8, w.slot_chunk, w.kp, w.vp, 1.0, 1.0, ws_rows, kws8, vws8)),
        ("dequant_workspace", lambda: nk.nvfp4_kv_dequant_workspace_fp8(w.kp, w.vp, w.bt, w.cached_lens,
                                                                        w.ws_row_offsets, kws8, vws8)),
        decode,
    ]
    t8, per8 = time_calls(calls8, steps, warmup)
    q_rd = by["quant_read"] // 2                        # FP8 chunk: one byte per element
    q_wr = by["quant_write"] + q_rd                     # NVFP4 + the chunk copied into the workspace
    dq_wr = by["dequant_write"] // 2
    res["fp8_path2"] = {
        "ms_per_step": round(t8 * 1e3, 4), "steps_per_s": round(1.0 / t8, 2),
        "quantize_with_chunk_copy": {"ms": round(per8["quantize"] * 1e3, 4),
                                     "gbs": round((q_rd + q_wr) / per8["quantize"] / 1e9, 1)},
        "dequant_workspace_fp8": {"ms": round(per8["dequant_workspace"] * 1e3, 4),
                                  "gbs_unique": round((by["dequant_read_unique"] + dq_wr)
                                                      / per8["dequant_workspace"] / 1e9, 1),
                                  "write_gbs": round(dq_wr / per8["dequant_workspace"] / 1e9, 1)},
        "decode": {"ms": round(per8["decode"] * 1e3, 4)},
    }
    log(f"[bench] agentic fp8 path-2 step {t8 * 1e3:.3f} ms: "
        + ", ".join(f"{k} {v * 1e3:.3f} ms" for k, v in per8.items()))

    # extend attention of the chunk over the bf16 workspace (path 2's consumer), not part of the step:
    # the chunk's K/V go to the workspace rows after each prefix, then its queries attend causally
    crow = torch.from_numpy(np.concatenate([offs[b] + w.host_cached_lens[b] + np.arange(C)
                                            for b in range(B)]).astype(np.int64)).cuda()
    w.k_ws[crow] = w.k_chunk
    w.v_ws[crow] = w.v_chunk
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 2000)
    qx = torch.randn((B * C, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    q_offs = torch.arange(0, B * C + 1, C, dtype=torch.int64, device="cuda")
    ox = torch.empty_like(qx)
    ext = lambda: nk.nvfp4_extend_attn(qx, q_offs, w.k_ws, w.v_ws, w.ws_row_offsets, w.cached_lens, wl.sm_scale,
                                       max_chunk=C, out=ox)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        ext()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        ext()
    e1.record(stream)
    torch.cuda.synchronize()
    t_ext = e0.elapsed_time(e1) / steps / 1e3
    Lc = w.host_cached_lens.astype(np.float64)
    flops = 4.0 * d * Hq * float(np.sum(C * Lc + C * (C + 1) / 2.0))
    res["extend_attention"] = {"ms": round(t_ext * 1e3, 4), "tflops": round(flops / t_ext / 1e12, 1),
                               "bf16_mfma_peak_frac": round(flops / t_ext / 2.5e15, 4), "flops": flops}
    log(f"[bench] extend attention {t_ext * 1e3:.3f} ms, {flops / t_ext / 1e12:.1f} TFLOP/s")

    # global-scale calibration of the chunk (absmax of K and V), not part of the step
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    cal = lambda: (nk.nvfp4_kv_absmax(w.k_chunk, amax[0:1]), nk.nvfp4_kv_absmax(w.v_chunk, amax[1:2]))
    for _ in range(warmup):
        cal()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        cal()
    e1.record(stream)
    torch.cuda.synchronize()
    t_cal = e0.elapsed_time(e1) / steps / 1e3
    res["absmax_calibration"] = {"ms": round(t_cal * 1e3, 4), "gbs": round(by["quant_read"] / t_cal / 1e9, 1)}
    log(f"[bench] absmax calibration {t_cal * 1e3:.3f} ms")
    del w, ws, out, kws8, vws8, qx, ox
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, budget_s=12.0):
    """The oracle (dequantize + fp64 attention) on (sequence, KV head) slices of
    the workload, single-threaded, until ~budget_s of work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import attention as oatt
    from oracle import nvfp4 as onv

    rng = np.random.Generator(np.random.PCG64(wl.seed))
    gain_k = synth.outlier_mask(rng, 1, wl.head_dim) if wl.outliers else None
    gain_v = synth.outlier_mask(rng, 1, wl.head_dim) if wl.outliers else None
    caches = []
    for _ in range(2):                                # two distinct slices, quantized before timing
        kb = synth.host_values(rng, (wl.context, 1, wl.head_dim), gain_k)
        vb = synth.host_values(rng, (wl.context, 1, wl.head_dim), gain_v)
        caches.append(onv.quantize_rows(kb) + onv.quantize_rows(vb))
    slices, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while elapsed < budget_s and slices < 10000:
            kd, ks, vd, vs = caches[slices % len(caches)]
            qb = synth.host_values(rng, (wl.group, wl.head_dim))
            t = time.perf_counter()
            kh = onv.dequant_rows(kd, ks)
            vh = onv.dequant_rows(vd, vs)
            oatt.decode_heads(onv.bf16_to_f64(qb), kh, vh, wl.sm_scale)
            elapsed += time.perf_counter() - t
            slices += 1
    per_slice = wl.context * (wl.head_dim // 2 + wl.head_dim // 16) * 2
    gbs = slices * per_slice / elapsed / 1e9
    step_bytes = kv_bytes(wl)
    return {
        "value": round(gbs, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{slices} (sequence, KV head) slices of {wl.name}: oracle NVFP4 dequantize + float64 "
                  f"softmax attention of {wl.group} query heads over {wl.context} tokens each, "
                  f"{elapsed:.1f}s on 1 thread (BLAS limited to 1)",
        "steps_per_s": round(gbs * 1e9 / step_bytes, 6),
        "host_cpus": os.cpu_count(), "host_cpus_usable": len(os.sched_getaffinity(0)), "blas_threads": 1,
    }


def read_probe(nk, reps=10):
    """Achievable HBM read bandwidth: the library's streaming-read kernel over a 4 GiB buffer (far
    beyond the 256 MB last-level cache), a few launch shapes, HIP events; the best one."""
    import torch
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    runs = []
    for flags in (nk.PROBE_NONTEMPORAL, 0, nk.PROBE_NONTEMPORAL | nk.PROBE_RANGE, nk.PROBE_RANGE):
        for per_cu in (4, 8, 16, 32):
            blocks = 256 * per_cu
            for _ in range(2):
                nk.hbm_read_probe(buf, blocks, flags, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                nk.hbm_read_probe(buf, blocks, flags, sink)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps / 1e3
            runs.append({"nontemporal": bool(flags & nk.PROBE_NONTEMPORAL), "range_per_workgroup": bool(flags & nk.PROBE_RANGE),
                         "workgroups": blocks, "gbs": round(buf.numel() / t / 1e9, 1)})
    del buf
    torch.cuda.empty_cache()
    best = max(runs, key=lambda r: r["gbs"])
    log(f"[bench] read probe best {best['gbs']} GB/s ({best})")
    return {"gbs": best["gbs"], "bytes": 4 << 30, "best": best, "runs": runs}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variant", choices=["auto", "valu", "mfma", "mfma_lut"], default="auto")
    ap.add_argument("--only", choices=["nvfp4", "fp8", "agentic", "all"], default="all",
                    help="nvfp4 / fp8: only that 32K decode step; agentic: only the prefix-reuse step with "
                         "its extend attention and calibration (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path runs on a single "
              f"MI355X; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_quantized_paged_amd as nk
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))
        return
    nk.lib()
    variant = {"auto": nk.VARIANT_AUTO, "valu": nk.VARIANT_VALU, "mfma": nk.VARIANT_MFMA,
               "mfma_lut": nk.VARIANT_MFMA_LUT}[args.variant]
    wl = synth.WORKLOADS[3]
    if args.only == "agentic":
        res = agentic(nk, synth.WORKLOADS[5], max(5, args.steps // 2), args.warmup)
        print(json.dumps({"agentic_prefix_reuse": res}), flush=True)
        return
    if args.only == "fp8":
        f8 = Bench(nk, wl, True, variant)
        t8 = f8.time_steps(args.steps, args.warmup)
        log(f"[bench] fp8 step {t8 * 1e3:.3f} ms")
        print(json.dumps({"fp8_ms_per_step": round(t8 * 1e3, 4)}))
        return

    nv = Bench(nk, wl, False, variant)
    t_step = nv.time_steps(args.steps, args.warmup)
    t_part, t_part_min = nv.time_partial(max(10, args.steps))
    log(f"[bench] nvfp4 step {t_step * 1e3:.3f} ms, partial mean {t_part * 1e3:.3f} ms min {t_part_min * 1e3:.3f} ms")
    S = nv.S
    nv.free()

    kvb = kv_bytes(wl)
    result = {
        "metric": METRIC,
        "value": round(kvb / t_step / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_ramp_s": RAMP_S,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.variant == "valu" else "f16 (MFMA, f32 accumulate)",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: batch {wl.batch}, {wl.num_q_heads} q / {wl.num_kv_heads} kv heads, "
                               f"head_dim {wl.head_dim}, context {wl.context}, page {wl.page_size}, "
                               f"{S} splits, 2% outlier channels x20, NVFP4 KV (E2M1 + E4M3/16, global scale 1.0)",
                   "batch": wl.batch, "context": wl.context, "num_splits": S},
        "steps_per_s": round(1.0 / t_step, 2),
        "hbm_roofline_frac": round((kvb + io_bytes(wl)) / t_step / 1e9 / HBM_PEAK_GBS, 4),
    }
    alg = kvb + wl.batch * wl.num_q_heads * wl.head_dim * 2 + partial_bytes(wl, S)
    achieved = alg / t_part / 1e9
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic("decode_partial_nvfp4_32k"),
                          "kernel": "decode_partial (NVFP4)", "algorithmic_bytes_per_launch": alg,
                          "mean_launch_ms": round(t_part * 1e3, 4)}
    probe = read_probe(nk)
    result["roofline"]["measured_read_gbs"] = probe["gbs"]
    result["roofline"]["frac_of_measured_read"] = round(achieved / probe["gbs"], 4)
    result["hbm_read_probe"] = probe

    if args.only == "all":
        f8 = Bench(nk, wl, True, variant)
        t8 = f8.time_steps(args.steps, args.warmup)
        f8.free()
        result["fp8"] = {"ms_per_step": round(t8 * 1e3, 4), "steps_per_s": round(1.0 / t8, 2),
                         "kv_gbs": round(kv_bytes(wl, True) / t8 / 1e9, 2),
                         "hbm_roofline_frac": round((kv_bytes(wl, True) + io_bytes(wl)) / t8 / 1e9 / HBM_PEAK_GBS, 4)}
        result["nvfp4_over_fp8_steps"] = round(t8 / t_step, 3)
        log(f"[bench] fp8 step {t8 * 1e3:.3f} ms")

        wl4 = synth.WORKLOADS[4]
        b4 = Bench(nk, wl4, False, variant)
        t4 = b4.time_steps(max(5, args.steps // 2), args.warmup)
        b4.free()
        result["extreme_context_1m"] = {
            "ms_per_step": round(t4 * 1e3, 4), "steps_per_s": round(1.0 / t4, 2),
            "kv_gbs": round(kv_bytes(wl4) / t4 / 1e9, 2),
            "hbm_roofline_frac": round((kv_bytes(wl4) + io_bytes(wl4)) / t4 / 1e9 / HBM_PEAK_GBS, 4),
            "num_splits": wl4.num_splits}
        log(f"[bench] 1m step {t4 * 1e3:.3f} ms")

        result["agentic_prefix_reuse"] = agentic(nk, synth.WORKLOADS[5], max(5, args.steps // 2), args.warmup)

        measured = {(3, wl.batch, False): (t_step, S), (3, wl.batch, True): (t8, S),
                    (4, wl4.batch, False): (t4, wl4.num_splits)}
        result["decode_figures"] = decode_figures(nk, variant, max(5, args.steps // 2), args.warmup, measured)

    if not args.no_cpu_baseline:
        t = time.time()
        result["cpu_baseline"] = cpu_baseline(wl)
        log(f"[bench] cpu baseline {time.time() - t:.1f}s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
