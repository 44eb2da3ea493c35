#!/usr/bin/env python3
"""Benchmark of the NVFP4 paged decode path on one MI355X.

Headline workload: batch 44, 40 query / 8 KV heads, head_dim 128, context
32,768, page 64, 32 splits, K/V ~ N(0,1) bf16 with 2% of channels x20 --
the iso-concurrency long-context point of "Accelerating Long-Context and
Agentic Inference with NVFP4 KV Cache" (section A4, Fig. 6), with the same
layer also run over an FP8-E4M3 cache.

One step = quantize-on-write of the step's new token of every sequence into
the pool (it overwrites the last slot, so the shape stays fixed) + split-KV
decode partials + log-sum-exp merge. The library's decode-with-append call
does the first two in one kernel (the wave whose split holds the new token
encodes and stores it), and with one split (the tiny workload) that kernel
also writes the output, so there is no merge launch; the same step as
separate launches (quantize kernel, partial kernel, merge) is timed beside
it. Inputs are resident in HBM before timing.

Timing method (every figure): after an untimed ramp and the warm-up, each
timed iteration is preceded by an untimed flush (a 1 GiB write, four times
the 256 MB last-level cache, then a 1 GiB read of another buffer, so that the
write's dirty lines are written back before the timed call), so no iteration
finds its predecessor's data in a cache; each iteration is timed with HIP
events on the stream the library launches on; the median, minimum and mean
are reported. Throughput figures use the median unless named otherwise. The
fused step, the separate launches and the partial kernel of a workload are
timed in interleaved rounds (one iteration of each per round), so that they
see the same GPU state.

Prints ONE JSON line on stdout; diagnostics go to stderr.

  value           KV GB/s of the headline step: (packed + scale bytes) / median step
  roofline        dominant kernel (the decode partial kernel with the new token
                  appended, NVFP4, headline workload): (KV + q + out + new-token
                  bytes) / its mean launch time; also against the measured read
                  bandwidth; partial-result bytes reported apart
  configs         the five workloads (tiny, moderate, 32K, 1M, agentic): NVFP4
                  and FP8 step and partial-kernel times, KV GB/s, steps/s,
                  fraction of 8 TB/s, the NVFP4/FP8 step-rate ratio, and the
                  oracle parity of the same run's outputs
  hbm_read_probe  read bandwidth of the library's plain streaming-read kernel
  cpu_baseline    the CPU oracle (dequantize + fp64 attention) on a bounded
                  sample of (sequence, KV head) slices of the headline workload,
                  on all usable host cores and on one
  decode_figures  decode tokens/s of NVFP4 and FP8 at the batch sizes of the
                  page's decode figures (Fig. 6 iso-concurrency: 44 / 10 / 1
                  at 32K / 160K / 1M; Fig. 7 iso-capacity: NVFP4 70 / 15 / 2
                  against FP8 44 / 10 / 1)
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "NVFP4 paged decode attn: KV GB/s + % HBM roofline; steps/s vs FP8-KV kernel"
DECODE_SOURCES = ["nvfp4_quantized_paged_amd/csrc/decode_mfma.hip",
                  "nvfp4_quantized_paged_amd/csrc/common.hpp",
                  "nvfp4_quantized_paged_amd/csrc/encode.hpp"]
FLUSH_BYTES = 1 << 30
TOL_MAX, TOL_MEAN = 2e-2, 2e-3
PIECE = 1 << 16             # token rows per oracle work item


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes(wl, fp8=False, batch=None):
    B = wl.batch if batch is None else batch
    per = wl.head_dim if fp8 else wl.head_dim // 2 + wl.head_dim // 16
    return 2 * B * wl.context * wl.num_kv_heads * per


def io_bytes(wl, batch=None):
    B = wl.batch if batch is None else batch
    return 2 * B * wl.num_q_heads * wl.head_dim * 2      # q read + out written (bf16)


def new_token_bytes(wl, fp8=False, batch=None):
    """The step's new token of every sequence: bf16 K and V rows read, their
    encoded bytes written."""
    B = wl.batch if batch is None else batch
    per = wl.head_dim if fp8 else wl.head_dim // 2 + wl.head_dim // 16
    return 2 * B * wl.num_kv_heads * (2 * wl.head_dim + per)


def partial_bytes(wl, splits, batch=None):
    B = wl.batch if batch is None else batch
    return B * wl.num_q_heads * splits * (wl.head_dim * 2 + 8)      # f16 o / l, fp32 (m, l)


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


# ---------------------------------------------------------------------------
# oracle work on the host cores (worker processes; started before the GPU is touched)
# ---------------------------------------------------------------------------

def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _noop(i):
    return i


def _oracle_quantize_piece(args):
    """Oracle encode of K and V token rows [n][1][d] (bf16 bits): NVFP4 (data,
    scale) pairs, or FP8 bytes."""
    fmt, kb, vb = args
    if fmt == "fp8":
        from oracle import fp8 as of8
        return of8.quantize_rows(kb), of8.quantize_rows(vb)
    from oracle import nvfp4 as onv
    return onv.quantize_rows(kb), onv.quantize_rows(vb)


def _oracle_rate_worker(args):
    """CPU baseline work of one process: quantize two (sequence, KV head) slices
    of the workload, then time the oracle's dequantize + float64 attention over
    them, alternately, for ~budget_s. Returns (slices, seconds)."""
    import numpy as np

    import synth
    from oracle import attention as oatt
    from oracle import nvfp4 as onv
    wl_index, seed, budget_s = args
    wl = synth.WORKLOADS[wl_index]
    rng = np.random.Generator(np.random.PCG64(seed))
    gain_k = synth.outlier_mask(rng, 1, wl.head_dim) if wl.outliers else None
    gain_v = synth.outlier_mask(rng, 1, wl.head_dim) if wl.outliers else None
    caches = []
    for _ in range(2):
        kb = synth.host_values(rng, (wl.context, 1, wl.head_dim), gain_k)
        vb = synth.host_values(rng, (wl.context, 1, wl.head_dim), gain_v)
        caches.append(onv.quantize_rows(kb) + onv.quantize_rows(vb))
    slices, elapsed = 0, 0.0
    while elapsed < budget_s and slices < 100000:
        kd, ks, vd, vs = caches[slices % 2]
        qb = synth.host_values(rng, (wl.group, wl.head_dim))
        t = time.perf_counter()
        oatt.decode_heads(onv.bf16_to_f64(qb), onv.dequant_rows(kd, ks), onv.dequant_rows(vd, vs), wl.sm_scale)
        elapsed += time.perf_counter() - t
        slices += 1
    return slices, elapsed


def usable_cpus():
    return len(os.sched_getaffinity(0))


def make_pool(workers):
    """Worker processes for the oracle, all started now (before any GPU call),
    one BLAS thread each. Their map() keeps the order of its inputs."""
    import multiprocessing
    pool = multiprocessing.get_context("spawn").Pool(processes=workers, initializer=_worker_init)
    pool.map(_noop, range(workers), chunksize=1)
    return pool


def cpu_baseline(wl, budget_s=12.0, pool=None, workers=1):
    """The oracle (dequantize + fp64 attention) on (sequence, KV head) slices
    of the workload: in this process on one thread, and, given a pool, on
    `workers` processes at once (one thread each)."""
    from threadpoolctl import threadpool_limits
    per_slice = wl.context * (wl.head_dim // 2 + wl.head_dim // 16) * 2
    step_bytes = kv_bytes(wl)
    with threadpool_limits(limits=1):
        slices, elapsed = _oracle_rate_worker((wl.index, wl.seed, budget_s))
    gbs1 = slices * per_slice / elapsed / 1e9
    single = {"value": round(gbs1, 5), "unit": "GB/s", "cores": 1,
              "sample": f"{slices} slices, {elapsed:.1f}s on 1 thread",
              "steps_per_s": round(gbs1 * 1e9 / step_bytes, 6)}
    res = {
        "value": single["value"], "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"(sequence, KV head) slices of {wl.name}: oracle NVFP4 dequantize + float64 softmax "
                  f"attention of {wl.group} query heads over {wl.context} tokens each; {slices} slices in "
                  f"{elapsed:.1f}s on 1 thread (BLAS limited to 1)",
        "steps_per_s": single["steps_per_s"],
        "host_cpus": os.cpu_count(), "host_cpus_usable": usable_cpus(), "blas_threads": 1,
        "single_core": single,
    }
    if pool is not None and workers > 1:
        t0 = time.perf_counter()
        runs = pool.map(_oracle_rate_worker, [(wl.index, wl.seed + 17 * (i + 1), budget_s)
                                              for i in range(workers)], chunksize=1)
        wall = time.perf_counter() - t0
        gbs = sum(s * per_slice / e for s, e in runs) / 1e9
        n = sum(s for s, _ in runs)
        res.update({
            "value": round(gbs, 5), "cores": workers,
            "sample": f"(sequence, KV head) slices of {wl.name}: oracle NVFP4 dequantize + float64 softmax "
                      f"attention of {wl.group} query heads over {wl.context} tokens each; {n} slices on "
                      f"{workers} processes at once (one thread each), ~{budget_s:.0f}s of timed work per "
                      f"process ({wall:.1f}s wall with setup); rate = sum of the processes' rates",
            "steps_per_s": round(gbs * 1e9 / step_bytes, 6),
            "all_cores": {"value": round(gbs, 5), "cores": workers, "slices": n},
        })
    return res


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

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


class Flush:
    """Untimed cache flush before each timed iteration: a 1 GiB write, then a
    1 GiB read of another buffer with cached loads (the library's streaming
    read kernel). The write evicts the previous iteration's data; the read
    makes the caches write back the dirty lines of the write before the timed
    call starts instead of during it, and leaves them holding clean, unrelated
    lines."""

    def __init__(self, nk):
        import torch
        self.nk = nk
        self.wbuf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.rbuf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.wbuf.fill_(self.n & 0xFF)
        self.nk.hbm_read_probe(self.rbuf, 2048, 0, self.sink)


def time_flushed(fn, iters, warmup, flush, ramp_s=RAMP_S):
    """Median / minimum / mean duration of `iters` calls of fn, each preceded by
    the flush, timed with HIP events on the launch stream (torch's current
    stream, which the binding passes to the library)."""
    import torch
    if ramp_s > 0:
        ramp(fn, ramp_s)
    for _ in range(warmup):
        flush()
        fn()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median_ms": round(statistics.median(ms), 5), "min_ms": round(ms[0], 5),
            "mean_ms": round(sum(ms) / len(ms), 5), "iters": iters, "wall_s": round(wall, 4)}


def time_flushed_interleaved(fns, iters, warmup, flush, ramp_s=0.2):
    """time_flushed for several calls at once: each timed round runs every call
    of `fns` (name -> callable) once, each after its own flush, so that a slow
    drift of the GPU's state over the first second after a workload is built
    (clocks, translation caches) weighs on all of them alike rather than on
    whichever happens to be timed first. Returns name -> the time_flushed
    figures."""
    import torch
    for fn in fns.values():
        if ramp_s > 0:
            ramp(fn, ramp_s)
    for _ in range(warmup):
        for fn in fns.values():
            flush()
            fn()
    stream = torch.cuda.current_stream()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
          for k in fns}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(iters):
        for k, fn in fns.items():
            a, b = ev[k][i]
            flush()
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out = {}
    for k in fns:
        ms = sorted(a.elapsed_time(b) for a, b in ev[k])
        out[k] = {"median_ms": round(statistics.median(ms), 5), "min_ms": round(ms[0], 5),
                  "mean_ms": round(sum(ms) / len(ms), 5), "iters": iters, "wall_s": round(wall / len(fns), 4)}
    return out


# ---------------------------------------------------------------------------
# uniform-context decode workloads
# ---------------------------------------------------------------------------

class Bench:
    def __init__(self, nk, wl, fp8, variant, batch=None, keep_bf16=False):
        import torch
        from synth.workload import build_uniform_workload
        self.torch = torch
        self.nk, self.wl, self.fp8, self.variant = nk, wl, fp8, variant
        self.batch = B = wl.batch if batch is None else batch
        t = time.time()
        self.w = build_uniform_workload(nk, wl, fp8=fp8, batch=B, keep_bf16=keep_bf16)
        log(f"[bench] built {'fp8' if fp8 else 'nvfp4'} {wl.name} batch {B} in {time.time() - t:.1f}s")
        H, d, P, L = wl.num_kv_heads, wl.head_dim, wl.page_size, wl.context
        g = torch.Generator(device="cuda")
        g.manual_seed(wl.seed + 1000)
        self.k_new = torch.randn((B, H, d), generator=g, device="cuda").to(torch.bfloat16)
        self.v_new = torch.randn((B, H, d), generator=g, device="cuda").to(torch.bfloat16)
        last = L - 1
        self.slots_new = (self.w.bt[:, last // P].to(torch.int64) * P + last % P).contiguous()
        # the workload's split count at its own batch; at another batch (the decode figures) it is kept
        # if it still fills one round of the kernel's resident waves (3 per SIMD for NVFP4, 2 for FP8:
        # 3072 / 2048 items), else the library's automatic count
        self.S = wl.num_splits
        if not self.S or (B != wl.batch and B * H * self.S < (2048 if fp8 else 3072)):
            self.S = nk.nvfp4_paged_decode_num_splits(B, H, self.w.bt.shape[1], P)
        self.ws = nk.decode_workspace(B, wl.num_q_heads, d, self.S)
        self.out = torch.empty_like(self.w.q)

    def quantize(self):
        f = self.nk.fp8_kv_quantize if self.fp8 else self.nk.nvfp4_kv_quantize
        f(self.k_new, self.v_new, self.slots_new, self.w.kp, self.w.vp)

    def partial(self):
        f = self.nk.fp8_paged_decode_partial if self.fp8 else self.nk.nvfp4_paged_decode_partial
        f(self.w.q, self.w.kp, self.w.vp, self.w.bt, self.w.sl, self.wl.sm_scale, self.S,
          variant=self.variant, workspace=self.ws)

    def partial_append(self):
        """The step's partial kernel: the partials with the new token appended by the kernel."""
        if self.variant == self.nk.VARIANT_VALU:
            return self.partial()
        f = self.nk.fp8_paged_decode_append_partial if self.fp8 else self.nk.nvfp4_paged_decode_append_partial
        f(self.w.q, self.k_new, self.v_new, self.w.kp, self.w.vp, self.w.bt, self.w.sl, self.wl.sm_scale, self.S,
          workspace=self.ws)

    def merge(self):
        scale = self.w.vp.scale if self.fp8 else self.w.vp.global_scale
        self.nk.nvfp4kv_lse_merge(self.ws, self.batch, self.wl.num_q_heads, self.wl.head_dim, self.S,
                                  scale, self.out)

    def step(self):
        """One decode step: each sequence's new token quantized into its pool slot by the decode
        kernel itself (quantize-on-write fused into the partial kernel), the partials, the merge
        (with one split the decode kernel writes the output and no merge runs).
        The VALU variant has no fused form and runs the separate step."""
        if self.variant == self.nk.VARIANT_VALU:
            return self.step_separate()
        f = self.nk.fp8_paged_decode_append_attn if self.fp8 else self.nk.nvfp4_paged_decode_append_attn
        f(self.w.q, self.k_new, self.v_new, self.w.kp, self.w.vp, self.w.bt, self.w.sl, self.wl.sm_scale,
          num_splits=self.S, workspace=self.ws, out=self.out)

    def step_separate(self):
        """The same step as three launches: the quantize kernel, the partial kernel, the merge."""
        self.quantize()
        self.partial()
        self.merge()

    def parity(self, pool, samples):
        """Oracle check of this run's outputs (the step has run: the new token
        sits in the last slot): for each sampled (sequence, KV head), the pool
        bytes of every token against the oracle's encode of the bf16 rows, and
        the decode output against the oracle's float64 attention."""
        import numpy as np
        import synth
        from oracle import attention as oatt
        from oracle import fp8 as of8
        from oracle import nvfp4 as onv
        torch = self.torch
        self.step()
        torch.cuda.synchronize()
        wl, w = self.wl, self.w
        G, L, P, d = wl.group, wl.context, wl.page_size, wl.head_dim
        fmt = "fp8" if self.fp8 else "nvfp4"
        bt = w.bt.cpu().numpy()
        got_all = self.out.float().cpu().numpy().astype(np.float64)
        errs, raws, bytes_exact = [], [], True
        t0 = time.time()
        for b, g in samples:
            k_rows = synth.bf16_tensor_bits(w.k_bf16[b, :, g])[:, None, :]
            v_rows = synth.bf16_tensor_bits(w.v_bf16[b, :, g])[:, None, :]
            k_rows[L - 1, 0] = synth.bf16_tensor_bits(self.k_new[b, g])
            v_rows[L - 1, 0] = synth.bf16_tensor_bits(self.v_new[b, g])
            jobs = [(fmt, k_rows[t:t + PIECE], v_rows[t:t + PIECE]) for t in range(0, L, PIECE)]
            parts = pool.map(_oracle_quantize_piece, jobs, chunksize=1) if pool is not None else \
                [_oracle_quantize_piece(j) for j in jobs]
            t = np.arange(L)
            pages = torch.from_numpy(bt[b][t // P].astype(np.int64)).cuda()
            offs = torch.from_numpy(t % P).cuda()
            if self.fp8:
                kr = np.concatenate([p[0] for p in parts])
                vr = np.concatenate([p[1] for p in parts])
                bytes_exact &= np.array_equal(w.kp.data[pages, g, offs].cpu().numpy(), kr[:, 0])
                bytes_exact &= np.array_equal(w.vp.data[pages, g, offs].cpu().numpy(), vr[:, 0])
                khat, vhat = of8.dequant_cache(kr, w.kp.scale), of8.dequant_cache(vr, w.vp.scale)
            else:
                kd = np.concatenate([p[0][0] for p in parts])
                ks = np.concatenate([p[0][1] for p in parts])
                vd = np.concatenate([p[1][0] for p in parts])
                vs = np.concatenate([p[1][1] for p in parts])
                for pool_t, ref in ((w.kp.data, kd), (w.kp.scale, ks), (w.vp.data, vd), (w.vp.scale, vs)):
                    bytes_exact &= np.array_equal(pool_t[pages, g, offs].cpu().numpy(), ref[:, 0])
                khat, vhat = onv.dequant_rows(kd, ks), onv.dequant_rows(vd, vs)
            qb = synth.bf16_tensor_bits(w.q[b, g * G:(g + 1) * G])
            ref, mass = oatt.decode_heads(onv.bf16_to_f64(qb), khat, vhat, wl.sm_scale)
            raw = np.abs(got_all[b, g * G:(g + 1) * G] - ref)
            errs.append(raw / np.maximum(1.0, mass))
            raws.append(raw)
        e, raw = np.concatenate([x.ravel() for x in errs]), np.concatenate([x.ravel() for x in raws])
        ok = bool(bytes_exact and e.max() <= TOL_MAX and e.mean() <= TOL_MEAN)
        res = {"samples": f"{len(samples)} whole (sequence, KV head) outputs over all {L} tokens "
                          f"({len(samples) * G} query heads), and the pool bytes of those tokens",
               "bytes_exact": bool(bytes_exact), "max_e": float(f"{e.max():.4g}"), "mean_e": float(f"{e.mean():.4g}"),
               "raw_max_abs": float(f"{raw.max():.4g}"), "raw_mean_abs": float(f"{raw.mean():.4g}"),
               "tolerance": "e = |gpu - oracle| / max(1, sum_t p_t |v_t|): max <= 2e-2, mean <= 2e-3",
               "pass": ok, "oracle_s": round(time.time() - t0, 1)}
        log(f"[bench] parity {fmt} {wl.name} B{self.batch}: bytes exact {bytes_exact}, max e {e.max():.3e} "
            f"mean e {e.mean():.3e} ({time.time() - t0:.1f}s)")
        return res

    def free(self):
        del self.w, self.ws, self.out
        self.torch.cuda.empty_cache()


def _samples(wl, B, which):
    H = wl.num_kv_heads
    if which == "all":
        return [(b, g) for b in range(B) for g in range(H)]
    if which == "two":
        return [(0, 0), (B - 1, H - 1)]
    return [(B - 1, H - 2 if H > 1 else 0)]


def uniform_config(nk, wl, variant, iters, warmup, flush, pool, parity_samples, formats=("nvfp4", "fp8"),
                   batch=None):
    """One uniform-context workload over the NVFP4 and FP8 caches: the whole
    step, the same step as separate launches, the step's partial kernel alone
    (with the append) and the partial kernel without the append, timed in
    interleaved rounds, and the same run's parity."""
    B = wl.batch if batch is None else batch
    res = {"workload": wl.name, "batch": B, "context": wl.context, "num_q_heads": wl.num_q_heads,
           "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "page_size": wl.page_size,
           "outliers": wl.outliers}
    for fmt in formats:
        fp8 = fmt == "fp8"
        bch = Bench(nk, wl, fp8, variant, batch=B, keep_bf16=parity_samples is not None)
        tt = time_flushed_interleaved({"step": bch.step, "separate": bch.step_separate,
                                       "partial": bch.partial_append, "partial_plain": bch.partial},
                                      iters, warmup, flush)
        step, step_sep, part, part_plain = tt["step"], tt["separate"], tt["partial"], tt["partial_plain"]
        kvb = kv_bytes(wl, fp8, B)
        io = io_bytes(wl, B) + new_token_bytes(wl, fp8, B)
        t = step["median_ms"] / 1e3
        tp = part["median_ms"] / 1e3
        r = {"num_splits": bch.S, "step": step, "step_separate": step_sep, "partial": part,
             "partial_without_append": part_plain,
             "kv_gbs": round(kvb / t / 1e9, 1), "steps_per_s": round(1.0 / t, 2),
             "hbm_roofline_frac": round((kvb + io) / t / 1e9 / HBM_PEAK_GBS, 4),
             "partial_hbm_roofline_frac": round((kvb + io) / tp / 1e9 / HBM_PEAK_GBS, 4),
             "kv_bytes": kvb, "q_out_bytes": io, "partial_bytes_written": partial_bytes(wl, bch.S, B)}
        if parity_samples is not None:
            r["parity"] = bch.parity(pool, _samples(wl, B, parity_samples))
        log(f"[bench] {fmt} {wl.name} B{B}: step median {step['median_ms']:.4f} ms min {step['min_ms']:.4f} "
            f"(separate launches {step_sep['median_ms']:.4f}), partial median {part['median_ms']:.4f} ms "
            f"(without the append {part_plain['median_ms']:.4f}), "
            f"{r['kv_gbs']} GB/s KV")
        res[fmt] = r
        bch.free()
    if "nvfp4" in res and "fp8" in res:
        res["nvfp4_over_fp8_steps"] = round(res["fp8"]["step"]["median_ms"] / res["nvfp4"]["step"]["median_ms"], 3)
    return res


def decode_figures(nk, variant, iters, warmup, flush, measured):
    """Kernel-level decode throughput at the batch sizes of the NVFP4 page's
    decode figures: iso-concurrency (Fig. 6, both caches at the same batch)
    and iso-capacity (Fig. 7, each cache at the batch it fits in the same
    memory), at 32K, 160K and 1M context. One step = append the new token
    + decode partial + merge; decode tokens/s = batch / median step time.
    Steps already timed are reused from `measured`."""
    import synth

    def run(idx, batch, fp8):
        key = (idx, batch, fp8)
        if key not in measured:
            b = Bench(nk, synth.WORKLOADS[idx], fp8, variant, batch=batch)
            measured[key] = (time_flushed(b.step, iters, warmup, flush, ramp_s=0.2)["median_ms"] / 1e3, b.S)
            b.free()
        t, S = measured[key]
        wl = synth.WORKLOADS[idx]
        return {"batch": batch, "num_splits": S, "ms_per_step": round(t * 1e3, 4),
                "decode_tokens_per_s": round(batch / t, 1), "kv_gbs": round(kv_bytes(wl, fp8, batch) / t / 1e9, 1)}
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


# ---------------------------------------------------------------------------
# agentic prefix reuse
# ---------------------------------------------------------------------------

def _oracle_sequence_rows(w, b, pool):
    """The oracle's NVFP4 rows (K data, K scales, V data, V scales) of every
    token of agentic sequence b (shared prefix, private tokens, the new chunk),
    quantized from the generated bf16 sources."""
    import numpy as np
    import synth
    C, H = w.wl.chunk, w.wl.num_kv_heads
    kb = np.concatenate([synth.bf16_tensor_bits(w.k_shared), synth.bf16_tensor_bits(w.k_private[b]),
                         synth.bf16_tensor_bits(w.k_chunk[b * C:(b + 1) * C])])
    vb = np.concatenate([synth.bf16_tensor_bits(w.v_shared), synth.bf16_tensor_bits(w.v_private[b]),
                         synth.bf16_tensor_bits(w.v_chunk[b * C:(b + 1) * C])])
    step = max(1, PIECE // H)
    jobs = [("nvfp4", kb[t:t + step], vb[t:t + step]) for t in range(0, len(kb), step)]
    parts = pool.map(_oracle_quantize_piece, jobs, chunksize=1) if pool is not None else \
        [_oracle_quantize_piece(j) for j in jobs]
    return tuple(np.concatenate([p[i][j] for p in parts]) for i in (0, 1) for j in (0, 1))


def agentic_parity(nk, w, out, pool, seqs=(0, 37)):
    """Oracle check of the agentic step's outputs for sampled sequences: the
    pool bytes of every token (shared prefix, private tokens, the new chunk),
    the workspace rows (bit-exact) and the decode output."""
    import numpy as np
    import torch
    import synth
    from oracle import attention as oatt
    from oracle import nvfp4 as onv
    wl = w.wl
    H, P, G, C = wl.num_kv_heads, wl.page_size, wl.group, wl.chunk
    offs = w.ws_row_offsets.cpu().numpy()
    got = out.float().cpu().numpy().astype(np.float64)
    errs, raws, exact = [], [], True
    t0 = time.time()
    for b in seqs:
        L = int(w.host_cached_lens[b])
        kd, ks, vd, vs = _oracle_sequence_rows(w, b, pool)
        t = np.arange(L + C)
        pages = torch.from_numpy(w.host_bt[b][t // P].astype(np.int64)).cuda()
        offp = torch.from_numpy(t % P).cuda()
        for pool_t, ref in ((w.kp.data, kd), (w.kp.scale, ks), (w.vp.data, vd), (w.vp.scale, vs)):
            exact &= np.array_equal(pool_t[pages, :, offp].cpu().numpy(), ref)
        khat, vhat = onv.dequant_rows(kd, ks), onv.dequant_rows(vd, vs)
        exact &= np.array_equal(synth.bf16_tensor_bits(w.k_ws[offs[b]:offs[b] + L]), oatt.f64_to_bf16_exact(khat[:L]))
        exact &= np.array_equal(synth.bf16_tensor_bits(w.v_ws[offs[b]:offs[b] + L]), oatt.f64_to_bf16_exact(vhat[:L]))
        qb = onv.bf16_to_f64(synth.bf16_tensor_bits(w.q[b]))
        ref, mass = oatt.decode_heads(qb, khat, vhat, wl.sm_scale)
        raw = np.abs(got[b] - ref)
        errs.append((raw / np.maximum(1.0, mass)).ravel())
        raws.append(raw.ravel())
    e, raw = np.concatenate(errs), np.concatenate(raws)
    res = {"samples": f"sequences {list(seqs)}: pool bytes of all their tokens, their workspace rows, "
                      f"their decode outputs",
           "bytes_exact": bool(exact), "max_e": float(f"{e.max():.4g}"), "mean_e": float(f"{e.mean():.4g}"),
           "raw_max_abs": float(f"{raw.max():.4g}"), "raw_mean_abs": float(f"{raw.mean():.4g}"),
           "pass": bool(exact and e.max() <= TOL_MAX and e.mean() <= TOL_MEAN), "oracle_s": round(time.time() - t0, 1)}
    log(f"[bench] parity agentic: bytes and workspace exact {exact}, max e {e.max():.3e} mean e {e.mean():.3e}")
    return res


def extend_parity(w, qx, ox, q_offs_host, pool, b=5, last=4, chunk8=None):
    """Oracle check of the extend output: the last `last` queries of sequence b,
    as an extend problem whose prefix is the cached prefix plus the chunk
    tokens before them (the same keys and positions). The keys and values are
    the oracle's: the cached prefix quantized and dequantized by the oracle
    (bf16 workspace), or its E4M3 workspace bytes (chunk8 = the chunk's FP8
    source bytes: FP8 workspace, scales 1), then the chunk's own rows."""
    import numpy as np
    import synth
    from oracle import attention as oatt
    from oracle import nvfp4 as onv
    wl = w.wl
    C, L = wl.chunk, int(w.host_cached_lens[b])
    n = L + C
    kd, ks, vd, vs = _oracle_sequence_rows(w, b, pool)
    if chunk8 is None:
        kc = synth.bf16_bits_to_f64(synth.bf16_tensor_bits(w.k_chunk[b * C:(b + 1) * C]))
        vc = synth.bf16_bits_to_f64(synth.bf16_tensor_bits(w.v_chunk[b * C:(b + 1) * C]))
        kw = np.concatenate([onv.dequant_rows(kd[:L], ks[:L]), kc])
        vw = np.concatenate([onv.dequant_rows(vd[:L], vs[:L]), vc])
    else:
        k8, v8 = (c[b * C:(b + 1) * C].cpu().numpy() for c in chunk8)
        kw = onv.E4M3_VALUES[np.concatenate([onv.workspace_fp8_bytes(kd[:L], ks[:L]), k8]).astype(np.int64)]
        vw = onv.E4M3_VALUES[np.concatenate([onv.workspace_fp8_bytes(vd[:L], vs[:L]), v8]).astype(np.int64)]
    r0 = int(q_offs_host[b]) + C - last
    q = synth.bf16_bits_to_f64(synth.bf16_tensor_bits(qx[r0:r0 + last]))
    ref, mass = oatt.extend_attention(q, kw, vw, np.array([0, last]), np.array([0, n]),
                                      np.array([n - last], np.int32), wl.sm_scale)
    got = ox[r0:r0 + last].float().cpu().numpy().astype(np.float64)
    raw = np.abs(got - ref)
    e = raw / np.maximum(1.0, mass)
    return {"samples": f"the last {last} chunk queries of sequence {b} (all {wl.num_q_heads} heads, {n - last + 1}.."
                       f"{n} keys)", "max_e": float(f"{e.max():.4g}"), "mean_e": float(f"{e.mean():.4g}"),
            "raw_max_abs": float(f"{raw.max():.4g}"), "pass": bool(e.max() <= TOL_MAX and e.mean() <= TOL_MEAN)}


def agentic(nk, wl, iters, warmup, flush, pool, parity=True):
    """The prefix-reuse step (quantize the new chunk, dequantize every cached
    prefix into the workspace, decode all sequences with the shared-prefix
    decode, which unpacks the batch's common 2,800-token prefix once per 16
    query columns): the whole step and each kernel alone, timed as
    time_flushed does; the plain decode of the same batch is timed beside it. Run twice: with bf16 chunk and
    workspace (the workload definition) and with the pages' FP8 types (FP8
    chunk quantized to NVFP4 and copied into an FP8 workspace in one pass,
    FP8 workspace). Then extend attention over the bf16 workspace and over
    the FP8 one, and the calibration absmax, outside the step."""
    import numpy as np
    import torch
    from synth.workload import agentic_bytes, build_agentic_workload
    t = time.time()
    w = build_agentic_workload(nk, wl, keep_bf16=parity)
    log(f"[bench] built agentic workload in {time.time() - t:.1f}s")
    B, Hq, d, H, C = wl.batch, wl.num_q_heads, wl.head_dim, wl.num_kv_heads, wl.chunk
    S = nk.nvfp4_paged_decode_num_splits(B, H, w.bt.shape[1], wl.page_size)
    ws = nk.decode_workspace(B, Hq, d, S)
    out = torch.empty_like(w.q)
    out_plain = torch.empty_like(w.q)
    shared = wl.shared_prefix
    wsc = torch.empty(nk.nvfp4_paged_decode_shared_prefix_workspace_bytes(w.kp, w.bt.shape[1], B, Hq, shared),
                      dtype=torch.uint8, device="cuda")
    quant = lambda: nk.nvfp4_kv_quantize(w.k_chunk, w.v_chunk, w.slot_chunk, w.kp, w.vp)
    deq = lambda: nk.nvfp4_kv_dequant_workspace(w.kp, w.vp, w.bt, w.cached_lens, w.ws_row_offsets, w.k_ws, w.v_ws)
    decode = lambda: nk.nvfp4_paged_decode_attn_shared_prefix(w.q, w.kp, w.vp, w.bt, w.seq_lens, wl.sm_scale,
                                                              shared, workspace=wsc, out=out)
    decode_plain = lambda: nk.nvfp4_paged_decode_attn(w.q, w.kp, w.vp, w.bt, w.seq_lens, wl.sm_scale,
                                                      num_splits=S, workspace=ws, out=out_plain)

    def step():
        quant()
        deq()
        decode()
    by = agentic_bytes(w)
    ts = time_flushed(step, iters, warmup, flush, ramp_s=0.2)
    tq = time_flushed(quant, iters, warmup, flush, ramp_s=0.1)
    td = time_flushed(deq, iters, warmup, flush, ramp_s=0.1)
    tcs = time_flushed_interleaved({"shared": decode, "plain": decode_plain}, iters, warmup, flush, ramp_s=0.1)
    tc, tcp = tcs["shared"], tcs["plain"]
    med = lambda r: r["median_ms"] / 1e3
    res = {
        "workload": wl.name, "batch": B, "len_min": wl.len_min, "len_max": wl.len_max,
        "shared_prefix": wl.shared_prefix, "chunk": C, "num_splits": S,
        "step": ts, "steps_per_s": round(1.0 / med(ts), 2),
        "quantize": {**tq, "gbs": round((by["quant_read"] + by["quant_write"]) / med(tq) / 1e9, 1)},
        "dequant_workspace": {**td, "gbs_unique": round((by["dequant_read_unique"] + by["dequant_write"]) / med(td) / 1e9, 1),
                              "write_gbs": round(by["dequant_write"] / med(td) / 1e9, 1)},
        "decode": {**tc, "kv_gbs_logical": round(by["decode_read_logical"] / med(tc) / 1e9, 1),
                   "kv_gbs_unique": round(by["decode_read_unique"] / med(tc) / 1e9, 1),
                   "kind": f"shared-prefix decode, {shared}-token prefix"},
        "decode_plain": {**tcp, "kv_gbs_logical": round(by["decode_read_logical"] / med(tcp) / 1e9, 1),
                         "kv_gbs_unique": round(by["decode_read_unique"] / med(tcp) / 1e9, 1),
                         "num_splits": S},
        "bytes": by,
    }
    log(f"[bench] agentic step {ts['median_ms']:.4f} ms: quantize {tq['median_ms']:.4f}, workspace "
        f"{td['median_ms']:.4f}, decode {tc['median_ms']:.4f} ms (plain decode {tcp['median_ms']:.4f})")
    if parity:
        step()
        torch.cuda.synchronize()
        res["parity"] = agentic_parity(nk, w, out, pool)

    # the pages' path-2 types: FP8 chunk and FP8 workspace
    k8 = w.k_chunk.to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = w.v_chunk.to(torch.float8_e4m3fn).view(torch.uint8)
    rows = int(w.ws_row_offsets[-1].item())
    kws8 = torch.empty((rows, H, d), dtype=torch.uint8, device="cuda")
    vws8 = torch.empty((rows, H, d), dtype=torch.uint8, device="cuda")
    offs = w.ws_row_offsets.cpu().numpy()
    chunk_rows = np.concatenate([offs[b] + w.host_cached_lens[b] + np.arange(C) for b in range(B)]).astype(np.int64)
    ws_rows = torch.from_numpy(chunk_rows).cuda()
    quant8 = lambda: nk.nvfp4_kv_quantize_fp8(k8, v8, w.slot_chunk, w.kp, w.vp, 1.0, 1.0, ws_rows, kws8, vws8)
    deq8 = lambda: nk.nvfp4_kv_dequant_workspace_fp8(w.kp, w.vp, w.bt, w.cached_lens, w.ws_row_offsets, kws8, vws8)

    def step8():
        quant8()
        deq8()
        decode()
    ts8 = time_flushed(step8, iters, warmup, flush, ramp_s=0.2)
    tq8 = time_flushed(quant8, iters, warmup, flush, ramp_s=0.1)
    td8 = time_flushed(deq8, iters, warmup, flush, ramp_s=0.1)
    q_rd = by["quant_read"] // 2                        # FP8 chunk: one byte per element
    q_wr = by["quant_write"] + q_rd                     # NVFP4 + the chunk copied into the workspace
    dq_wr = by["dequant_write"] // 2
    res["fp8_path2"] = {
        "step": ts8, "steps_per_s": round(1.0 / med(ts8), 2),
        "quantize_with_chunk_copy": {**tq8, "gbs": round((q_rd + q_wr) / med(tq8) / 1e9, 1)},
        "dequant_workspace_fp8": {**td8, "gbs_unique": round((by["dequant_read_unique"] + dq_wr) / med(td8) / 1e9, 1),
                                  "write_gbs": round(dq_wr / med(td8) / 1e9, 1)},
    }
    log(f"[bench] agentic fp8 path-2 step {ts8['median_ms']:.4f} ms: quantize {tq8['median_ms']:.4f}, "
        f"workspace {td8['median_ms']:.4f} ms")

    # extend attention of the chunk over the bf16 workspace (path 2's consumer), not part of the step:
    # the chunk's K/V go to the workspace rows after each prefix, then its queries attend causally
    deq()
    crow = torch.from_numpy(chunk_rows).cuda()
    w.k_ws[crow] = w.k_chunk
    w.v_ws[crow] = w.v_chunk
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 2000)
    qx = torch.randn((B * C, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    q_offs_host = np.arange(0, B * C + 1, C, dtype=np.int64)
    q_offs = torch.from_numpy(q_offs_host).cuda()
    ox = torch.empty_like(qx)
    ext = lambda: nk.nvfp4_extend_attn(qx, q_offs, w.k_ws, w.v_ws, w.ws_row_offsets, w.cached_lens, wl.sm_scale,
                                       max_chunk=C, out=ox)
    te = time_flushed(ext, max(5, iters // 3), 2, flush, ramp_s=0.0)
    Lc = w.host_cached_lens.astype(np.float64)
    flops = 4.0 * d * Hq * float(np.sum(C * Lc + C * (C + 1) / 2.0))
    res["extend_attention"] = {**te, "tflops": round(flops / med(te) / 1e12, 1),
                               "bf16_mfma_peak_frac": round(flops / med(te) / 2.5e15, 4), "flops": flops}
    log(f"[bench] extend attention {te['median_ms']:.3f} ms, {flops / med(te) / 1e12:.1f} TFLOP/s")
    if parity:
        res["extend_attention"]["parity"] = extend_parity(w, qx, ox, q_offs_host, pool)

    # the same over the pages' FP8 workspace: the prefix from the FP8 workspace kernel, the chunk's FP8 bytes
    # copied next to it by the FP8 quantize (both above), workspace scales 1
    deq8()
    quant8()
    ext8 = lambda: nk.nvfp4_extend_attn_fp8(qx, q_offs, kws8, vws8, w.ws_row_offsets, w.cached_lens, wl.sm_scale,
                                            1.0, 1.0, max_chunk=C, out=ox)
    te8 = time_flushed(ext8, max(5, iters // 3), 2, flush, ramp_s=0.0)
    res["fp8_path2"]["extend_attention_fp8"] = {**te8, "tflops": round(flops / med(te8) / 1e12, 1),
                                                "bf16_mfma_peak_frac": round(flops / med(te8) / 2.5e15, 4)}
    log(f"[bench] extend attention over the FP8 workspace {te8['median_ms']:.3f} ms, "
        f"{flops / med(te8) / 1e12:.1f} TFLOP/s")
    if parity:
        res["fp8_path2"]["extend_attention_fp8"]["parity"] = extend_parity(w, qx, ox, q_offs_host, pool,
                                                                           chunk8=(k8, v8))

    # global-scale calibration of the chunk (absmax of K and V), not part of the step
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    cal = lambda: (nk.nvfp4_kv_absmax(w.k_chunk, amax[0:1]), nk.nvfp4_kv_absmax(w.v_chunk, amax[1:2]))
    tcal = time_flushed(cal, iters, warmup, flush, ramp_s=0.1)
    res["absmax_calibration"] = {**tcal, "gbs": round(by["quant_read"] / med(tcal) / 1e9, 1)}
    log(f"[bench] absmax calibration {tcal['median_ms']:.4f} ms")
    del w, ws, out, kws8, vws8, qx, ox
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# read ceiling
# ---------------------------------------------------------------------------

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


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30, help="timed iterations of each figure")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variant", choices=["auto", "valu", "mfma", "mfma_lut"], default="auto")
    ap.add_argument("--only", choices=["nvfp4", "fp8", "agentic", "all"], default="all",
                    help="nvfp4 / fp8: only that 32K decode step; agentic: only the prefix-reuse step with "
                         "its extend attention and calibration (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle checks of the outputs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path runs on a single "
              f"MI355X; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        # no worker pool here: under a counter-collecting profiler every worker process would
        # load the profiler's tool as well
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))
        return

    parity = not args.no_parity and args.only in ("all", "agentic")
    workers = min(16, usable_cpus())
    pool = make_pool(workers) if (parity or (not args.no_cpu_baseline and args.only == "all")) else None

    import torch
    import nvfp4_quantized_paged_amd as nk
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nk.lib()
    variant = {"auto": nk.VARIANT_AUTO, "valu": nk.VARIANT_VALU, "mfma": nk.VARIANT_MFMA,
               "mfma_lut": nk.VARIANT_MFMA_LUT}[args.variant]
    flush = Flush(nk)
    iters, warmup = args.steps, args.warmup
    wl = synth.WORKLOADS[3]
    if args.only == "agentic":
        res = agentic(nk, synth.WORKLOADS[5], iters, warmup, flush, pool, parity=parity)
        print(json.dumps({"agentic_prefix_reuse": res}), flush=True)
        return
    if args.only in ("nvfp4", "fp8"):
        r = uniform_config(nk, wl, variant, iters, warmup, flush, None, None, formats=(args.only,))
        print(json.dumps(r), flush=True)
        return

    # headline: the 32K workload, NVFP4 and FP8, same-run parity
    c3 = uniform_config(nk, wl, variant, iters, warmup, flush, pool, "two" if parity else None)
    nv = c3["nvfp4"]
    t_step = nv["step"]["median_ms"] / 1e3
    kvb, io = kv_bytes(wl), io_bytes(wl) + new_token_bytes(wl)
    alg = kvb + io
    t_part = nv["partial"]["mean_ms"] / 1e3
    achieved = alg / t_part / 1e9
    result = {
        "metric": METRIC,
        "value": round(kvb / t_step / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": iters,
        "warmup": warmup,
        "warmup_ramp_s": RAMP_S,
        "ms_per_step": round(t_step * 1e3, 4),
        "ms_per_step_min": nv["step"]["min_ms"],
        "timing": "median of the timed steps, each preceded by an untimed flush (1 GiB write, then 1 GiB "
                  "read of another buffer); HIP events on the launch stream",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.variant == "valu" else "f16 (MFMA, f32 accumulate)",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: batch {wl.batch}, {wl.num_q_heads} q / {wl.num_kv_heads} kv heads, "
                               f"head_dim {wl.head_dim}, context {wl.context}, page {wl.page_size}, "
                               f"{nv['num_splits']} splits, 2% outlier channels x20, NVFP4 KV (E2M1 + E4M3/16, "
                               f"global scale 1.0)",
                   "batch": wl.batch, "context": wl.context, "num_splits": nv["num_splits"]},
        "steps_per_s": nv["steps_per_s"],
        "hbm_roofline_frac": nv["hbm_roofline_frac"],
        "fp8_steps_per_s": c3["fp8"]["steps_per_s"],
        "nvfp4_over_fp8_steps": c3["nvfp4_over_fp8_steps"],
    }
    result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4),
                          "traffic": read_traffic("decode_partial_nvfp4_32k"),
                          "kernel": "decode_partial with the new token appended (NVFP4)",
                          "algorithmic_bytes_per_launch": alg,
                          "algorithmic_bytes": "packed KV + block scales + q + out (bf16) + the new token "
                                               "(bf16 K/V rows in, encoded bytes out)",
                          "partial_bytes_written": nv["partial_bytes_written"],
                          "mean_launch_ms": nv["partial"]["mean_ms"], "median_launch_ms": nv["partial"]["median_ms"],
                          "min_launch_ms": nv["partial"]["min_ms"]}
    probe = read_probe(nk)
    result["roofline"]["measured_read_gbs"] = probe["gbs"]
    result["roofline"]["frac_of_measured_read"] = round(achieved / probe["gbs"], 4)
    result["hbm_read_probe"] = probe

    if args.only == "all":
        ps = lambda which: which if parity else None
        configs = {
            "tiny": uniform_config(nk, synth.WORKLOADS[1], variant, iters, warmup, flush, pool, ps("all")),
            "moderate_batch": uniform_config(nk, synth.WORKLOADS[2], variant, iters, warmup, flush, pool, ps("all")),
            "long_context_32k": c3,
            "extreme_context_1m": uniform_config(nk, synth.WORKLOADS[4], variant, iters, warmup, flush, pool,
                                                 ps("one")),
            "agentic_prefix_reuse": agentic(nk, synth.WORKLOADS[5], iters, warmup, flush, pool, parity=parity),
        }
        result["configs"] = configs
        c4 = configs["extreme_context_1m"]
        measured = {(3, wl.batch, False): (t_step, nv["num_splits"]),
                    (3, wl.batch, True): (c3["fp8"]["step"]["median_ms"] / 1e3, c3["fp8"]["num_splits"]),
                    (4, synth.WORKLOADS[4].batch, False): (c4["nvfp4"]["step"]["median_ms"] / 1e3,
                                                          c4["nvfp4"]["num_splits"])}
        result["decode_figures"] = decode_figures(nk, variant, iters, warmup, flush, measured)
        ag = configs["agentic_prefix_reuse"]
        agentic_checks = (ag.get("parity"), ag.get("extend_attention", {}).get("parity"),
                          ag.get("fp8_path2", {}).get("extend_attention_fp8", {}).get("parity"))
        result["parity_all_pass"] = all(
            c[f]["parity"]["pass"] for c in configs.values() for f in ("nvfp4", "fp8") if f in c and "parity" in c[f]
        ) and all(p["pass"] for p in agentic_checks if p is not None) if parity else None

    if not args.no_cpu_baseline:
        t = time.time()
        result["cpu_baseline"] = cpu_baseline(wl, pool=pool, workers=workers)
        log(f"[bench] cpu baseline {time.time() - t:.1f}s")
    if pool is not None:
        pool.close()
        pool.join()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
