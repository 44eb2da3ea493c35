"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts behind the roofline figure, and the traffic read-back's guard on
the decode kernel's source digest; the CPU-oracle baseline's report."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_long_context_decode_launch():
    """The roofline's bytes are packed KV + scales (144 B per token per KV head
    at d = 128) + q and out in bf16 + the new token of every sequence (bf16 K/V
    rows in, 144 B encoded out per KV head): 1,662,076,416 B per step at 32K,
    batch 44. The partials (f16 o / l and fp32 (m, l): 14,868,480 B at 32
    splits) are reported apart."""
    wl = synth.WORKLOADS[3]
    assert (wl.batch, wl.context, wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.num_splits) == \
        (44, 32768, 8, 40, 128, 32)
    kvb = bench.kv_bytes(wl)
    assert kvb == 44 * 32768 * 8 * 144
    assert kvb + bench.io_bytes(wl) == 1_661_845_504
    assert bench.new_token_bytes(wl) == 44 * 8 * (2 * 128 * 2 + 144)
    assert kvb + bench.io_bytes(wl) + bench.new_token_bytes(wl) == 1_662_076_416
    assert bench.partial_bytes(wl, wl.num_splits) == 44 * 40 * 32 * (128 * 2 + 8) == 14_868_480
    # the FP8 cache moves d bytes per element pair instead of d/2 + d/16: 1/0.5625 as many
    assert bench.kv_bytes(wl, fp8=True) * 9 == kvb * 16
    # other batch sizes (the decode figures) scale linearly
    assert bench.kv_bytes(wl, batch=70) * 44 == kvb * 70


def test_traffic_read_back_follows_the_source_digest(tmp_path, monkeypatch):
    assert bench.read_traffic("no_such_kernel") is None
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_traffic.txt").write_text(f"# comment: ignored\nsource_digest: {bench.source_digest()}\n"
                                        "hbm_bytes_per_launch: 1234\n")
    (prof / "old_traffic.txt").write_text("source_digest: 0000000000000000\nhbm_bytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "DECODE_SOURCES", [os.path.join(ROOT, p) for p in bench.DECODE_SOURCES])
    assert bench.read_traffic("k") == 1234.0
    assert bench.read_traffic("old") is None


def test_cpu_baseline_reports_the_oracle_and_the_host_cores():
    # the tiny decode workload, a fraction of a second of oracle work
    res = bench.cpu_baseline(synth.WORKLOADS[1], budget_s=0.2)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["cores"] == 1
    assert res["value"] > 0 and res["steps_per_s"] > 0
    assert res["host_cpus"] >= res["host_cpus_usable"] >= 1 and res["blas_threads"] == 1
    assert "slices of" in res["sample"]


def test_cpu_baseline_on_several_processes():
    """The all-cores leg: the same oracle work in worker processes started
    before any GPU call, the rate summed over them, the thread count stated."""
    pool = bench.make_pool(2)
    try:
        res = bench.cpu_baseline(synth.WORKLOADS[1], budget_s=0.2, pool=pool, workers=2)
    finally:
        pool.close()
        pool.join()
    assert res["cores"] == 2 and res["all_cores"]["cores"] == 2 and res["single_core"]["cores"] == 1
    assert res["value"] > 0 and res["single_core"]["value"] > 0
    assert "2 processes" in res["sample"]


def test_oracle_pieces_match_the_whole():
    """The bench's parity splits a slice's rows into pieces for the worker
    processes; the oracle's encode is per token, so the pieces joined equal
    the whole (NVFP4 and FP8)."""
    import numpy as np
    rng = np.random.default_rng(3)
    kb = synth.host_values(rng, (1000, 1, 64))
    vb = synth.host_values(rng, (1000, 1, 64))
    for fmt in ("nvfp4", "fp8"):
        whole = bench._oracle_quantize_piece((fmt, kb, vb))
        parts = [bench._oracle_quantize_piece((fmt, kb[t:t + 300], vb[t:t + 300])) for t in range(0, 1000, 300)]
        if fmt == "fp8":
            assert np.array_equal(np.concatenate([p[0] for p in parts]), whole[0])
        else:
            for i in range(2):
                for j in range(2):
                    assert np.array_equal(np.concatenate([p[i][j] for p in parts]), whole[i][j])
