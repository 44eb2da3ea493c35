"""GPU parity of the HIP path (called through the C ABI) against the CPU oracle.

Bars:
  * quantize (NVFP4 and FP8) and the dequantized workspace: bit-exact, over
    the whole pool including bytes that must stay untouched;
  * decode output: per element e = |gpu - ref| / max(1, sum_t p_t |v_t|) with
    max e <= 2e-2 and mean e <= 2e-3 (the absolute tolerance read against
    each output's natural magnitude; raw errors are printed too).
Every case prints its name, shape and seed before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import fp8 as of8
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu

SENT = 0xAB
TOL_MAX, TOL_MEAN = 2e-2, 2e-3


@pytest.fixture(scope="module")
def nk():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import nvfp4_quantized_paged_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def nv_pools(nk, num_pages, H, P, d, gs=1.0):
    k = nk.NVFP4Pool.empty(num_pages, H, P, d, global_scale=gs)
    v = nk.NVFP4Pool.empty(num_pages, H, P, d, global_scale=gs)
    for t in (k.data, k.scale, v.data, v.scale):
        t.fill_(SENT)
    return k, v


def f8_pools(nk, num_pages, H, P, d, scale=1.0):
    k = nk.FP8Pool.empty(num_pages, H, P, d, scale=scale)
    v = nk.FP8Pool.empty(num_pages, H, P, d, scale=scale)
    k.data.fill_(SENT)
    v.data.fill_(SENT)
    return k, v


def oracle_nv(num_pages, H, P, d, k_bits, v_bits, slots, gs=1.0):
    kd, ks = onv.empty_cache(num_pages, H, P, d, fill=SENT)
    vd, vs = onv.empty_cache(num_pages, H, P, d, fill=SENT)
    onv.write_cache(kd, ks, k_bits, slots, gs)
    onv.write_cache(vd, vs, v_bits, slots, gs)
    return kd, ks, vd, vs


def gpu_quantize_nv(nk, num_pages, H, P, d, k_bits, v_bits, slots, gs=1.0, kt=None, vt=None):
    kp, vp = nv_pools(nk, num_pages, H, P, d, gs)
    kt = synth.to_device_bf16(k_bits) if kt is None else kt
    vt = synth.to_device_bf16(v_bits) if vt is None else vt
    nk.nvfp4_kv_quantize(kt, vt, synth.to_device(slots.astype(np.int64)), kp, vp)
    torch.cuda.synchronize()
    return kp, vp


def assert_pool_equal(gpu_t, ref, what):
    got = gpu_t.cpu().numpy()
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} bytes differ; first at {i}: gpu {got[i]:#04x} oracle {ref[i]:#04x}")


def check_out(out_t, ref, mass, what):
    got = out_t.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    raw = np.abs(got - ref)
    e = raw / np.maximum(1.0, mass)
    say(f"  {what}: max e {e.max():.3e} mean e {e.mean():.3e} | raw max {raw.max():.3e} mean {raw.mean():.3e}")
    assert e.max() <= TOL_MAX and e.mean() <= TOL_MEAN, what


def decode_problem(nk, inp, splits_list=(0,), variants=(None,), gs=1.0, label=""):
    """Quantize inp on both sides, check bytes, decode on the GPU, compare."""
    wl = inp.wl
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    kp, vp = gpu_quantize_nv(nk, inp.num_pages, H, P, d, inp.k, inp.v, inp.slot_mapping, gs)
    kd, ks, vd, vs = oracle_nv(inp.num_pages, H, P, d, inp.k, inp.v, inp.slot_mapping, gs)
    assert_pool_equal(kp.data, kd, f"{label} K data")
    assert_pool_equal(kp.scale, ks, f"{label} K scale")
    assert_pool_equal(vp.data, vd, f"{label} V data")
    assert_pool_equal(vp.scale, vs, f"{label} V scale")
    ref, mass = oatt.paged_decode(inp.q, onv.dequant_cache(kd, ks, gs), onv.dequant_cache(vd, vs, gs),
                                  inp.block_tables, inp.seq_lens, wl.sm_scale)
    q = synth.to_device_bf16(inp.q)
    bt = synth.to_device(inp.block_tables)
    sl = synth.to_device(inp.seq_lens)
    outs = []
    for S in splits_list:
        for var in variants:
            if var is None:
                out = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl, wl.sm_scale, num_splits=S)
            else:
                Sx = S or nk.nvfp4_paged_decode_num_splits(q.shape[0], H, bt.shape[1], P)
                ws = nk.nvfp4_paged_decode_partial(q, kp, vp, bt, sl, wl.sm_scale, Sx, variant=var)
                out = torch.empty_like(q)
                nk.nvfp4kv_lse_merge(ws, q.shape[0], q.shape[1], d, Sx, vp.global_scale, out)
            torch.cuda.synchronize()
            check_out(out, ref, mass, f"{label} splits={S} variant={var}")
            outs.append(out)
    return outs, (kp, vp), (ref, mass)


# ---------------------------------------------------------------------------
# quantize-on-write
# ---------------------------------------------------------------------------

def test_quantize_tiny_workload(nk):
    wl = synth.WORKLOADS[1]
    say(f"case quantize tiny: {wl} seed {wl.seed}")
    inp = synth.host_uniform_decode(wl)
    kp, vp = gpu_quantize_nv(nk, inp.num_pages, 1, 16, 64, inp.k, inp.v, inp.slot_mapping)
    kd, ks, vd, vs = oracle_nv(inp.num_pages, 1, 16, 64, inp.k, inp.v, inp.slot_mapping)
    for t, r, n in ((kp.data, kd, "K data"), (kp.scale, ks, "K scale"), (vp.data, vd, "V data"),
                    (vp.scale, vs, "V scale")):
        assert_pool_equal(t, r, n)


def test_quantize_moderate_workload_with_outliers(nk):
    wl = synth.WORKLOADS[2]
    say(f"case quantize moderate: {wl} seed {wl.seed}")
    inp = synth.host_uniform_decode(wl)
    kp, vp = gpu_quantize_nv(nk, inp.num_pages, 8, 16, 128, inp.k, inp.v, inp.slot_mapping)
    kd, ks, vd, vs = oracle_nv(inp.num_pages, 8, 16, 128, inp.k, inp.v, inp.slot_mapping)
    for t, r, n in ((kp.data, kd, "K data"), (kp.scale, ks, "K scale"), (vp.data, vd, "V data"),
                    (vp.scale, vs, "V scale")):
        assert_pool_equal(t, r, n)


def _crafted_rows(rng, T, H, d):
    """bf16 rows mixing exact E2M1 midpoints, saturating values, tiny and huge
    magnitudes, negative zeros and every-bf16 sweeps."""
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    blocks = x.reshape(T, H, d // 16, 16)
    S = np.float32(2.0) ** rng.integers(-12, 8, size=blocks.shape[:3]).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, 0.5, 1, 1.5, 2, 3, 4, 6.375], np.float32)
    kind = rng.integers(0, 5, size=blocks.shape[:3])
    for idx in np.argwhere(kind == 0):                       # exact ties against S
        blocks[tuple(idx)] = rng.permutation(mids) * S[tuple(idx)] * rng.choice([-1, 1], 16)
    blocks[kind == 1] *= 1e-30                                 # scale underflows to 0
    blocks[kind == 2] *= 1e30                                  # scale saturates at 448
    blocks[kind == 3] = -0.0
    bits = synth.f32_to_bf16_bits(blocks.reshape(T, H, d))
    sweep = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    sweep = sweep[np.isfinite(synth.bf16_bits_to_f64(sweep))]
    n = min(sweep.size, bits.size // 2)
    flat = bits.reshape(-1)
    flat[:n] = rng.permutation(sweep)[:n]
    return flat.reshape(T, H, d)


GS_THIRD = float(np.float32(1.0 / 3.0))     # a calibrated (non-power-of-two) global scale


@pytest.mark.parametrize("gs", [1.0, 2.0, 0.5, GS_THIRD])
def test_quantize_crafted_values_and_skipped_slots(nk, gs):
    rng = np.random.default_rng(11)
    T, H, P, d, pages = 1536, 2, 32, 64, 64
    say(f"case quantize crafted: T {T} H {H} P {P} d {d} gs {gs}")
    with np.errstate(over="ignore", invalid="ignore"):
        k = _crafted_rows(rng, T, H, d)
        v = _crafted_rows(rng, T, H, d)
    slots = rng.permutation(pages * P)[:T].astype(np.int64)
    slots[rng.random(T) < 0.05] = -1                           # padding tokens
    outside = rng.random(T) < 0.02                             # slots past the pool are skipped too
    slots_gpu = slots.copy()
    slots_gpu[outside] = pages * P + rng.integers(0, 1 << 20, size=int(outside.sum()))
    slots[outside] = -1
    kp, vp = gpu_quantize_nv(nk, pages, H, P, d, k, v, slots_gpu, gs)
    kd, ks, vd, vs = oracle_nv(pages, H, P, d, k, v, slots, gs)
    for t, r, n in ((kp.data, kd, "K data"), (kp.scale, ks, "K scale"), (vp.data, vd, "V data"),
                    (vp.scale, vs, "V scale")):
        assert_pool_equal(t, r, n)


@pytest.mark.parametrize("gs", [1.0, GS_THIRD])
def test_quantize_non_finite_elements(nk, gs):
    """NaN (either sign) and +-inf elements among finite ones, against the FP32
    recipe (the documented arithmetic; at a power-of-two gs it equals the exact
    encode on finite inputs, which has no code for NaN): NaN is ignored by the
    block maximum and gets magnitude 0 with its sign bit, inf saturates the
    scale and its own code, the other elements of such blocks are encoded
    normally. Blocks without them take the quotient path at a power-of-two gs."""
    rng = np.random.default_rng(29)
    T, H, P, d, pages = 64, 2, 16, 128, 4
    say(f"case quantize non-finite: gs {gs}")
    bits = synth.host_values(rng, (T, H, d))
    flat = bits.reshape(-1)
    pos = rng.permutation(flat.size)[:300]
    specials = np.array([0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80], np.uint16)   # NaNs, +inf, -inf
    flat[pos] = specials[rng.integers(0, specials.size, pos.size)]
    slots = rng.permutation(pages * P)[:T].astype(np.int64)
    kp, _ = gpu_quantize_nv(nk, pages, H, P, d, bits, bits, slots, gs)
    with np.errstate(invalid="ignore", over="ignore"):
        codes, s = onv.encode_blocks_fp32(onv.bf16_to_f64(bits).reshape(T, H, d // 16, 16), gs)
    data = onv.pack_nibbles(codes.reshape(T, H, d))
    kd, ks = onv.empty_cache(pages, H, P, d, fill=SENT)
    kd[slots // P, :, slots % P] = data
    ks[slots // P, :, slots % P] = s
    assert_pool_equal(kp.data, kd, "K data")
    assert_pool_equal(kp.scale, ks, "K scale")


@pytest.mark.parametrize("gs", [1.0, 0.125])
def test_quantize_every_value_under_every_scale(nk, gs):
    """Every E4M3 block scale S (0x01..0x7E) with every finite bf16 magnitude up
    to 6*S*gs, both signs: each block holds an anchor 6*S*gs (which fixes the
    scale byte) and 15 of the values; about 4.3M elements through the library's
    quantize, bit-exact against the oracle."""
    rng = np.random.default_rng(37)
    pos = np.arange(1, 0x7F80, dtype=np.uint32)
    mags = synth.bf16_bits_to_f64(pos.astype(np.uint16))
    blocks = []
    for b in range(1, 0x7F):
        s = float(onv.E4M3_VALUES[b]) * gs
        vals = pos[mags <= 6.0 * s].astype(np.uint16)
        vals = np.concatenate([vals, vals | 0x8000])
        vals = rng.permutation(vals)
        n = -(-vals.size // 15)
        vals = np.resize(vals, n * 15).reshape(n, 15)
        anc = synth.f32_to_bf16_bits(np.array([6.0 * s], np.float32))[0]
        blk = np.empty((n, 16), np.uint16)
        blk[:, :15] = vals
        blk[:, 15] = anc
        idx, k = np.arange(n), np.arange(n) % 16                   # the anchor at a varying position
        moved = blk[idx, k].copy()
        blk[idx, k] = anc
        blk[:, 15] = np.where(k == 15, anc, moved)
        blocks.append(blk)
    blocks = np.concatenate(blocks)
    d = 128
    T = -(-blocks.shape[0] // (d // 16))
    rows = np.zeros((T * (d // 16), 16), np.uint16)
    rows[:blocks.shape[0]] = blocks
    bits = rows.reshape(T, 1, d)
    P = 16
    pages = -(-T // P)
    say(f"case quantize every value under every scale: gs {gs}, {blocks.shape[0]} blocks, {T} tokens")
    slots = rng.permutation(pages * P)[:T].astype(np.int64)
    kp, _ = gpu_quantize_nv(nk, pages, 1, P, d, bits, bits, slots, gs)
    kd, ks, _, _ = oracle_nv(pages, 1, P, d, bits, bits, slots, gs)
    assert_pool_equal(kp.scale, ks, "K scale")
    assert_pool_equal(kp.data, kd, "K data")


def test_quantize_golden_blocks(nk):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_block_vectors.txt")
    rows = []
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        rows.append([float(t) for t in line.split("|")[1].split()])
    x = np.zeros((1, 1, 128), np.float32)
    blocks = np.array(rows, np.float32)[:8]
    x[0, 0, :16 * len(blocks)] = blocks.reshape(-1)
    bits = synth.f32_to_bf16_bits(x)
    say("case quantize golden blocks")
    kp, vp = gpu_quantize_nv(nk, 1, 1, 16, 128, bits, bits, np.array([3], np.int64))
    kd, ks, _, _ = oracle_nv(1, 1, 16, 128, bits, bits, np.array([3], np.int64))
    assert_pool_equal(kp.data, kd, "golden data")
    assert_pool_equal(kp.scale, ks, "golden scale")


def test_quantize_strided_source(nk):
    """K and V read out of a fused [T][3][Hkv][d] buffer (token stride 3*Hkv*d)."""
    rng = np.random.default_rng(12)
    T, H, P, d, pages = 200, 4, 16, 128, 16
    say(f"case quantize strided: T {T} H {H} d {d}")
    qkv = synth.f32_to_bf16_bits(rng.standard_normal((T, 3, H, d)).astype(np.float32))
    slots = rng.permutation(pages * P)[:T].astype(np.int64)
    dev = synth.to_device_bf16(qkv)
    kt, vt = dev[:, 1], dev[:, 2]
    kp, vp = gpu_quantize_nv(nk, pages, H, P, d, None, None, slots, kt=kt, vt=vt)
    kd, ks, vd, vs = oracle_nv(pages, H, P, d, qkv[:, 1].copy(), qkv[:, 2].copy(), slots)
    assert_pool_equal(kp.data, kd, "K data")
    assert_pool_equal(vp.scale, vs, "V scale")


def test_fp8_quantize_every_bf16_value(nk):
    rng = np.random.default_rng(13)
    sweep = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    sweep = sweep[np.isfinite(synth.bf16_bits_to_f64(sweep))]
    H, P, d = 1, 16, 64
    T = -(-sweep.size // d)
    pad = np.zeros(T * d, np.uint16)
    pad[:sweep.size] = rng.permutation(sweep)
    k = pad.reshape(T, H, d)
    v = k[::-1].copy()
    pages = -(-T // P)
    slots = np.arange(T, dtype=np.int64)
    say(f"case fp8 quantize sweep: T {T}")
    kp, vp = f8_pools(nk, pages, H, P, d)
    nk.fp8_kv_quantize(synth.to_device_bf16(k), synth.to_device_bf16(v), synth.to_device(slots), kp, vp)
    torch.cuda.synchronize()
    kr = np.full((pages, H, P, d), SENT, np.uint8)
    vr = np.full((pages, H, P, d), SENT, np.uint8)
    of8.write_cache(kr, k, slots)
    of8.write_cache(vr, v, slots)
    assert_pool_equal(kp.data, kr, "fp8 K")
    assert_pool_equal(vp.data, vr, "fp8 V")


# ---------------------------------------------------------------------------
# dequantize-to-workspace
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(8, 128, 16, 1.0), (1, 64, 16, 1.0), (3, 64, 32, 1.0), (8, 128, 16, GS_THIRD),
                                   (2, 128, 48, 1.0)])
def test_dequant_workspace_agentic_small(nk, shape):
    H0, d0, P0, gs = shape
    wl = synth.Workload(95, "ws", 7, 2 * H0, H0, d0, P0, 0, False, 0, len_min=48, len_max=131,
                        shared_prefix=max(32, P0), chunk=9)   # the shared prefix is whole pages
    a = synth.host_agentic(wl)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    say(f"case workspace small agentic: B 7 pages {a.num_pages} gs {gs}")
    kp, vp = gpu_quantize_nv(nk, a.num_pages, H, P, d, a.k_cached, a.v_cached, a.slot_cached, gs)
    kd, ks, vd, vs = oracle_nv(a.num_pages, H, P, d, a.k_cached, a.v_cached, a.slot_cached, gs)
    prefix = a.cached_lens.copy()
    prefix[3] = 0                                         # an empty prefix
    prefix[5] = 17                                        # a ragged partial page
    rows = int(a.ws_row_offsets[-1])
    kws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
    vws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
    nk.nvfp4_kv_dequant_workspace(kp, vp, synth.to_device(a.block_tables), synth.to_device(prefix),
                                  synth.to_device(a.ws_row_offsets), kws, vws)
    torch.cuda.synchronize()
    fill = int(synth.bf16_tensor_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0])
    kref = oatt.dequant_workspace(onv.dequant_cache(kd, ks, gs), a.block_tables, prefix, a.ws_row_offsets, rows, fill,
                                  cache_bits=onv.workspace_bits(kd, ks, gs))
    vref = oatt.dequant_workspace(onv.dequant_cache(vd, vs, gs), a.block_tables, prefix, a.ws_row_offsets, rows, fill,
                                  cache_bits=onv.workspace_bits(vd, vs, gs))
    assert np.array_equal(synth.bf16_tensor_bits(kws), kref)
    assert np.array_equal(synth.bf16_tensor_bits(vws), vref)


@pytest.mark.parametrize("case", range(6))
def test_quantize_and_workspace_randomized(nk, case):
    """Seeded random geometries (KV heads, head_dim, page size), tokens written
    to a random permutation of slots with some skipped (negative or past the
    pool), then ragged prefixes dequantized through block tables whose
    leading pages are sometimes shared: pool bytes and workspace bits exact,
    untouched bytes and spare rows unchanged."""
    rng = np.random.default_rng(6161 + case)
    H = int(rng.choice([1, 2, 3, 5]))
    d = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 48, 64]))
    B = int(rng.integers(1, 6))
    gs = [1.0, 0.25, GS_THIRD][case % 3]
    lens = rng.integers(0, 400, B).astype(np.int32)
    pages_per = max(1, int(-(-lens.max() // P)))
    num_pages = B * pages_per + int(rng.integers(0, 4))
    bt = rng.permutation(num_pages)[:B * pages_per].astype(np.int32).reshape(B, pages_per)
    if B > 1 and case % 2 == 0:                        # sequence 1 shares sequence 0's first page(s)
        k = int(rng.integers(1, pages_per + 1))
        bt[1, :k] = bt[0, :k]
    toks = [(b, t) for b in range(B) for t in range(int(lens[b]))
            if not (B > 1 and case % 2 == 0 and b == 1 and t < k * P)]   # shared pages are written once
    T = len(toks)
    slots = np.array([int(bt[b, t // P]) * P + t % P for b, t in toks], np.int64)
    extra = np.array([-1, -5, num_pages * P, num_pages * P + 3], np.int64)  # skipped slots
    kb = synth.host_values(rng, (T + 4, H, d))
    vb = synth.host_values(rng, (T + 4, H, d))
    all_slots = np.concatenate([slots, extra])
    order = rng.permutation(T + 4)
    say(f"case quantize+workspace random {case}: H {H} d {d} P {P} B {B} gs {gs} lens {lens.tolist()} pages {num_pages}")
    kp, vp = gpu_quantize_nv(nk, num_pages, H, P, d, kb[order], vb[order], all_slots[order], gs)
    kd, ks, vd, vs = oracle_nv(num_pages, H, P, d, kb[order], vb[order], all_slots[order], gs)
    assert_pool_equal(kp.data, kd, "K data")
    assert_pool_equal(kp.scale, ks, "K scale")
    assert_pool_equal(vp.data, vd, "V data")
    assert_pool_equal(vp.scale, vs, "V scale")
    prefix = np.array([int(rng.integers(0, n + 1)) for n in lens], np.int32)
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(lens + rng.integers(0, 4, B))
    rows = max(1, int(ws_offs[-1]))
    kws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
    vws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
    nk.nvfp4_kv_dequant_workspace(kp, vp, synth.to_device(bt), synth.to_device(prefix), synth.to_device(ws_offs),
                                  kws, vws)
    torch.cuda.synchronize()
    fill = int(synth.bf16_tensor_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0])
    kref = oatt.dequant_workspace(onv.dequant_cache(kd, ks, gs), bt, prefix, ws_offs, rows, fill,
                                  cache_bits=onv.workspace_bits(kd, ks, gs))
    vref = oatt.dequant_workspace(onv.dequant_cache(vd, vs, gs), bt, prefix, ws_offs, rows, fill,
                                  cache_bits=onv.workspace_bits(vd, vs, gs))
    assert np.array_equal(synth.bf16_tensor_bits(kws), kref)
    assert np.array_equal(synth.bf16_tensor_bits(vws), vref)


@pytest.mark.parametrize("fp8_ws", [False, True])
def test_dequant_workspace_every_scale_byte(nk, fp8_ws):
    """Pools written directly with every finite E4M3 scale byte (both signs,
    subnormals included) against random data bytes (every nibble), read back
    through the page table into the bf16 or the FP8 workspace; bit-exact
    against the oracle."""
    rng = np.random.default_rng(23)
    H, P, d, pages = 2, 16, 128, 40
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    say(f"case workspace every scale byte: fp8 {fp8_ws}")
    pools, ref_bytes = [], []
    for _ in range(2):
        data = rng.integers(0, 256, size=(pages, H, P, d // 2)).astype(np.uint8)
        scale = np.resize(rng.permutation(finite), pages * H * P * (d // 16)).reshape(pages, H, P, d // 16)
        pool = nk.NVFP4Pool.empty(pages, H, P, d)
        pool.data.copy_(torch.from_numpy(data))
        pool.scale.copy_(torch.from_numpy(scale))
        pools.append(pool)
        ref_bytes.append((data, scale))
    B = 3
    prefix = np.array([pages * P // 2, 37, pages * P // 2 - 37], np.int32)
    bt = rng.permutation(pages).astype(np.int32)
    tables = np.zeros((B, pages), np.int32)
    tables[0, :pages // 2] = bt[:pages // 2]
    tables[1, :3] = bt[pages // 2:pages // 2 + 3]
    tables[2, :pages // 2] = bt[pages // 2:]
    offs = np.zeros(B + 1, np.int64)
    offs[1:] = np.cumsum(prefix + 5)
    rows = int(offs[-1])
    if fp8_ws:
        kws = torch.full((rows, H, d), 0xA5, dtype=torch.uint8, device="cuda")
        vws = torch.full((rows, H, d), 0xA5, dtype=torch.uint8, device="cuda")
        nk.nvfp4_kv_dequant_workspace_fp8(pools[0], pools[1], synth.to_device(tables), synth.to_device(prefix),
                                          synth.to_device(offs), kws, vws)
    else:
        kws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
        vws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
        nk.nvfp4_kv_dequant_workspace(pools[0], pools[1], synth.to_device(tables), synth.to_device(prefix),
                                      synth.to_device(offs), kws, vws)
    torch.cuda.synchronize()
    for ws_t, (data, scale) in ((kws, ref_bytes[0]), (vws, ref_bytes[1])):
        if fp8_ws:
            cache = onv.workspace_fp8_bytes(data, scale, 1.0, 1.0)
            ref = np.full((rows, H, d), 0xA5, np.uint8)
            got = ws_t.cpu().numpy()
        else:
            cache = onv.workspace_bits(data, scale, 1.0)
            ref = np.full((rows, H, d), int(synth.bf16_tensor_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0]),
                          np.uint16)
            got = synth.bf16_tensor_bits(ws_t)
        for b in range(B):
            n, off = int(prefix[b]), int(offs[b])
            ref[off:off + n] = oatt.gather_tokens(cache, tables[b], n)
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)
            i = tuple(bad[0])
            raise AssertionError(f"{len(bad)} workspace elements differ; first at {i}: gpu {got[i]:#x} oracle {ref[i]:#x}")


def _fp8_bytes(rng, shape):
    """Random FP8-E4M3 bytes over the whole finite range (NaN bytes replaced)."""
    b = rng.integers(0, 256, size=shape).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x3A
    return b


@pytest.mark.parametrize("src_scale,gs", [(1.0, 1.0), (1.0, GS_THIRD), (0.37, 1.0)])
def test_quantize_fp8_source_and_fused_chunk_copy(nk, src_scale, gs):
    """The pages' path-2 types: FP8 K/V (strided, fused-QKV-like source) are
    quantized to NVFP4 bit-exactly against the oracle, and in the same pass
    copied unchanged into FP8 workspace rows (rows < 0 not copied)."""
    rng = np.random.default_rng(41)
    T, H, d, P, pages = 150, 2, 128, 16, 24
    say(f"case quantize fp8 source: T {T} src_scale {src_scale} gs {gs}")
    kb, vb = _fp8_bytes(rng, (T, H, d)), _fp8_bytes(rng, (T, H, d))
    kb[:4, 0, :16] = 0                                                    # zero blocks
    kb[4, 1, :16] = 0x80                                                  # -0.0 block
    slots = rng.permutation(pages * P)[:T].astype(np.int64)
    slots[7] = -1
    rows = rng.permutation(T + 20)[:T].astype(np.int64)
    rows[11] = -5
    wide = np.zeros((T, 3 * H, d), np.uint8)                              # token stride 3 * H * d bytes
    wide[:, :H], wide[:, H:2 * H] = kb, vb
    wt = torch.from_numpy(wide).cuda()
    kt, vt = wt[:, :H], wt[:, H:2 * H]
    kp, vp = nv_pools(nk, pages, H, P, d, gs)
    kws = torch.full((T + 20, H, d), SENT, dtype=torch.uint8, device="cuda")
    vws = torch.full((T + 20, H, d), SENT, dtype=torch.uint8, device="cuda")
    nk.nvfp4_kv_quantize_fp8(kt, vt, synth.to_device(slots), kp, vp, src_scale, src_scale,
                             synth.to_device(rows), kws, vws)
    torch.cuda.synchronize()
    kd, ks = onv.empty_cache(pages, H, P, d, fill=SENT)
    vd, vs = onv.empty_cache(pages, H, P, d, fill=SENT)
    keep = slots >= 0
    for (dd, ss), x in (((kd, ks), kb), ((vd, vs), vb)):
        rd, rs = onv.quantize_rows_fp8(x, src_scale, gs)
        dd[slots[keep] // P, :, slots[keep] % P] = rd[keep]
        ss[slots[keep] // P, :, slots[keep] % P] = rs[keep]
    assert_pool_equal(kp.data, kd, "fp8-source K data")
    assert_pool_equal(kp.scale, ks, "fp8-source K scale")
    assert_pool_equal(vp.data, vd, "fp8-source V data")
    assert_pool_equal(vp.scale, vs, "fp8-source V scale")
    for ws_t, x in ((kws, kb), (vws, vb)):
        ref = np.full((T + 20, H, d), SENT, np.uint8)
        ok = rows >= 0
        ref[rows[ok]] = x[ok]
        assert_pool_equal(ws_t, ref, "fused chunk copy")


@pytest.mark.parametrize("gs,ws_scale", [(1.0, 1.0), (GS_THIRD, 1.0), (1.0, 0.5), (1.0, 0.3)])
def test_dequant_workspace_fp8(nk, gs, ws_scale):
    """The pages' FP8 workspace: bytes bit-exact against the oracle's E4M3
    rounding of the dequantized prefix; rows past each prefix untouched."""
    wl = synth.Workload(97, "wsfp8", 7, 16, 8, 128, 16, 0, False, 0, len_min=48, len_max=131,
                        shared_prefix=32, chunk=9)
    a = synth.host_agentic(wl)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    say(f"case fp8 workspace: gs {gs} ws_scale {ws_scale}")
    kp, vp = gpu_quantize_nv(nk, a.num_pages, H, P, d, a.k_cached, a.v_cached, a.slot_cached, gs)
    kd, ks, vd, vs = oracle_nv(a.num_pages, H, P, d, a.k_cached, a.v_cached, a.slot_cached, gs)
    prefix = a.cached_lens.copy()
    prefix[2] = 0
    rows = int(a.ws_row_offsets[-1])
    kws = torch.full((rows, H, d), SENT, dtype=torch.uint8, device="cuda")
    vws = torch.full((rows, H, d), SENT, dtype=torch.uint8, device="cuda")
    nk.nvfp4_kv_dequant_workspace_fp8(kp, vp, synth.to_device(a.block_tables), synth.to_device(prefix),
                                      synth.to_device(a.ws_row_offsets), kws, vws, ws_scale, ws_scale)
    torch.cuda.synchronize()
    for ws_t, (dd, ss) in ((kws, (kd, ks)), (vws, (vd, vs))):
        cache_b = onv.workspace_fp8_bytes(dd, ss, gs, ws_scale)
        ref = np.full((rows, H, d), SENT, np.uint8)
        for b in range(len(prefix)):
            n, off = int(prefix[b]), int(a.ws_row_offsets[b])
            ref[off:off + n] = oatt.gather_tokens(cache_b, a.block_tables[b], n)
        assert_pool_equal(ws_t, ref, "fp8 workspace")


@pytest.mark.parametrize("G,Hkv,d,P", [(4, 2, 128, 16), (1, 2, 64, 32), (8, 1, 128, 16), (16, 1, 64, 16)])
def test_extend_attention_over_workspace(nk, G, Hkv, d, P):
    """Path 2 end to end at a small size: the prefix is quantized into the
    pool and dequantized into the bf16 workspace by the library, the chunk's
    K/V follow it in the workspace, and the chunk's queries attend (causally
    within the chunk) through nvfp4_extend_attn; against the oracle. Ragged
    chunks, an empty prefix, a one-token chunk and an empty chunk included."""
    rng = np.random.default_rng(42)
    B = 6
    prefix = np.array([37, 0, 120, 64, 5, 90], np.int32)
    chunk = np.array([33, 17, 1, 48, 0, 40], np.int32)
    Hq = G * Hkv
    say(f"case extend attention: G {G} Hkv {Hkv} d {d} P {P}")
    pages_per = -(-(prefix + chunk).max() // P)
    num_pages = B * pages_per
    bt = rng.permutation(num_pages).astype(np.int32).reshape(B, pages_per)
    kb = synth.host_values(rng, (int(prefix.sum()), Hkv, d))
    vb = synth.host_values(rng, (int(prefix.sum()), Hkv, d))
    slots = np.concatenate([bt[b, np.arange(prefix[b]) // P].astype(np.int64) * P + np.arange(prefix[b]) % P
                            for b in range(B)])
    kp, vp = gpu_quantize_nv(nk, num_pages, Hkv, P, d, kb, vb, slots)
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(prefix + chunk + 3)                  # 3 spare rows per sequence
    rows = int(ws_offs[-1])
    kws = torch.zeros((rows, Hkv, d), dtype=torch.bfloat16, device="cuda")
    vws = torch.zeros((rows, Hkv, d), dtype=torch.bfloat16, device="cuda")
    nk.nvfp4_kv_dequant_workspace(kp, vp, synth.to_device(bt), synth.to_device(prefix), synth.to_device(ws_offs),
                                  kws, vws)
    # the chunk's own K/V go to the rows after each prefix
    kc = synth.host_values(rng, (int(chunk.sum()), Hkv, d))
    vc = synth.host_values(rng, (int(chunk.sum()), Hkv, d))
    crow = np.concatenate([ws_offs[b] + prefix[b] + np.arange(chunk[b]) for b in range(B)]).astype(np.int64)
    idx = torch.from_numpy(crow).cuda()
    kws[idx] = synth.to_device_bf16(kc)
    vws[idx] = synth.to_device_bf16(vc)
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    qb = synth.host_values(rng, (int(chunk.sum()), Hq, d))
    sm = 1.0 / math.sqrt(d)
    out = nk.nvfp4_extend_attn(synth.to_device_bf16(qb), synth.to_device(q_offs), kws, vws, synth.to_device(ws_offs),
                               synth.to_device(prefix), sm, max_chunk=int(chunk.max()) + 5)
    torch.cuda.synchronize()
    kw = synth.bf16_bits_to_f64(synth.bf16_tensor_bits(kws))
    vw = synth.bf16_bits_to_f64(synth.bf16_tensor_bits(vws))
    ref, mass = oatt.extend_attention(synth.bf16_bits_to_f64(qb), kw, vw, q_offs, ws_offs, prefix, sm)
    check_out(out, ref, mass, f"extend G{G} d{d}")


@pytest.mark.parametrize("G,d,sm_sign", [(4, 128, 1.0), (2, 64, -1.0), (16, 128, -1.0), (1, 128, 1.0)])
def test_extend_attention_long_prefix(nk, G, d, sm_sign):
    """Prefixes spanning many 64-key blocks and chunks spanning several query
    blocks of one KV head, with key magnitudes that grow along each sequence so
    that the running max of most queries rises many times over the keys; a
    negative logit scale included. The workspace is filled directly; against
    the oracle."""
    rng = np.random.default_rng(7)
    Hkv = 2
    Hq = G * Hkv
    prefix = np.array([700, 0, 1290], np.int32)
    chunk = np.array([150, 203, 75], np.int32)
    B = len(prefix)
    say(f"case extend long prefix: G {G} d {d} sm sign {sm_sign:+.0f}")
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(prefix + chunk)
    rows = int(ws_offs[-1])
    gain = np.concatenate([0.5 + 5.5 * np.arange(n) / n for n in prefix + chunk])
    kx = rng.standard_normal((rows, Hkv, d)) * gain[:, None, None]
    kb = synth.f32_to_bf16_bits(kx.astype(np.float32))
    vb = synth.host_values(rng, (rows, Hkv, d))
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    qb = synth.host_values(rng, (int(chunk.sum()), Hq, d))
    sm = sm_sign / math.sqrt(d)
    out = nk.nvfp4_extend_attn(synth.to_device_bf16(qb), synth.to_device(q_offs), synth.to_device_bf16(kb),
                               synth.to_device_bf16(vb), synth.to_device(ws_offs), synth.to_device(prefix), sm)
    torch.cuda.synchronize()
    ref, mass = oatt.extend_attention(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                      synth.bf16_bits_to_f64(vb), q_offs, ws_offs, prefix, sm)
    check_out(out, ref, mass, f"extend long G{G} d{d} sm{sm:+.3f}")


def test_extend_attention_negative_prefix_is_empty(nk):
    """A negative prefix length is taken as an empty prefix: the chunk's
    queries attend causally to the chunk alone, read from the rows at the
    sequence's workspace offset; against the oracle with prefix 0."""
    rng = np.random.default_rng(8)
    G, Hkv, d = 4, 2, 128
    chunk = np.array([70, 33], np.int32)
    prefix = np.array([-5, -100000], np.int32)
    B = len(chunk)
    say(f"case extend negative prefix: prefix {prefix.tolist()} chunk {chunk.tolist()}")
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(chunk + 2)
    rows = int(ws_offs[-1])
    kb = synth.host_values(rng, (rows, Hkv, d))
    vb = synth.host_values(rng, (rows, Hkv, d))
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    qb = synth.host_values(rng, (int(chunk.sum()), G * Hkv, d))
    sm = 1.0 / math.sqrt(d)
    out = nk.nvfp4_extend_attn(synth.to_device_bf16(qb), synth.to_device(q_offs), synth.to_device_bf16(kb),
                               synth.to_device_bf16(vb), synth.to_device(ws_offs), synth.to_device(prefix), sm)
    torch.cuda.synchronize()
    ref, mass = oatt.extend_attention(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                      synth.bf16_bits_to_f64(vb), q_offs, ws_offs, np.zeros(B, np.int32), sm)
    check_out(out, ref, mass, "extend negative prefix")


@pytest.mark.parametrize("case", range(8))
def test_extend_attention_randomized(nk, case):
    """Seeded random extend problems: batch, query group, KV heads, head_dim,
    ragged prefixes and chunks (zeros included), spare workspace rows between
    sequences, a max_chunk above the longest chunk and either sign of the logit
    scale; against the oracle."""
    rng = np.random.default_rng(5151 + case)
    B = int(rng.integers(1, 6))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 3]))
    d = int(rng.choice([64, 128]))
    Hq = G * Hkv
    prefix = rng.integers(0, 701, B).astype(np.int32)
    chunk = rng.integers(0, 261, B).astype(np.int32)
    full = int(rng.integers(0, B))
    chunk[full] = int(rng.integers(1, 261))                     # at least one query
    if case % 2 == 0:
        prefix[0] = 0                                           # an empty prefix
    if B > 1 and case % 3 == 0:
        chunk[(full + 1) % B] = 0                               # an empty chunk
    spare = rng.integers(0, 6, B)
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(prefix + chunk + spare)
    rows = int(ws_offs[-1])
    sm = float(rng.choice([1.0, -1.0])) / math.sqrt(d)
    say(f"case extend random {case}: B {B} G {G} Hkv {Hkv} d {d} prefix {prefix.tolist()} chunk {chunk.tolist()} "
        f"sm {sm:+.3f}")
    kb = synth.host_values(rng, (rows, Hkv, d))
    vb = synth.host_values(rng, (rows, Hkv, d))
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    qb = synth.host_values(rng, (int(chunk.sum()), Hq, d))
    out = nk.nvfp4_extend_attn(synth.to_device_bf16(qb), synth.to_device(q_offs), synth.to_device_bf16(kb),
                               synth.to_device_bf16(vb), synth.to_device(ws_offs), synth.to_device(prefix), sm,
                               max_chunk=int(chunk.max()) + int(rng.integers(0, 40)))
    torch.cuda.synchronize()
    ref, mass = oatt.extend_attention(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                      synth.bf16_bits_to_f64(vb), q_offs, ws_offs, prefix, sm)
    check_out(out, ref, mass, f"extend random {case}")


@pytest.mark.parametrize("B", [9, 37, 64, 70])
def test_extend_attention_many_sequences(nk, B):
    """Batches around the 64-sequence limit of the longest-first workgroup
    order (above it the natural order): ragged prefixes and chunks with ties
    and empty chunks; every query against the oracle, for both workspace
    types."""
    rng = np.random.default_rng(9100 + B)
    G, Hkv, d = 4, 2, 64
    prefix = rng.integers(0, 260, B).astype(np.int32)
    chunk = rng.integers(0, 40, B).astype(np.int32)
    chunk[::7] = 0                                            # empty chunks
    prefix[1::5] = prefix[0]                                  # equal work for several sequences
    chunk[1::5] = chunk[0]
    chunk[2] = max(int(chunk[2]), 1)
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(prefix + chunk + 1)
    rows = int(ws_offs[-1])
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    say(f"case extend many sequences: B {B}, {int(chunk.sum())} queries")
    qb = synth.host_values(rng, (int(chunk.sum()), G * Hkv, d))
    kb = synth.host_values(rng, (rows, Hkv, d))
    vb = synth.host_values(rng, (rows, Hkv, d))
    sm = 1.0 / math.sqrt(d)
    out = nk.nvfp4_extend_attn(synth.to_device_bf16(qb), synth.to_device(q_offs), synth.to_device_bf16(kb),
                               synth.to_device_bf16(vb), synth.to_device(ws_offs), synth.to_device(prefix), sm)
    k8, v8 = _fp8_bytes(rng, (rows, Hkv, d)), _fp8_bytes(rng, (rows, Hkv, d))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out8 = nk.nvfp4_extend_attn_fp8(synth.to_device_bf16(qb), synth.to_device(q_offs), dev(k8), dev(v8),
                                    synth.to_device(ws_offs), synth.to_device(prefix), sm, 1.0 / 64, 0.5)
    torch.cuda.synchronize()
    q64 = synth.bf16_bits_to_f64(qb)
    ref, mass = oatt.extend_attention(q64, synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb), q_offs, ws_offs,
                                      prefix, sm)
    check_out(out, ref, mass, f"extend B{B}")
    ref8, mass8 = oatt.extend_attention(q64, _e4m3_f64(k8, 1.0 / 64), _e4m3_f64(v8, 0.5), q_offs, ws_offs, prefix, sm)
    check_out(out8, ref8, mass8, f"extend fp8 B{B}")


def _e4m3_f64(b, scale):
    """Workspace bytes -> float64 values e4m3(byte) * scale (the oracle's E4M3 table)."""
    return onv.E4M3_VALUES[np.asarray(b, dtype=np.int64)] * float(scale)


@pytest.mark.parametrize("G,Hkv,d,P,scale", [(4, 2, 128, 16, 1.0), (1, 2, 64, 32, 0.5), (8, 1, 128, 16, 0.37),
                                             (16, 1, 64, 16, 1.0), (16, 2, 128, 16, 0.5), (8, 3, 64, 64, 2.0)])
def test_extend_fp8_path2_end_to_end(nk, G, Hkv, d, P, scale):
    """The pages' path 2 in its own types at a small size: FP8 K/V of earlier
    turns quantized into the NVFP4 pool, the cached prefix dequantized into the
    FP8 workspace, the current chunk quantized into the pool and copied into the
    workspace in the same pass, then the chunk's queries attend through
    nvfp4_extend_attn_fp8 with the workspace scale as K and V tensor scale.
    Workspace bytes bit-exact against the oracle; the output against the
    oracle's attention over the oracle's workspace values. Ragged chunks, an
    empty prefix, a one-token and an empty chunk."""
    rng = np.random.default_rng(4242)
    prefix = np.array([37, 0, 120, 64, 5, 90], np.int32)
    chunk = np.array([33, 17, 1, 48, 0, 40], np.int32)
    B, Hq = len(prefix), G * Hkv
    say(f"case extend fp8 path 2: G {G} Hkv {Hkv} d {d} P {P} scale {scale}")
    pages_per = -(-(prefix + chunk).max() // P)
    num_pages = B * pages_per
    bt = rng.permutation(num_pages).astype(np.int32).reshape(B, pages_per)
    pos_p = [np.arange(prefix[b]) for b in range(B)]
    pos_c = [prefix[b] + np.arange(chunk[b]) for b in range(B)]
    slot = lambda b, t: bt[b, t // P].astype(np.int64) * P + t % P
    slots_p = np.concatenate([slot(b, pos_p[b]) for b in range(B)])
    slots_c = np.concatenate([slot(b, pos_c[b]) for b in range(B)])
    kp_src, vp_src = _fp8_bytes(rng, (len(slots_p), Hkv, d)), _fp8_bytes(rng, (len(slots_p), Hkv, d))
    kc_src, vc_src = _fp8_bytes(rng, (len(slots_c), Hkv, d)), _fp8_bytes(rng, (len(slots_c), Hkv, d))
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(prefix + chunk + 3)                  # 3 spare rows per sequence
    rows = int(ws_offs[-1])
    crow = np.concatenate([ws_offs[b] + pos_c[b] for b in range(B)]).astype(np.int64)
    # library side
    kp, vp = nv_pools(nk, num_pages, Hkv, P, d)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    nk.nvfp4_kv_quantize_fp8(dev(kp_src), dev(vp_src), synth.to_device(slots_p), kp, vp, scale, scale)
    kws = torch.zeros((rows, Hkv, d), dtype=torch.uint8, device="cuda")
    vws = torch.zeros((rows, Hkv, d), dtype=torch.uint8, device="cuda")
    nk.nvfp4_kv_dequant_workspace_fp8(kp, vp, synth.to_device(bt), synth.to_device(prefix), synth.to_device(ws_offs),
                                      kws, vws, scale, scale)
    nk.nvfp4_kv_quantize_fp8(dev(kc_src), dev(vc_src), synth.to_device(slots_c), kp, vp, scale, scale,
                             synth.to_device(crow), kws, vws)
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    qb = synth.host_values(rng, (int(chunk.sum()), Hq, d))
    sm = 1.0 / math.sqrt(d)
    out = nk.nvfp4_extend_attn_fp8(synth.to_device_bf16(qb), synth.to_device(q_offs), kws, vws,
                                   synth.to_device(ws_offs), synth.to_device(prefix), sm, scale, scale,
                                   max_chunk=int(chunk.max()) + 5)
    torch.cuda.synchronize()
    # oracle side: the pool of the prefix, its FP8 workspace rows, the chunk's source bytes after them
    ref_ws = []
    for src in (kp_src, vp_src):
        dd, ss = onv.empty_cache(num_pages, Hkv, P, d, fill=0)
        rd, rs = onv.quantize_rows_fp8(src, scale, 1.0)
        dd[slots_p // P, :, slots_p % P] = rd
        ss[slots_p // P, :, slots_p % P] = rs
        cache_b = onv.workspace_fp8_bytes(dd, ss, 1.0, scale)
        ws = np.zeros((rows, Hkv, d), np.uint8)
        for b in range(B):
            ws[ws_offs[b]:ws_offs[b] + prefix[b]] = oatt.gather_tokens(cache_b, bt[b], int(prefix[b]))
        ref_ws.append(ws)
    ref_ws[0][crow], ref_ws[1][crow] = kc_src, vc_src
    assert_pool_equal(kws, ref_ws[0], "fp8 K workspace")
    assert_pool_equal(vws, ref_ws[1], "fp8 V workspace")
    ref, mass = oatt.extend_attention(synth.bf16_bits_to_f64(qb), _e4m3_f64(ref_ws[0], scale),
                                      _e4m3_f64(ref_ws[1], scale), q_offs, ws_offs, prefix, sm)
    check_out(out, ref, mass, f"extend fp8 G{G} d{d} scale {scale}")


@pytest.mark.parametrize("v_scale", [1.0, 0.125])
def test_extend_fp8_every_value_byte(nk, v_scale):
    """A query that sees one key returns that key's value row: with the value
    rows holding every finite E4M3 byte, the output is each E4M3 value times a
    power-of-two scale, exactly (the conversion to bf16 is exact)."""
    d, Hkv, G = 128, 1, 1
    vals = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    vals = np.concatenate([vals, np.zeros(2 * d - len(vals), np.uint8)])
    B = 2
    say(f"case extend fp8 every value byte: v_scale {v_scale}")
    prefix = np.zeros(B, np.int32)
    ws_offs = np.arange(B + 1, dtype=np.int64)
    q_offs = np.arange(B + 1, dtype=np.int64)
    vb = vals.reshape(B, Hkv, d)
    kb = np.full((B, Hkv, d), 0x38, np.uint8)                    # keys of 1.0
    qb = synth.host_values(np.random.default_rng(3), (B, G * Hkv, d))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = nk.nvfp4_extend_attn_fp8(synth.to_device_bf16(qb), synth.to_device(q_offs), dev(kb), dev(vb),
                                   synth.to_device(ws_offs), synth.to_device(prefix), 0.09, 0.75, v_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want = onv.E4M3_VALUES[vb.astype(np.int64)] * v_scale
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} values differ; first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs " \
                          f"{want[tuple(bad[0])]}"


@pytest.mark.parametrize("case", range(6))
def test_extend_fp8_randomized(nk, case):
    """Seeded random extend problems over FP8 workspaces filled directly with
    random finite E4M3 bytes: batch, query group, KV heads, head_dim, ragged
    prefixes to 1,000 keys and chunks (zeros included), spare rows, K and V
    tensor scales, either sign of the logit scale; against the oracle."""
    rng = np.random.default_rng(6161 + case)
    B = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 3]))
    d = int(rng.choice([64, 128]))
    Hq = G * Hkv
    prefix = rng.integers(0, 1001, B).astype(np.int32)
    chunk = rng.integers(0, 201, B).astype(np.int32)
    full = int(rng.integers(0, B))
    chunk[full] = int(rng.integers(1, 201))
    if case % 2 == 0:
        prefix[0] = 0
    spare = rng.integers(0, 6, B)
    ws_offs = np.zeros(B + 1, np.int64)
    ws_offs[1:] = np.cumsum(prefix + chunk + spare)
    rows = int(ws_offs[-1])
    k_scale = float(rng.choice([1.0 / 64, 1.0 / 300, 0.02]))
    v_scale = float(rng.choice([1.0, 0.01, 3.7]))
    sm = float(rng.choice([1.0, -1.0])) / math.sqrt(d)
    say(f"case extend fp8 random {case}: B {B} G {G} Hkv {Hkv} d {d} prefix {prefix.tolist()} "
        f"chunk {chunk.tolist()} k_scale {k_scale:.4g} v_scale {v_scale} sm {sm:+.3f}")
    kb, vb = _fp8_bytes(rng, (rows, Hkv, d)), _fp8_bytes(rng, (rows, Hkv, d))
    q_offs = np.zeros(B + 1, np.int64)
    q_offs[1:] = np.cumsum(chunk)
    qb = synth.host_values(rng, (int(chunk.sum()), Hq, d))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = nk.nvfp4_extend_attn_fp8(synth.to_device_bf16(qb), synth.to_device(q_offs), dev(kb), dev(vb),
                                   synth.to_device(ws_offs), synth.to_device(prefix), sm, k_scale, v_scale,
                                   max_chunk=int(chunk.max()) + int(rng.integers(0, 40)))
    torch.cuda.synchronize()
    ref, mass = oatt.extend_attention(synth.bf16_bits_to_f64(qb), _e4m3_f64(kb, k_scale), _e4m3_f64(vb, v_scale),
                                      q_offs, ws_offs, prefix, sm)
    check_out(out, ref, mass, f"extend fp8 random {case}")


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

def test_decode_page_size_not_a_power_of_two(nk):
    """Page size 48 (a multiple of 16, not a power of two: the slot and page
    arithmetic take divisions), a context that ends inside a page, every
    kernel variant and several split counts, against the oracle."""
    wl = synth.Workload(98, "page48", 3, 8, 2, 128, 48, 1000, False, 0)
    inp = synth.host_uniform_decode(wl)
    say(f"case decode page 48: {wl}")
    decode_problem(nk, inp, splits_list=(0, 1, 3, 7),
                   variants=(None, nk.VARIANT_VALU, nk.VARIANT_MFMA, nk.VARIANT_MFMA_LUT), label="page48")


def test_decode_tiny_workload(nk):
    wl = synth.WORKLOADS[1]
    say(f"case decode tiny: {wl}")
    inp = synth.host_uniform_decode(wl)
    decode_problem(nk, inp, splits_list=(1, 3, 16),
                   variants=(None, nk.VARIANT_VALU, nk.VARIANT_MFMA, nk.VARIANT_MFMA_LUT), label="tiny")


def test_decode_moderate_workload(nk):
    wl = synth.WORKLOADS[2]
    say(f"case decode moderate: {wl}")
    inp = synth.host_uniform_decode(wl)
    decode_problem(nk, inp, splits_list=(0, 1, 7), variants=(None, nk.VARIANT_VALU), label="moderate")


@pytest.mark.parametrize("L", [0, 1, 17, 100, 1000])
def test_decode_ragged_and_degenerate_lengths(nk, L):
    wl = synth.Workload(90, "ragged", 3, 10, 2, 128, 32, L, True, 4)
    say(f"case decode ragged: L {L}")
    inp = synth.host_uniform_decode(wl)
    inp.seq_lens[:] = np.array([L, max(0, L - 5), L // 2], np.int32)[:inp.seq_lens.size]
    decode_problem(nk, inp, splits_list=(1, 4), variants=(None, nk.VARIANT_VALU), label=f"L={L}")


@pytest.mark.parametrize("shape", [(1, 1, 64, 16), (16, 1, 128, 64), (4, 4, 64, 48), (7, 1, 128, 16),
                                   (5, 2, 128, 208), (2, 1, 64, 1024)])
def test_decode_group_and_shape_coverage(nk, shape):
    G, H, d, P = shape
    wl = synth.Workload(91, "shape", 2, G * H, H, d, P, 333, False, 3)
    say(f"case decode shape: G {G} Hkv {H} d {d} P {P}")
    inp = synth.host_uniform_decode(wl)
    decode_problem(nk, inp, splits_list=(1, 3), variants=(None, nk.VARIANT_VALU), label=f"G{G}-H{H}-d{d}-P{P}")


@pytest.mark.parametrize("case", range(10))
def test_decode_randomized_shapes(nk, case):
    """Seeded random combinations of the shape dimensions the fixed cases take
    one at a time: batch, query group (odd sizes included), KV heads, head_dim,
    page size, ragged lengths within the batch (zeros included), pages of one
    sequence aliased by another, and split counts from 1 to more splits than
    pages; quantize bytes exact and every decode variant within tolerance, for
    the NVFP4 cache and the FP8-E4M3 baseline cache."""
    rng = np.random.default_rng(4242 + case)
    G = int(rng.choice([1, 2, 3, 5, 6, 8, 12, 16]))
    H = int(rng.choice([1, 2, 3]))
    d = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 48, 64]))
    B = int(rng.integers(1, 6))
    ctx = int(rng.integers(1, 801))
    wl = synth.Workload(200 + case, "random", B, G * H, H, d, P, ctx, bool(rng.integers(0, 2)), 0)
    inp = synth.host_uniform_decode(wl)
    inp.seq_lens[:] = rng.integers(0, ctx + 1, B).astype(np.int32)
    inp.seq_lens[int(rng.integers(0, B))] = ctx
    alias = B > 1 and bool(rng.integers(0, 2))
    if alias:   # sequence 1 reads sequence 0's leading pages (a shared prefix)
        k = int(rng.integers(1, inp.block_tables.shape[1] + 1))
        inp.block_tables[1, :k] = inp.block_tables[0, :k]
    splits = tuple(int(x) for x in rng.choice([0, 1, 2, 3, 5, 9, 17, 64], size=2, replace=False))
    say(f"case decode random {case}: B {B} G {G} Hkv {H} d {d} P {P} ctx {ctx} lens {inp.seq_lens.tolist()} "
        f"alias {alias} splits {splits}")
    decode_problem(nk, inp, splits_list=splits,
                   variants=(None, nk.VARIANT_VALU, nk.VARIANT_MFMA, nk.VARIANT_MFMA_LUT), label=f"random{case}")
    # the same problem over the FP8-E4M3 baseline cache
    kf, vf = f8_pools(nk, inp.num_pages, H, P, d)
    nk.fp8_kv_quantize(synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v), synth.to_device(inp.slot_mapping),
                       kf, vf)
    kr = np.full((inp.num_pages, H, P, d), SENT, np.uint8)
    vr = kr.copy()
    of8.write_cache(kr, inp.k, inp.slot_mapping)
    of8.write_cache(vr, inp.v, inp.slot_mapping)
    torch.cuda.synchronize()
    assert_pool_equal(kf.data, kr, "fp8 K")
    assert_pool_equal(vf.data, vr, "fp8 V")
    ref, mass = oatt.paged_decode(inp.q, of8.dequant_cache(kr), of8.dequant_cache(vr), inp.block_tables,
                                  inp.seq_lens, wl.sm_scale)
    q, bt, sl = synth.to_device_bf16(inp.q), synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens)
    for S in splits:
        out = nk.fp8_paged_decode_attn(q, kf, vf, bt, sl, wl.sm_scale, num_splits=S)
        torch.cuda.synchronize()
        check_out(out, ref, mass, f"random{case} fp8 splits={S}")
    Sx = splits[0] or nk.nvfp4_paged_decode_num_splits(B, H, bt.shape[1], P)
    ws = nk.fp8_paged_decode_partial(q, kf, vf, bt, sl, wl.sm_scale, Sx, variant=nk.VARIANT_VALU)
    out = torch.empty_like(q)
    nk.nvfp4kv_lse_merge(ws, B, G * H, d, Sx, vf.scale, out)
    torch.cuda.synchronize()
    check_out(out, ref, mass, f"random{case} fp8 VALU")


@pytest.mark.parametrize("shape", [(8, 128, 16, 4096), (4, 64, 32, 700), (5, 128, 64, 3000)])
def test_decode_lut_unpack_matches_conversion(nk, shape):
    """The register-LUT E2M1 unpack and the conversion-instruction unpack give
    the same f16 operands, hence bit-identical partials; both match the oracle."""
    G, d, P, L = shape
    wl = synth.Workload(95, "lut", 2, 2 * G, 2, d, P, L, True, 0)
    say(f"case decode lut vs cvt: G {G} d {d} P {P} L {L}")
    inp = synth.host_uniform_decode(wl)
    for S in (1, 7):
        outs, _, _ = decode_problem(nk, inp, splits_list=(S,), variants=(nk.VARIANT_MFMA, nk.VARIANT_MFMA_LUT),
                                    label=f"lut S={S}")
        assert torch.equal(outs[0], outs[1]), "LUT unpack changed the result"


@pytest.mark.parametrize("gs", [2.0, GS_THIRD])
def test_decode_global_scale(nk, gs):
    wl = synth.Workload(92, "gs", 2, 8, 2, 128, 16, 300, True, 2)
    inp = synth.host_uniform_decode(wl)
    say(f"case decode global scale {gs}")
    decode_problem(nk, inp, splits_list=(2,), variants=(None,), gs=gs, label=f"gs{gs:.4g}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_many_splits_against_oracle(nk, d):
    """Split counts above 64 (the merge's 16-wave branch) up to the maximum,
    4096, so that most splits are empty, through the one-call
    decode and the separate partial + merge with each kernel variant, over the
    NVFP4 cache and the FP8-E4M3 cache; whole outputs against the oracle."""
    wl = synth.Workload(94, "many-splits", 2, 10, 2, d, 16, 4096, True, 0)
    inp = synth.host_uniform_decode(wl)
    inp.seq_lens[1] = 1000
    splits = (65, 200, 256, 1024, 4096)
    say(f"case decode many splits: d {d} lens {inp.seq_lens.tolist()} splits {splits}")
    decode_problem(nk, inp, splits_list=splits, variants=(None, nk.VARIANT_MFMA, nk.VARIANT_VALU),
                   label=f"many-splits d{d}")
    H, P = wl.num_kv_heads, wl.page_size
    kf, vf = f8_pools(nk, inp.num_pages, H, P, d)
    nk.fp8_kv_quantize(synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v), synth.to_device(inp.slot_mapping),
                       kf, vf)
    kr = np.full((inp.num_pages, H, P, d), SENT, np.uint8)
    vr = kr.copy()
    of8.write_cache(kr, inp.k, inp.slot_mapping)
    of8.write_cache(vr, inp.v, inp.slot_mapping)
    ref, mass = oatt.paged_decode(inp.q, of8.dequant_cache(kr), of8.dequant_cache(vr), inp.block_tables,
                                  inp.seq_lens, wl.sm_scale)
    q, bt, sl = synth.to_device_bf16(inp.q), synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens)
    for S in splits:
        out = nk.fp8_paged_decode_attn(q, kf, vf, bt, sl, wl.sm_scale, num_splits=S)
        torch.cuda.synchronize()
        check_out(out, ref, mass, f"many-splits d{d} fp8 splits={S}")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_decode_small_queries_with_a_large_key_scale(nk, fmt):
    """Queries around 1e-6 against keys carried by a tensor scale of 2^16 (the
    stored K codes are those of ordinary N(0,1) keys): logits of ordinary size
    from a query far below f16's normal range. The query's power-of-two shift
    into f16 must go up as well as down, or its elements become f16
    subnormals with a few bits left. Against the oracle, NVFP4 and FP8."""
    wl = synth.Workload(89, "small-q", 3, 12, 3, 128, 16, 900, True, 0)
    inp = synth.host_uniform_decode(wl)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    gk = 2.0 ** 16
    k_bits = synth.f32_to_bf16_bits((synth.bf16_bits_to_f64(inp.k) * gk).astype(np.float32))    # exact
    q_bits = synth.f32_to_bf16_bits((synth.bf16_bits_to_f64(inp.q) * 1e-6).astype(np.float32))
    sm = 16.0 / math.sqrt(d)                                   # logits 16 * 2^16 * 1e-6 ~ 1.05 x the N(0,1) ones
    say(f"case decode small queries: {fmt}, |q| ~ 1e-6, K global scale 2^16, sm_scale {sm:.3f}")
    q, bt, sl = synth.to_device_bf16(q_bits), synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens)
    if fmt == "nvfp4":
        kp, vp = nv_pools(nk, inp.num_pages, H, P, d)
        kp.global_scale = gk
        nk.nvfp4_kv_quantize(synth.to_device_bf16(k_bits), synth.to_device_bf16(inp.v),
                             synth.to_device(inp.slot_mapping), kp, vp)
        kd, ks = onv.empty_cache(inp.num_pages, H, P, d, fill=SENT)
        vd, vs = onv.empty_cache(inp.num_pages, H, P, d, fill=SENT)
        onv.write_cache(kd, ks, k_bits, inp.slot_mapping, gk)
        onv.write_cache(vd, vs, inp.v, inp.slot_mapping, 1.0)
        torch.cuda.synchronize()
        assert_pool_equal(kp.data, kd, "K data")
        assert_pool_equal(kp.scale, ks, "K scale")
        khat, vhat = onv.dequant_cache(kd, ks, gk), onv.dequant_cache(vd, vs, 1.0)
        run = lambda S, var: _decode_out(nk, nk.nvfp4_paged_decode_attn, nk.nvfp4_paged_decode_partial,
                                         q, kp, vp, bt, sl, sm, S, var, vp.global_scale)
    else:
        kf, vf = f8_pools(nk, inp.num_pages, H, P, d)
        kf.scale = gk
        nk.fp8_kv_quantize(synth.to_device_bf16(k_bits), synth.to_device_bf16(inp.v),
                           synth.to_device(inp.slot_mapping), kf, vf)
        kr = np.full((inp.num_pages, H, P, d), SENT, np.uint8)
        vr = kr.copy()
        of8.write_cache(kr, k_bits, inp.slot_mapping, gk)
        of8.write_cache(vr, inp.v, inp.slot_mapping)
        torch.cuda.synchronize()
        assert_pool_equal(kf.data, kr, "fp8 K")
        khat, vhat = of8.dequant_cache(kr, gk), of8.dequant_cache(vr)
        run = lambda S, var: _decode_out(nk, nk.fp8_paged_decode_attn, nk.fp8_paged_decode_partial,
                                         q, kf, vf, bt, sl, sm, S, var, vf.scale)
    ref, mass = oatt.paged_decode(q_bits, khat, vhat, inp.block_tables, inp.seq_lens, sm)
    for S, var in ((0, None), (3, nk.VARIANT_MFMA), (3, nk.VARIANT_VALU)):
        check_out(run(S, var), ref, mass, f"small-q {fmt} splits={S} variant={var}")


def _decode_out(nk, attn, partial, q, kp, vp, bt, sl, sm, S, var, out_scale):
    if var is None:
        out = attn(q, kp, vp, bt, sl, sm, num_splits=S)
    else:
        ws = partial(q, kp, vp, bt, sl, sm, S, variant=var)
        out = torch.empty_like(q)
        nk.nvfp4kv_lse_merge(ws, q.shape[0], q.shape[1], q.shape[2], S, out_scale, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("mag", [3.0e4, 1.0e-5])
def test_calibrated_global_scale_end_to_end(nk, mag):
    """Calibration on the GPU: the absmax kernel folds two chunks (one with a
    strided source and quiet and signalling NaNs, which are ignored) into a running maximum; the
    global scale derived from it keeps a tensor far outside the E4M3 range
    quantizable; bytes bit-exact against the oracle's FP32 recipe, decode
    within tolerance."""
    wl = synth.Workload(96, "calibrated", 2, 8, 2, 128, 16, 200, False, 3)
    inp = synth.host_uniform_decode(wl)
    scale = lambda b: synth.f32_to_bf16_bits((synth.bf16_bits_to_f64(b) * mag).astype(np.float32))
    k_bits, v_bits = scale(inp.k), scale(inp.v)
    say(f"case calibrated global scale: magnitude {mag}")
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    refs = []
    for i, x in enumerate((k_bits, v_bits)):
        half = x.shape[0] // 2
        wide = np.zeros((half, x.shape[1] * 3, x.shape[2]), np.uint16)     # fused-QKV-like stride
        wide[:, :x.shape[1]] = x[:half]
        wide[0, x.shape[1] + 1, 5] = 0x7FC0                              # NaN outside the K/V heads: not read
        t = synth.to_device_bf16(wide)[:, :x.shape[1]]
        rest = x[half:].copy()
        rest[3, 0, 7] = 0x7FC0                                           # NaN inside: ignored
        snan = np.random.default_rng(31 + i).permutation(rest.size)[:24]
        rest.reshape(-1)[snan] = np.where(np.arange(24) % 2 == 0, 0x7F81, 0xFF81)   # signalling NaNs too
        nk.nvfp4_kv_absmax(t, amax[i:i + 1])
        nk.nvfp4_kv_absmax(synth.to_device_bf16(rest), amax[i:i + 1])
        refs.append(max(np.abs(synth.bf16_bits_to_f64(x[:half])).max(), np.nanmax(np.abs(synth.bf16_bits_to_f64(rest)))))
    torch.cuda.synchronize()
    got = amax.cpu().numpy()
    for i in range(2):
        assert got[i] == np.float32(refs[i]), (got[i], refs[i])
    gk, gv = nk.nvfp4_global_scale_from_absmax(got[0]), nk.nvfp4_global_scale_from_absmax(got[1])
    assert gk == float(np.float32(got[0]) / np.float32(2688.0))
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    kp = nk.NVFP4Pool.empty(inp.num_pages, H, P, d, global_scale=gk)
    vp = nk.NVFP4Pool.empty(inp.num_pages, H, P, d, global_scale=gv)
    for t in (kp.data, kp.scale, vp.data, vp.scale):
        t.fill_(SENT)
    nk.nvfp4_kv_quantize(synth.to_device_bf16(k_bits), synth.to_device_bf16(v_bits), synth.to_device(inp.slot_mapping),
                         kp, vp)
    kd, ks = onv.empty_cache(inp.num_pages, H, P, d, fill=SENT)
    vd, vs = onv.empty_cache(inp.num_pages, H, P, d, fill=SENT)
    onv.write_cache(kd, ks, k_bits, inp.slot_mapping, gk)
    onv.write_cache(vd, vs, v_bits, inp.slot_mapping, gv)
    torch.cuda.synchronize()
    assert_pool_equal(kp.data, kd, "calibrated K data")
    assert_pool_equal(kp.scale, ks, "calibrated K scale")
    assert_pool_equal(vp.data, vd, "calibrated V data")
    assert_pool_equal(vp.scale, vs, "calibrated V scale")
    q = synth.to_device_bf16(inp.q)
    out = nk.nvfp4_paged_decode_attn(q, kp, vp, synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens),
                                     wl.sm_scale, num_splits=3)
    torch.cuda.synchronize()
    ref, mass = oatt.paged_decode(inp.q, onv.dequant_cache(kd, ks, gk), onv.dequant_cache(vd, vs, gv),
                                  inp.block_tables, inp.seq_lens, wl.sm_scale)
    check_out(out, ref, mass, f"calibrated x{mag}")


def test_decode_invariants(nk):
    wl = synth.Workload(93, "inv", 4, 16, 2, 128, 16, 700, True, 0)
    inp = synth.host_uniform_decode(wl)
    say("case decode invariants: determinism, page permutation, aliasing")
    outs, (kp, vp), _ = decode_problem(nk, inp, splits_list=(5, 5), variants=(None,), label="inv")
    assert torch.equal(outs[0], outs[1]), "run-to-run determinism"
    # page permutation: move every page, remap the block tables
    perm = np.random.default_rng(14).permutation(inp.num_pages)
    inv = np.argsort(perm)
    kp2 = nk.NVFP4Pool(kp.data[torch.from_numpy(perm).cuda()].contiguous(),
                       kp.scale[torch.from_numpy(perm).cuda()].contiguous())
    vp2 = nk.NVFP4Pool(vp.data[torch.from_numpy(perm).cuda()].contiguous(),
                       vp.scale[torch.from_numpy(perm).cuda()].contiguous())
    bt2 = inv[inp.block_tables].astype(np.int32)
    q = synth.to_device_bf16(inp.q)
    o2 = nk.nvfp4_paged_decode_attn(q, kp2, vp2, synth.to_device(bt2), synth.to_device(inp.seq_lens),
                                    wl.sm_scale, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(o2, outs[0]), "page-permutation invariance"
    # aliasing: two rows naming the same pages with the same query give identical rows
    bt3 = inp.block_tables.copy()
    bt3[1] = bt3[0]
    q3 = inp.q.copy()
    q3[1] = q3[0]
    data_before = kp.data.clone()
    o3 = nk.nvfp4_paged_decode_attn(synth.to_device_bf16(q3), kp, vp, synth.to_device(bt3),
                                    synth.to_device(inp.seq_lens), wl.sm_scale, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(o3[0], o3[1])
    assert torch.equal(kp.data, data_before), "decode must not write the cache"


def test_side_stream_matches_default_stream(nk):
    """Quantize, dequantize and decode issued back to back on a side stream
    (default priority; each call ordered after the previous one on that stream
    only) give bytes and outputs identical to the default-stream run."""
    wl = synth.Workload(93, "inv", 4, 16, 2, 128, 16, 700, True, 0)
    inp = synth.host_uniform_decode(wl)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    say("case side stream")
    k, v = synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v)
    slots = synth.to_device(inp.slot_mapping)
    q = synth.to_device_bf16(inp.q)
    bt, sl = synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens)
    offs = np.zeros(wl.batch + 1, np.int64)
    offs[1:] = np.cumsum(inp.seq_lens)
    rows = int(offs[-1])
    results = []
    for side in (False, True):
        kp, vp = nv_pools(nk, inp.num_pages, H, P, d)
        kws = torch.empty((rows, H, d), dtype=torch.bfloat16, device="cuda")
        vws = torch.empty_like(kws)
        torch.cuda.synchronize()
        s = torch.cuda.Stream() if side else torch.cuda.current_stream()
        with torch.cuda.stream(s):
            nk.nvfp4_kv_quantize(k, v, slots, kp, vp, stream=s)
            nk.nvfp4_kv_dequant_workspace(kp, vp, bt, sl, synth.to_device(offs), kws, vws, stream=s)
            out = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl, wl.sm_scale, num_splits=5, stream=s)
        torch.cuda.synchronize()
        results.append((kp.data.clone(), kp.scale.clone(), kws.clone(), out.clone()))
    for a, b, what in zip(results[0], results[1], ("K data", "K scale", "K workspace", "decode output")):
        assert torch.equal(a, b), what


def test_lengths_past_the_block_table_are_clamped(nk):
    """A seq_len or prefix_len above max_pages_per_seq * page_size is taken as
    that many tokens: the decode output and the workspace equal those of the
    clamped length bit for bit, and no row past them is written."""
    wl = synth.Workload(94, "clamp", 3, 8, 2, 64, 16, 96, False, 0)
    inp = synth.host_uniform_decode(wl)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    say("case lengths past the block table")
    kp, vp = nv_pools(nk, inp.num_pages, H, P, d)
    nk.nvfp4_kv_quantize(synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v),
                         synth.to_device(inp.slot_mapping), kp, vp)
    q, bt = synth.to_device_bf16(inp.q), synth.to_device(inp.block_tables)
    reach = bt.shape[1] * P
    at = torch.full((wl.batch,), reach, dtype=torch.int32, device="cuda")
    past = torch.tensor([reach + 1, reach + 1000, 1 << 30], dtype=torch.int32, device="cuda")
    for S in (1, 3):
        a = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, at, wl.sm_scale, num_splits=S)
        b = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, past, wl.sm_scale, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"splits {S}"
    rows = wl.batch * (reach + 8)
    offs = torch.arange(0, rows + 1, reach + 8, dtype=torch.int64, device="cuda")
    results = []
    for lens in (at, past):
        kws = torch.full((rows, H, d), -7.0, dtype=torch.bfloat16, device="cuda")
        vws = torch.full_like(kws, -7.0)
        nk.nvfp4_kv_dequant_workspace(kp, vp, bt, lens, offs, kws, vws)
        torch.cuda.synchronize()
        results.append((kws, vws))
    assert torch.equal(results[0][0], results[1][0]) and torch.equal(results[0][1], results[1][1])
    for b_ in range(wl.batch):   # the 8 rows after each prefix keep their fill
        tail = results[1][0][b_ * (reach + 8) + reach:(b_ + 1) * (reach + 8)]
        assert bool((tail == -7.0).all())
    # the FP8 workspace (two rows per wave): clamped lengths, and an odd prefix whose last wave
    # has its second row past the end; rows past each prefix keep their fill
    odd = torch.full((wl.batch,), reach - 1, dtype=torch.int32, device="cuda")
    results8 = []
    for lens in (at, past, odd):
        kws = torch.full((rows, H, d), 0x55, dtype=torch.uint8, device="cuda")
        vws = torch.full_like(kws, 0x55)
        nk.nvfp4_kv_dequant_workspace_fp8(kp, vp, bt, lens, offs, kws, vws)
        torch.cuda.synchronize()
        results8.append((kws, vws))
    for i in range(2):
        assert torch.equal(results8[0][i], results8[1][i])
        for b_ in range(wl.batch):
            r0 = b_ * (reach + 8)
            assert bool((results8[1][i][r0 + reach:r0 + reach + 8] == 0x55).all())
            assert torch.equal(results8[2][i][r0:r0 + reach - 1], results8[0][i][r0:r0 + reach - 1])
            assert bool((results8[2][i][r0 + reach - 1:r0 + reach + 8] == 0x55).all())


def test_binding_rejects_mismatched_device_tensors(nk):
    """The wrappers compare every device tensor with the sizes they pass to the
    C ABI: a short V, slot mapping, seq_lens, output or V pool raises ValueError
    and nothing is launched (the pools keep their sentinel bytes)."""
    say("case binding shape checks")
    T, H, P, d, pages, B = 6, 2, 16, 64, 4, 2
    kp, vp = nv_pools(nk, pages, H, P, d)
    k = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        nk.nvfp4_kv_quantize(k, k[:T - 1], slots, kp, vp)
    with pytest.raises(ValueError):
        nk.nvfp4_kv_quantize(k, k, slots[:T - 1], kp, vp)
    small_v, _ = nv_pools(nk, pages - 1, H, P, d)
    with pytest.raises(ValueError):
        nk.nvfp4_kv_quantize(k, k, slots, kp, small_v)
    q = torch.zeros((B, 2 * H, d), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 2), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), 8, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl[:1], d ** -0.5)
    with pytest.raises(ValueError):
        nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl, d ** -0.5, out=q[:1].clone())
    ws = torch.zeros((16, H, d), dtype=torch.bfloat16, device="cuda")
    offs = torch.tensor([0, 8, 16], dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        nk.nvfp4_kv_dequant_workspace(kp, vp, bt, sl, offs, ws, ws[:8])
    torch.cuda.synchronize()
    for t in (kp.data, kp.scale, vp.data, vp.scale):
        assert bool((t == SENT).all()), "a rejected call must not launch anything"


def test_fp8_decode_moderate(nk):
    wl = synth.WORKLOADS[2]
    inp = synth.host_uniform_decode(wl, batch=4)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    say(f"case fp8 decode moderate (batch 4): {wl}")
    kp, vp = f8_pools(nk, inp.num_pages, H, P, d)
    nk.fp8_kv_quantize(synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v), synth.to_device(inp.slot_mapping),
                       kp, vp)
    kr = np.full((inp.num_pages, H, P, d), SENT, np.uint8)
    vr = kr.copy()
    of8.write_cache(kr, inp.k, inp.slot_mapping)
    of8.write_cache(vr, inp.v, inp.slot_mapping)
    torch.cuda.synchronize()
    assert_pool_equal(kp.data, kr, "fp8 K")
    ref, mass = oatt.paged_decode(inp.q, of8.dequant_cache(kr), of8.dequant_cache(vr), inp.block_tables,
                                  inp.seq_lens, wl.sm_scale)
    q = synth.to_device_bf16(inp.q)
    bt, sl = synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens)
    for S in (0, 1, 5):
        out = nk.fp8_paged_decode_attn(q, kp, vp, bt, sl, wl.sm_scale, num_splits=S)
        torch.cuda.synchronize()
        check_out(out, ref, mass, f"fp8 splits={S}")
    for var in (nk.VARIANT_VALU, nk.VARIANT_MFMA):
        ws = nk.fp8_paged_decode_partial(q, kp, vp, bt, sl, wl.sm_scale, 3, variant=var)
        out = torch.empty_like(q)
        nk.nvfp4kv_lse_merge(ws, q.shape[0], q.shape[1], wl.head_dim, 3, vp.scale, out)
        torch.cuda.synchronize()
        check_out(out, ref, mass, f"fp8 variant={var}")


@pytest.mark.parametrize("fmt,G,d,P,gs", [("nvfp4", 4, 128, 16, 1.0), ("nvfp4", 5, 64, 32, GS_THIRD),
                                          ("nvfp4", 16, 128, 64, 0.5), ("fp8", 8, 128, 16, 0.37),
                                          ("fp8", 1, 64, 48, 1.0)])
def test_single_split_decode_equals_partial_and_merge(nk, fmt, G, d, P, gs):
    """With one split the decode kernel writes the output itself (no merge
    launch): bit for bit the output of the one-split partial followed by the
    merge, for every entry point that takes that route (the decode, the decode
    with the append, the allocation-free decode), with an empty sequence and
    one past the block table's reach; and within tolerance of the oracle."""
    H = 2
    wl = synth.Workload(95, "single", 5, G * H, H, d, P, 150, True, 1)
    inp = synth.host_uniform_decode(wl)
    reach = inp.block_tables.shape[1] * P
    inp.seq_lens[:] = np.array([150, 0, 1, 77, 150], np.int32)
    say(f"case single split {fmt} G{G} d{d} P{P} gs {gs}")
    q = synth.to_device_bf16(inp.q)
    bt = synth.to_device(inp.block_tables)
    sl_np = inp.seq_lens.copy()
    sl_np[4] = reach + 300                                   # taken as the reach
    sl = synth.to_device(sl_np)
    if fmt == "nvfp4":
        kp, vp = gpu_quantize_nv(nk, inp.num_pages, H, P, d, inp.k, inp.v, inp.slot_mapping, gs)
        attn, part, vscale = nk.nvfp4_paged_decode_attn, nk.nvfp4_paged_decode_partial, vp.global_scale
        kd, ks, vd, vs = oracle_nv(inp.num_pages, H, P, d, inp.k, inp.v, inp.slot_mapping, gs)
        kh, vh = onv.dequant_cache(kd, ks, gs), onv.dequant_cache(vd, vs, gs)
    else:
        kp, vp = f8_pools(nk, inp.num_pages, H, P, d, gs)
        nk.fp8_kv_quantize(synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v),
                           synth.to_device(inp.slot_mapping), kp, vp)
        attn, part, vscale = nk.fp8_paged_decode_attn, nk.fp8_paged_decode_partial, vp.scale
        kr = np.full((inp.num_pages, H, P, d), SENT, np.uint8)
        vr = kr.copy()
        of8.write_cache(kr, inp.k, inp.slot_mapping, gs)
        of8.write_cache(vr, inp.v, inp.slot_mapping, gs)
        kh, vh = of8.dequant_cache(kr, gs), of8.dequant_cache(vr, gs)
    ws = part(q, kp, vp, bt, sl, wl.sm_scale, 1)
    ref2 = torch.empty_like(q)
    nk.nvfp4kv_lse_merge(ws, q.shape[0], q.shape[1], d, 1, vscale, ref2)
    direct = attn(q, kp, vp, bt, sl, wl.sm_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(direct.view(torch.int16), ref2.view(torch.int16)), "one-split decode differs from partial + merge"
    if fmt == "nvfp4":
        noalloc = torch.empty_like(q)
        nk.nvfp4_paged_decode_attn_noalloc(q, kp, vp, bt, sl, wl.sm_scale, noalloc, num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(noalloc.view(torch.int16), ref2.view(torch.int16)), "allocation-free decode differs"
    assert torch.all(direct[1].float() == 0)                 # the empty sequence
    rl = inp.seq_lens.copy()
    rl[4] = reach
    ref, mass = oatt.paged_decode(inp.q, kh, vh, inp.block_tables, rl, wl.sm_scale)
    check_out(direct, ref, mass, f"single split {fmt}")


def _shared_prefix_problem(nk, seed, B, H, G, d, P, shared, lens, gs=1.0, dev_lens=None):
    """A batch whose first `shared` tokens sit on the same physical pages in
    every block-table row (a sequence shorter than the prefix reads its own
    first tokens from those pages), private pages after it, quantized on both
    sides. Returns device inputs, the pools and the oracle's output."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_sh = shared // P
    priv = [max(0, -(-(L - shared) // P)) for L in lens]
    max_pages = max(1, n_sh + max(priv))
    num_pages = n_sh + sum(priv) + 2
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.zeros((B, max_pages), dtype=np.int32)
    pos = n_sh
    for b in range(B):
        bt[b, :n_sh] = perm[:n_sh]
        bt[b, n_sh:n_sh + priv[b]] = perm[pos:pos + priv[b]]
        bt[b, n_sh + priv[b]:] = perm[-1]                  # unused entries name a real page
        pos += priv[b]
    slots = [bt[0, t // P].astype(np.int64) * P + t % P for t in [np.arange(shared)]]
    for b, L in enumerate(lens):
        t = np.arange(shared, max(L, shared))
        slots.append(bt[b, t // P].astype(np.int64) * P + t % P)
    slots = np.concatenate(slots)
    k = synth.host_values(rng, (len(slots), H, d))
    v = synth.host_values(rng, (len(slots), H, d))
    q = synth.host_values(rng, (B, H * G, d))
    kp, vp = gpu_quantize_nv(nk, num_pages, H, P, d, k, v, slots, gs)
    kd, ks, vd, vs = oracle_nv(num_pages, H, P, d, k, v, slots, gs)
    sl = np.array(lens, dtype=np.int32)
    ref, mass = oatt.paged_decode(q, onv.dequant_cache(kd, ks, gs), onv.dequant_cache(vd, vs, gs), bt, sl, 0.125)
    sl_dev = sl if dev_lens is None else np.array(dev_lens, dtype=np.int32)   # lengths the library is given
    return (synth.to_device_bf16(q), synth.to_device(bt), synth.to_device(sl_dev)), (kp, vp), (ref, mass)


@pytest.mark.parametrize("G,d,P,shared,lens,sp,sr", [
    (4, 128, 16, 96, [0, 5, 96, 97, 300, 160, 95, 241, 96, 1, 400, 130, 17], 0, 0),   # partial last group
    (5, 128, 16, 64, [64, 200, 33, 150, 64, 90, 300], 3, 2),                            # 3 sequences = 15 columns
    (1, 64, 48, 144, [144 + 7 * i for i in range(20)] + [0, 3], 2, 3),                  # 16 sequences per item
    (16, 64, 16, 32, [40, 10, 100], 1, 1),                                              # one sequence per item
    (8, 128, 32, 128, [128, 64, 100, 128, 1], 4, 2),                                    # nothing past the prefix
    (4, 128, 16, 2048, [2048 + 37 * i for i in range(9)] + [1000], 0, 0),              # prefix over many chunks
])
def test_shared_prefix_decode_against_oracle(nk, G, d, P, shared, lens, sp, sr):
    """The shared-prefix decode (prefix items over 16 / G sequences' query
    columns, per-column length masks, the rest split per sequence, one merge)
    against the oracle, and beside the plain decode of the same pools."""
    B, H = len(lens), 2
    say(f"case shared prefix G{G} d{d} P{P} shared {shared} B {B} splits {sp}/{sr}")
    (q, bt, sl), (kp, vp), (ref, mass) = _shared_prefix_problem(nk, 1300 + G + d + P + shared, B, H, G, d, P, shared,
                                                                  lens)
    out = nk.nvfp4_paged_decode_attn_shared_prefix(q, kp, vp, bt, sl, 0.125, shared, prefix_splits=sp, num_splits=sr)
    plain = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl, 0.125)
    torch.cuda.synchronize()
    check_out(out, ref, mass, "shared prefix")
    check_out(plain, ref, mass, "plain decode")
    assert torch.all(out[torch.tensor(lens, device=out.device) == 0].float() == 0)


@pytest.mark.parametrize("G,d", [(4, 128), (5, 64)])
def test_shared_prefix_decode_scaled_and_clamped(nk, G, d):
    """The shared-prefix decode with calibrated (non-power-of-two) K and V
    tensor scales, and one sequence length past the block table's reach (taken
    as the reach, like the plain decode): against the oracle at the clamped
    length."""
    P, shared, H = 16, 64, 2
    lens = [64, 200, 33, 150, 64, 90, 304]                      # the last fills the table's reach (19 pages)
    dev_lens = lens[:6] + [lens[6] + 500]
    say(f"case shared prefix scaled and clamped G{G} d{d}: reach {lens[6]}, length {dev_lens[6]}")
    (q, bt, sl), (kp, vp), (ref, mass) = _shared_prefix_problem(nk, 1700 + G + d, len(lens), H, G, d, P, shared,
                                                                  lens, gs=GS_THIRD, dev_lens=dev_lens)
    assert bt.shape[1] * P == lens[6]
    out = nk.nvfp4_paged_decode_attn_shared_prefix(q, kp, vp, bt, sl, 0.125, shared)
    torch.cuda.synchronize()
    check_out(out, ref, mass, "shared prefix, scaled and clamped")


@pytest.mark.parametrize("S", [1, 3])
def test_shared_prefix_of_length_zero_is_the_plain_decode(nk, S):
    """With no shared prefix the items are the plain decode's splits: the
    output is bit-identical to nvfp4_paged_decode_attn at the same count."""
    lens = [0, 17, 300, 64, 129, 1000]
    (q, bt, sl), (kp, vp), _ = _shared_prefix_problem(nk, 1400 + S, len(lens), 2, 4, 128, 16, 0, lens)
    out = nk.nvfp4_paged_decode_attn_shared_prefix(q, kp, vp, bt, sl, 0.125, 0, num_splits=S)
    plain = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl, 0.125, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)


def _append_case(nk, fmt, d, G, P, gs, S, seed, special=False, partial=False):
    """Pools holding each sequence's earlier tokens, a block table over a page
    permutation, the step's new token per sequence, and lengths that cover an
    empty sequence, one token, page boundaries, odd lengths, a length past the
    table's reach and a new token whose table entry is outside the pool.
    special: the new tokens also hold NaN, infinities, signed zeros, bf16
    subnormals and values near the bf16 maximum, in blocks of their own and
    mixed with finite values at every lane position of a block.
    partial: the two sides stop at the partials (workspaces returned in place
    of the outputs): quantize + the MFMA partial kernel against the append
    partial."""
    rng = np.random.default_rng(seed)
    H, B = 2, 8
    Hq = H * G
    lens = [0, 1, P, P + 1, 3 * P - 1, 5 * P + 7, 2 * P + 3, 4 * P]
    max_pages = (max(lens) + P - 1) // P + 1
    reach = max_pages * P
    lens[7] = reach + 5                                  # past the table: nothing appended, clamped decode
    num_pages = B * max_pages + 3
    perm = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    perm[6, (lens[6] - 1) // P] = num_pages + 4          # the new token's page is outside the pool
    bt = torch.from_numpy(perm).cuda()
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    # earlier tokens: positions 0 .. L - 2 of every sequence (within the table and the pool)
    slots, rows = [], []
    for b, L in enumerate(lens):
        for t in range(min(L, reach) - 1):
            if perm[b, t // P] < num_pages:
                slots.append(int(perm[b, t // P]) * P + t % P)
    T = len(slots)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    k_old = (torch.randn((T, H, d), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    v_old = (torch.randn((T, H, d), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    k_new = (torch.randn((B, H, d), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    v_new = (torch.randn((B, H, d), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    k_new[2, 0, :16] = 0.0                               # an all-zero block
    v_new[3, 1, 5] = 1e30                                # a block scale that saturates
    if special:
        nan, inf = float("nan"), float("inf")
        for b in range(B):
            for h in range(H):
                for t in (k_new, v_new):
                    row = t[b, h]
                    blk = (b + 2 * h + (t is v_new)) % (d // 16)
                    pos = (3 * b + h) % 16
                    kind = (b + h + (t is v_new)) % 6
                    if kind == 0:
                        row[16 * blk + pos] = nan                    # NaN among finite values
                    elif kind == 1:
                        row[16 * blk:16 * blk + 16] = nan            # a block of NaN only
                    elif kind == 2:
                        row[16 * blk + pos] = inf if b % 2 else -inf  # an infinity
                        row[16 * blk + (pos + 5) % 16] = nan
                    elif kind == 3:
                        row[16 * blk:16 * blk + 16] = 1e-39          # bf16 subnormals
                        row[16 * blk + pos] = -0.0
                    elif kind == 4:
                        row[16 * blk + pos] = 3.3e38                 # near the bf16 maximum
                    else:
                        row[16 * blk:16 * blk + 16] = -0.0           # negative zeros only
    q = torch.randn((B, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
    if fmt == "nvfp4":
        mk = lambda: nv_pools(nk, num_pages, H, P, d, gs)
        quant, attn, app = nk.nvfp4_kv_quantize, nk.nvfp4_paged_decode_attn, nk.nvfp4_paged_decode_append_attn
    else:
        mk = lambda: f8_pools(nk, num_pages, H, P, d, scale=gs)
        quant, attn, app = nk.fp8_kv_quantize, nk.fp8_paged_decode_attn, nk.fp8_paged_decode_append_attn
    kA, vA = mk()
    if T:
        quant(k_old, v_old, torch.tensor(slots, dtype=torch.int64, device="cuda"), kA, vA)
    kB, vB = mk()
    for dst, src in ((kB, kA), (vB, vA)):
        dst.data.copy_(src.data)
        if fmt == "nvfp4":
            dst.scale.copy_(src.scale)
    # the composition: quantize each new token into the slot of position L - 1, then decode
    new_slots = []
    for b, L in enumerate(lens):
        if 1 <= L <= reach:
            new_slots.append(int(perm[b, (L - 1) // P]) * P + (L - 1) % P)
        else:
            new_slots.append(-1)
    quant(k_new, v_new, torch.tensor(new_slots, dtype=torch.int64, device="cuda"), kA, vA)
    if partial:
        if fmt == "nvfp4":
            part, app_part = nk.nvfp4_paged_decode_partial, nk.nvfp4_paged_decode_append_partial
        else:
            part, app_part = nk.fp8_paged_decode_partial, nk.fp8_paged_decode_append_partial
        outA = part(q, kA, vA, bt, sl, 0.125, S, variant=nk.VARIANT_MFMA)
        outB = app_part(q, k_new, v_new, kB, vB, bt, sl, 0.125, S)
    else:
        outA = attn(q, kA, vA, bt, sl, 0.125, num_splits=S)
        outB = app(q, k_new, v_new, kB, vB, bt, sl, 0.125, num_splits=S)
    torch.cuda.synchronize()
    return (kA, vA, outA), (kB, vB, outB)


@pytest.mark.parametrize("fmt,d,G,P,gs,S", [
    ("nvfp4", 128, 5, 64, 1.0, 0), ("nvfp4", 128, 5, 16, 1.0, 3), ("nvfp4", 128, 4, 48, 1.0 / 3.0, 2),
    ("nvfp4", 64, 8, 16, 2.0, 1), ("nvfp4", 64, 1, 32, 0.3, 5), ("nvfp4", 128, 16, 16, 0.25, 7),
    ("fp8", 128, 5, 64, 1.0, 0), ("fp8", 64, 4, 16, 0.5, 3), ("fp8", 128, 8, 48, 0.3, 2),
])
def test_decode_append_matches_quantize_then_decode(nk, fmt, d, G, P, gs, S):
    """The decode step with the new token encoded by the decode kernel leaves
    every pool byte and the output equal, bit for bit, to quantize-on-write of
    the new tokens into their slots followed by the decode."""
    say(f"case append {fmt} d{d} G{G} P{P} gs {gs} splits {S}")
    (kA, vA, outA), (kB, vB, outB) = _append_case(nk, fmt, d, G, P, gs, S, seed=700 + d + G + P)
    assert torch.equal(kA.data, kB.data) and torch.equal(vA.data, vB.data)
    if fmt == "nvfp4":
        assert torch.equal(kA.scale, kB.scale) and torch.equal(vA.scale, vB.scale)
    assert torch.equal(outA, outB)


@pytest.mark.parametrize("fmt,d,G,P,gs,S", [("nvfp4", 128, 5, 64, 1.0, 4), ("nvfp4", 64, 4, 48, 0.3, 2),
                                             ("fp8", 128, 8, 16, 0.5, 3), ("fp8", 64, 2, 32, 1.0, 1)])
def test_decode_append_partial_then_merge(nk, fmt, d, G, P, gs, S):
    """The append step without the merge: pool bytes and partials equal,
    bit for bit, quantize-on-write followed by the MFMA partial kernel, and the
    merge of those partials gives the full append step's output."""
    say(f"case append partial {fmt} d{d} G{G} P{P} gs {gs} splits {S}")
    (kA, vA, wsA), (kB, vB, wsB) = _append_case(nk, fmt, d, G, P, gs, S, seed=800 + d + G + P, partial=True)
    assert torch.equal(kA.data, kB.data) and torch.equal(vA.data, vB.data)
    if fmt == "nvfp4":
        assert torch.equal(kA.scale, kB.scale) and torch.equal(vA.scale, vB.scale)
    assert torch.equal(wsA, wsB)
    # the full step (and the separate calls) on the same inputs
    (_, _, outA), (_, _, outB) = _append_case(nk, fmt, d, G, P, gs, S, seed=800 + d + G + P)
    B, Hq = outA.shape[0], outA.shape[1]
    merged = nk.nvfp4kv_lse_merge(wsB, B, Hq, d, S, vB.global_scale if fmt == "nvfp4" else vB.scale,
                                  torch.empty_like(outB))
    torch.cuda.synchronize()
    assert torch.equal(merged, outB) and torch.equal(outA, outB)


@pytest.mark.parametrize("fmt,d,gs", [("nvfp4", 128, 1.0), ("nvfp4", 64, 0.5), ("nvfp4", 128, 0.3),
                                       ("nvfp4", 64, 3.0), ("fp8", 128, 1.0), ("fp8", 64, 0.3)])
def test_decode_append_special_values(nk, fmt, d, gs):
    """New tokens with NaN, infinities, signed zeros, subnormals and values near
    the bf16 maximum: the appended pool bytes equal quantize-on-write's, bit for
    bit (both the quotient and the compare encode routes), and so do the
    outputs' bit patterns (NaN included)."""
    say(f"case append special values {fmt} d{d} gs {gs}")
    (kA, vA, outA), (kB, vB, outB) = _append_case(nk, fmt, d, 4, 16, gs, 3, seed=900 + d, special=True)
    assert torch.equal(kA.data, kB.data) and torch.equal(vA.data, vB.data)
    if fmt == "nvfp4":
        assert torch.equal(kA.scale, kB.scale) and torch.equal(vA.scale, vB.scale)
    assert torch.equal(outA.view(torch.int16), outB.view(torch.int16))


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_decode_pool_above_2gib(nk, fmt):
    """Pools of more than 2 GiB per array (buffer offsets are 32-bit, so the
    decode kernel switches to per-page addressing): the same pages placed at
    the far end of a large pool give bit-identical outputs to a small pool,
    and both match the oracle; on both pools the shared-prefix form (no
    prefix) and the decode step that appends each sequence's last token again
    give the plain decode's bits."""
    wl = synth.Workload(94, "bigpool", 3, 16, 2, 128, 64, 700, True, 3)
    inp = synth.host_uniform_decode(wl)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    row = d // 2 if fmt == "nvfp4" else d
    big = (2 ** 31) // (H * P * row) + 64          # just past 2 GiB of data per array
    say(f"case decode pool above 2 GiB: {fmt} pages {big} ({big * H * P * row / 2**30:.2f} GiB per array)")
    # small page p -> big page: spread over the pool, the last one at its very end
    remap = (big - 1 - np.arange(inp.num_pages, dtype=np.int64) * 997).astype(np.int32)
    bt_big = remap[inp.block_tables]
    slots_big = remap[inp.slot_mapping // P].astype(np.int64) * P + inp.slot_mapping % P
    q = synth.to_device_bf16(inp.q)
    kt, vt = synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v)
    sl = synth.to_device(inp.seq_lens)
    outs = []
    for pages, bt, slots in ((inp.num_pages, inp.block_tables, inp.slot_mapping), (big, bt_big, slots_big)):
        if fmt == "nvfp4":
            kp, vp = nk.NVFP4Pool.empty(pages, H, P, d), nk.NVFP4Pool.empty(pages, H, P, d)
            nk.nvfp4_kv_quantize(kt, vt, synth.to_device(slots), kp, vp)
            out = nk.nvfp4_paged_decode_attn(q, kp, vp, synth.to_device(bt), sl, wl.sm_scale, num_splits=3)
            # the shared-prefix instantiation with no prefix: the same splits, the same bits
            outc = nk.nvfp4_paged_decode_attn_shared_prefix(q, kp, vp, synth.to_device(bt), sl, wl.sm_scale, 0,
                                                            num_splits=3)
            app = nk.nvfp4_paged_decode_append_attn
        else:
            kp, vp = nk.FP8Pool.empty(pages, H, P, d), nk.FP8Pool.empty(pages, H, P, d)
            nk.fp8_kv_quantize(kt, vt, synth.to_device(slots), kp, vp)
            out = nk.fp8_paged_decode_attn(q, kp, vp, synth.to_device(bt), sl, wl.sm_scale, num_splits=3)
            outc = out
            app = nk.fp8_paged_decode_append_attn
        # the decode step with each sequence's last token appended again (same values, same bytes):
        # the append's stores and read-back through this pool's addressing leave the result unchanged
        L = int(inp.seq_lens[0])
        last = torch.arange(len(inp.seq_lens), device="cuda") * L + (L - 1)
        outa = app(q, kt[last].contiguous(), vt[last].contiguous(), kp, vp, synth.to_device(bt), sl, wl.sm_scale,
                   num_splits=3)
        torch.cuda.synchronize()
        assert torch.equal(outc, out) and torch.equal(outa, out), "shared-prefix or append form differs"
        outs.append(out)
        del kp, vp
    torch.cuda.empty_cache()
    assert torch.equal(outs[0], outs[1]), "large-pool addressing changed the result"
    if fmt == "nvfp4":
        kd, ks, vd, vs = oracle_nv(inp.num_pages, H, P, d, inp.k, inp.v, inp.slot_mapping)
        kh, vh = onv.dequant_cache(kd, ks), onv.dequant_cache(vd, vs)
    else:
        kr = np.zeros((inp.num_pages, H, P, d), np.uint8)
        vr = kr.copy()
        of8.write_cache(kr, inp.k, inp.slot_mapping)
        of8.write_cache(vr, inp.v, inp.slot_mapping)
        kh, vh = of8.dequant_cache(kr), of8.dequant_cache(vr)
    ref, mass = oatt.paged_decode(inp.q, kh, vh, inp.block_tables, inp.seq_lens, wl.sm_scale)
    check_out(outs[1], ref, mass, f"{fmt} large pool")


# ---------------------------------------------------------------------------
# the agentic prefix-reuse step at a reduced size
# ---------------------------------------------------------------------------

def test_agentic_step_small(nk):
    wl = synth.WORKLOADS[5]
    a = synth.host_agentic(wl, batch=12, len_min=120, len_max=300, shared_prefix=96, chunk=37)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    say(f"case agentic step small: B 12 pages {a.num_pages}")
    kp, vp = gpu_quantize_nv(nk, a.num_pages, H, P, d, a.k_cached, a.v_cached, a.slot_cached)
    shared = torch.from_numpy(a.shared_pages.astype(np.int64)).cuda()
    shared_before = (kp.data[shared].clone(), kp.scale[shared].clone(), vp.data[shared].clone())
    # step: quantize the chunk, dequantize prefixes, decode at the new length
    nk.nvfp4_kv_quantize(synth.to_device_bf16(a.k_chunk), synth.to_device_bf16(a.v_chunk),
                         synth.to_device(a.slot_chunk), kp, vp)
    rows = int(a.ws_row_offsets[-1])
    kws = torch.zeros((rows, H, d), dtype=torch.bfloat16, device="cuda")
    vws = torch.zeros((rows, H, d), dtype=torch.bfloat16, device="cuda")
    bt = synth.to_device(a.block_tables)
    nk.nvfp4_kv_dequant_workspace(kp, vp, bt, synth.to_device(a.cached_lens), synth.to_device(a.ws_row_offsets),
                                  kws, vws)
    q = synth.to_device_bf16(a.q)
    out = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, synth.to_device(a.seq_lens), wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(kp.data[shared], shared_before[0]) and torch.equal(kp.scale[shared], shared_before[1])
    assert torch.equal(vp.data[shared], shared_before[2])
    # oracle: the same three steps
    kd, ks, vd, vs = oracle_nv(a.num_pages, H, P, d, a.k_cached, a.v_cached, a.slot_cached)
    onv.write_cache(kd, ks, a.k_chunk, a.slot_chunk)
    onv.write_cache(vd, vs, a.v_chunk, a.slot_chunk)
    assert_pool_equal(kp.data, kd, "K data after step")
    assert_pool_equal(vp.scale, vs, "V scale after step")
    kh, vh = onv.dequant_cache(kd, ks), onv.dequant_cache(vd, vs)
    kref = oatt.dequant_workspace(kh, a.block_tables, a.cached_lens, a.ws_row_offsets, rows)
    assert np.array_equal(synth.bf16_tensor_bits(kws), kref)
    ref, mass = oatt.paged_decode(a.q, kh, vh, a.block_tables, a.seq_lens, wl.sm_scale)
    check_out(out, ref, mass, "agentic decode")


# ---------------------------------------------------------------------------
# full-size workloads, sampled (launch configuration of the benchmark)
# ---------------------------------------------------------------------------

def _sample_rows(w, b, g, t0, t1):
    """bf16 bits of K and V tokens [t0, t1) of sequence b, KV head g (logical order)."""
    kb = synth.bf16_tensor_bits(w.k_bf16[b, t0:t1, g])
    vb = synth.bf16_tensor_bits(w.v_bf16[b, t0:t1, g])
    return kb[:, None, :], vb[:, None, :]


def _check_sampled_bytes(w, b, g, t0, t1, rd, rs):
    """GPU pool bytes of tokens [t0, t1) of (b, g) equal the oracle's encode of the same rows."""
    P, d = w.wl.page_size, w.wl.head_dim
    t = np.arange(t0, t1)
    pages = torch.from_numpy(w.bt[b].cpu().numpy()[t // P].astype(np.int64)).cuda()
    offs = torch.from_numpy(t % P).cuda()
    gd = w.kp.data[pages, g, offs].cpu().numpy()
    gsc = w.kp.scale[pages, g, offs].cpu().numpy()
    assert np.array_equal(gd, rd[:, 0]) and np.array_equal(gsc, rs[:, 0]), "sampled K bytes"


def test_full_size_long_context_32k_sampled(nk):
    """Batch 44, 32K context, 32 splits (the benchmark's launch): whole (b, g)
    outputs against the oracle over all 32,768 tokens."""
    from synth.workload import build_uniform_workload
    wl = synth.WORKLOADS[3]
    say(f"case full size {wl.name}: B {wl.batch} L {wl.context} splits {wl.num_splits}")
    w = build_uniform_workload(nk, wl, keep_bf16=True)
    out = nk.nvfp4_paged_decode_attn(w.q, w.kp, w.vp, w.bt, w.sl, wl.sm_scale, num_splits=wl.num_splits)
    torch.cuda.synchronize()
    G = wl.group
    rng = np.random.default_rng(15)
    for b, g in [(0, 0), (43, 7), (int(rng.integers(44)), int(rng.integers(8)))]:
        say(f"  sample b {b} g {g}")
        kb, vb = _sample_rows(w, b, g, 0, wl.context)
        rd, rs = onv.quantize_rows(kb)
        _check_sampled_bytes(w, b, g, 0, wl.context, rd, rs)
        vd_, vs_ = onv.quantize_rows(vb)
        qb = synth.bf16_tensor_bits(w.q[b, g * G:(g + 1) * G])
        ref, mass = oatt.decode_heads(onv.bf16_to_f64(qb), onv.dequant_rows(rd, rs), onv.dequant_rows(vd_, vs_),
                                      wl.sm_scale)
        check_out(out[b, g * G:(g + 1) * G], ref, mass, f"{wl.name} b{b} g{g}")
    del w
    torch.cuda.empty_cache()


def test_full_size_extreme_context_1m_sampled(nk):
    """Batch 2, 1M context, 256 splits (the benchmark's launch). Each sampled
    split's normalised partial o/l is checked against the oracle's attention
    over that split's 4,096 tokens; the merged output against an fp64
    log-sum-exp merge of all the kernel's partials (a property that holds at
    any size); and one whole (sequence, KV head) output against the oracle
    over all 1,048,576 tokens."""
    from synth.workload import build_uniform_workload
    wl = synth.WORKLOADS[4]
    S, G, d = wl.num_splits, wl.group, wl.head_dim
    say(f"case full size {wl.name}: B {wl.batch} L {wl.context} splits {S}")
    w = build_uniform_workload(nk, wl, keep_bf16=True)
    B, Hq = w.q.shape[0], w.q.shape[1]
    ws = nk.nvfp4_paged_decode_partial(w.q, w.kp, w.vp, w.bt, w.sl, wl.sm_scale, S)
    out = torch.empty_like(w.q)
    nk.nvfp4kv_lse_merge(ws, B, Hq, d, S, 1.0, out)
    torch.cuda.synchronize()
    po, pml = nk.split_partials(ws, B, Hq, d, S)
    po, pml = po.double().cpu().numpy(), pml.double().cpu().numpy()
    per = wl.context // S
    rng = np.random.default_rng(16)
    for b, g, j in [(0, 3, 0), (1, 5, S - 1), (int(rng.integers(2)), int(rng.integers(8)), int(rng.integers(S)))]:
        say(f"  sample b {b} g {g} split {j}")
        kb, vb = _sample_rows(w, b, g, j * per, (j + 1) * per)
        rd, rs = onv.quantize_rows(kb)
        _check_sampled_bytes(w, b, g, j * per, (j + 1) * per, rd, rs)
        vd_, vs_ = onv.quantize_rows(vb)
        qb = synth.bf16_tensor_bits(w.q[b, g * G:(g + 1) * G])
        qf = onv.bf16_to_f64(qb)
        khat = onv.dequant_rows(rd, rs)
        ref, mass = oatt.decode_heads(qf, khat, onv.dequant_rows(vd_, vs_), wl.sm_scale)
        hs = slice(g * G, (g + 1) * G)
        part = po[b, hs, j]                               # the workspace holds o / l
        e = np.abs(part - ref) / np.maximum(1.0, mass)
        say(f"    partial max e {e.max():.3e} mean e {e.mean():.3e}")
        assert e.max() <= TOL_MAX and e.mean() <= TOL_MEAN
        mref = (np.einsum("gd,td->gt", qf, khat[:, 0]) * wl.sm_scale).max(axis=1) / math.log(2.0)
        assert np.allclose(pml[b, hs, j, 0], mref, rtol=1e-4, atol=1e-3)
    M = pml[..., 0].max(axis=2, keepdims=True)
    wgt = np.exp2(pml[..., 0] - M)
    merged = (po * (wgt * pml[..., 1])[..., None]).sum(axis=2) / (pml[..., 1] * wgt).sum(axis=2)[..., None]
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - merged) <= 2.0 ** -8 * np.abs(merged) + 1e-6), "merge property"
    # one whole (sequence, KV head) output against the oracle over all 1,048,576 tokens
    b, g = 1, 6
    say(f"  whole slice b {b} g {g}: {wl.context} tokens")
    ref, mass = _oracle_whole_slice(w, b, g)
    check_out(out[b, g * G:(g + 1) * G], ref, mass, f"{wl.name} b{b} g{g} whole")
    del w, ws
    torch.cuda.empty_cache()


def _oracle_whole_slice(w, b, g, piece=1 << 16):
    """Oracle decode of one (sequence, KV head) over its whole context: the kept
    bf16 rows are quantized by the oracle piece by piece (the pool bytes checked
    against them on the way), then float64 attention over all dequantized tokens."""
    wl = w.wl
    G, L, d = wl.group, wl.context, wl.head_dim
    khat = np.empty((L, 1, d))
    vhat = np.empty((L, 1, d))
    for t0 in range(0, L, piece):
        t1 = min(L, t0 + piece)
        kb, vb = _sample_rows(w, b, g, t0, t1)
        rd, rs = onv.quantize_rows(kb)
        _check_sampled_bytes(w, b, g, t0, t1, rd, rs)
        vd_, vs_ = onv.quantize_rows(vb)
        khat[t0:t1] = onv.dequant_rows(rd, rs)
        vhat[t0:t1] = onv.dequant_rows(vd_, vs_)
    qb = synth.bf16_tensor_bits(w.q[b, g * G:(g + 1) * G])
    return oatt.decode_heads(onv.bf16_to_f64(qb), khat, vhat, wl.sm_scale)


@pytest.mark.parametrize("idx,batch,fp8", [(6, 15, False), (6, 10, True), (3, 70, False), (4, 1, True)],
                         ids=["160k-b15-nvfp4", "160k-b10-fp8", "32k-b70-nvfp4", "1m-b1-fp8"])
def test_full_size_decode_figure_shapes_sampled(nk, idx, batch, fp8):
    """The other batch sizes of the page's decode figures (iso-concurrency and
    iso-capacity), in the benchmark's launch configuration. Up to 160K the
    sampled (sequence, KV head) outputs are checked whole against the oracle;
    at 1M, sampled splits' normalised partials over their own tokens."""
    from synth.workload import build_uniform_workload
    wl = synth.WORKLOADS[idx]
    G, d, P, L = wl.group, wl.head_dim, wl.page_size, wl.context
    w = build_uniform_workload(nk, wl, keep_bf16=True, fp8=fp8, batch=batch)
    S = wl.num_splits or nk.nvfp4_paged_decode_num_splits(batch, wl.num_kv_heads, w.bt.shape[1], P)
    say(f"case full size {wl.name}: B {batch} L {L} splits {S} {'fp8' if fp8 else 'nvfp4'}")
    partial = nk.fp8_paged_decode_partial if fp8 else nk.nvfp4_paged_decode_partial
    ws = partial(w.q, w.kp, w.vp, w.bt, w.sl, wl.sm_scale, S)
    out = torch.empty_like(w.q)
    nk.nvfp4kv_lse_merge(ws, batch, wl.num_q_heads, d, S, 1.0, out)
    torch.cuda.synchronize()
    per = -(-(-(-L // S)) // P) * P
    split_level = L > 200_000
    if split_level:
        po, pml = nk.split_partials(ws, batch, wl.num_q_heads, d, S)
        po, pml = po.double().cpu().numpy(), pml.double().cpu().numpy()
    rng = np.random.default_rng(17 + idx)
    for b, g in [(0, 0), (batch - 1, wl.num_kv_heads - 1), (int(rng.integers(batch)), int(rng.integers(8)))]:
        j = int(rng.integers(S)) if split_level else 0
        t0, t1 = (j * per, min(L, (j + 1) * per)) if split_level else (0, L)
        say(f"  sample b {b} g {g}" + (f" split {j} tokens [{t0}, {t1})" if split_level else ""))
        kb, vb = _sample_rows(w, b, g, t0, t1)
        t = np.arange(t0, t1)
        pages = torch.from_numpy(w.bt[b].cpu().numpy()[t // P].astype(np.int64)).cuda()
        offs = torch.from_numpy(t % P).cuda()
        if fp8:
            kr, vr = of8.quantize_rows(kb), of8.quantize_rows(vb)
            assert np.array_equal(w.kp.data[pages, g, offs].cpu().numpy(), kr[:, 0]), "sampled K bytes"
            khat, vhat = of8.dequant_cache(kr), of8.dequant_cache(vr)
        else:
            rd, rs = onv.quantize_rows(kb)
            _check_sampled_bytes(w, b, g, t0, t1, rd, rs)
            vd_, vs_ = onv.quantize_rows(vb)
            khat, vhat = onv.dequant_rows(rd, rs), onv.dequant_rows(vd_, vs_)
        qb = synth.bf16_tensor_bits(w.q[b, g * G:(g + 1) * G])
        ref, mass = oatt.decode_heads(onv.bf16_to_f64(qb), khat, vhat, wl.sm_scale)
        if split_level:
            hs = slice(g * G, (g + 1) * G)
            part = po[b, hs, j]                           # the workspace holds o / l
            e = np.abs(part - ref) / np.maximum(1.0, mass)
            say(f"    partial max e {e.max():.3e} mean e {e.mean():.3e}")
            assert e.max() <= TOL_MAX and e.mean() <= TOL_MEAN
        else:
            check_out(out[b, g * G:(g + 1) * G], ref, mass, f"{wl.name} B{batch} b{b} g{g}")
    del w, ws
    torch.cuda.empty_cache()


def test_full_size_agentic_sampled(nk):
    """64 sequences, L_b ~ U[3200, 10000], a 2,800-token prefix on 175 shared
    pages, 500-token chunks: the whole step at full size, then sampled
    sequences checked against the oracle (cache bytes, workspace rows,
    decode output of both the plain and the shared-prefix decode)."""
    from synth.workload import build_agentic_workload
    wl = synth.WORKLOADS[5]
    say(f"case full size agentic: B {wl.batch} prefix {wl.shared_prefix} chunk {wl.chunk}")
    w = build_agentic_workload(nk, wl, keep_bf16=True)
    shared = torch.from_numpy(w.shared_pages.astype(np.int64)).cuda()
    before = (w.kp.data[shared].clone(), w.kp.scale[shared].clone(), w.vp.data[shared].clone(),
              w.vp.scale[shared].clone())
    nk.nvfp4_kv_quantize(w.k_chunk, w.v_chunk, w.slot_chunk, w.kp, w.vp)
    nk.nvfp4_kv_dequant_workspace(w.kp, w.vp, w.bt, w.cached_lens, w.ws_row_offsets, w.k_ws, w.v_ws)
    out = nk.nvfp4_paged_decode_attn(w.q, w.kp, w.vp, w.bt, w.seq_lens, wl.sm_scale)
    outc = nk.nvfp4_paged_decode_attn_shared_prefix(w.q, w.kp, w.vp, w.bt, w.seq_lens, wl.sm_scale, wl.shared_prefix)
    torch.cuda.synchronize()
    after = (w.kp.data[shared], w.kp.scale[shared], w.vp.data[shared], w.vp.scale[shared])
    assert all(torch.equal(x, y) for x, y in zip(before, after)), "shared prefix pages were written"
    H, P, d, G, C = wl.num_kv_heads, wl.page_size, wl.head_dim, wl.group, wl.chunk
    offs = w.ws_row_offsets.cpu().numpy()
    for b in (0, 37, wl.batch - 1):
        L = int(w.host_cached_lens[b])
        say(f"  sample sequence {b}: cached {L}")
        kb = np.concatenate([synth.bf16_tensor_bits(w.k_shared), synth.bf16_tensor_bits(w.k_private[b]),
                             synth.bf16_tensor_bits(w.k_chunk[b * C:(b + 1) * C])])
        vb = np.concatenate([synth.bf16_tensor_bits(w.v_shared), synth.bf16_tensor_bits(w.v_private[b]),
                             synth.bf16_tensor_bits(w.v_chunk[b * C:(b + 1) * C])])
        kd, ks = onv.quantize_rows(kb)
        vd, vs = onv.quantize_rows(vb)
        t = np.arange(L + C)
        pages = torch.from_numpy(w.host_bt[b][t // P].astype(np.int64)).cuda()
        offp = torch.from_numpy(t % P).cuda()
        assert np.array_equal(w.kp.data[pages, :, offp].cpu().numpy(), kd), "K data"
        assert np.array_equal(w.kp.scale[pages, :, offp].cpu().numpy(), ks), "K scale"
        assert np.array_equal(w.vp.data[pages, :, offp].cpu().numpy(), vd), "V data"
        assert np.array_equal(w.vp.scale[pages, :, offp].cpu().numpy(), vs), "V scale"
        khat, vhat = onv.dequant_rows(kd, ks), onv.dequant_rows(vd, vs)
        rows = synth.bf16_tensor_bits(w.k_ws[offs[b]:offs[b] + L])
        assert np.array_equal(rows, oatt.f64_to_bf16_exact(khat[:L])), "K workspace"
        rows = synth.bf16_tensor_bits(w.v_ws[offs[b]:offs[b] + L])
        assert np.array_equal(rows, oatt.f64_to_bf16_exact(vhat[:L])), "V workspace"
        qb = onv.bf16_to_f64(synth.bf16_tensor_bits(w.q[b]))
        ref, mass = oatt.decode_heads(qb, khat, vhat, wl.sm_scale)
        check_out(out[b], ref, mass, f"agentic b{b}")
        check_out(outc[b], ref, mass, f"agentic shared-prefix decode b{b}")
    del w
    torch.cuda.empty_cache()
