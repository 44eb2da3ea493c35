"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: each check uses a closed form,
a hand derivation stored under tests/golden/, an independent library routine
(torch's float8_e4m3fn cast and scaled_dot_product_attention, Python's
round-half-even), brute force, or an invariant of the definition.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, formats, fp8, nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits(x):
    """bf16 bits of float values that bf16 represents exactly (test helper)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF)
    return (u >> 16).astype(np.uint16)


def _all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = nvfp4.bf16_to_f64(b)
    ok = np.isfinite(v)
    return b[ok], v[ok]


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def test_e2m1_table_matches_golden():
    with open(os.path.join(GOLDEN, "e2m1_magnitudes.txt")) as f:
        vals = [float(t) for line in f if not line.startswith("#") for t in line.split()]
    assert vals == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(formats.E2M1_VALUES[:8]) == vals
    assert list(formats.E2M1_VALUES[8:]) == [-v for v in vals]
    assert math.copysign(1.0, formats.E2M1_VALUES[8]) == -1.0


def test_e4m3_closed_form_points():
    v = formats.E4M3_VALUES
    assert v[0x7E] == 448.0 and formats.E4M3_MAX == 448.0
    assert v[0x01] == 2.0 ** -9
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    finite = v[:127]
    assert np.all(np.diff(finite) > 0)


def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.E4M3_VALUES
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], ours[m])


def test_e4m3_encode_matches_torch_on_every_bf16():
    bits, vals = _all_bf16_finite()
    in_range = np.abs(vals) < 464.0          # torch's cast does not saturate beyond
    x = vals[in_range]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = formats.e4m3_encode(x)
    assert np.array_equal(ours, ref)
    big = vals[~in_range]
    enc = formats.e4m3_encode(big)
    assert np.all((enc & 0x7F) == 0x7E)      # saturation to +-448
    assert np.array_equal(enc >> 7, np.signbit(big).astype(np.uint8))


def _e2m1_code_by_round(r: float) -> int:
    """Independent rounding: the E2M1 grid is uniform on [0,2] (step 0.5),
    [2,4] (step 1) and [4,6] (step 2); Python's round() is half-to-even, and on
    each piece an even rounded value is an even code."""
    if r >= 6:
        return 7
    if r <= 2:
        return int(round(r * 2))            # codes 0..4 are 0, .5, 1, 1.5, 2
    if r <= 4:
        return int(round(r)) + 2            # codes 4..6 are 2, 3, 4
    return 6 if round(r / 2) == 2 else 7    # codes 6..7 are 4, 6


def test_e2m1_rounding_matches_piecewise_round():
    _, vals = _all_bf16_finite()
    r = np.abs(vals[(np.abs(vals) <= 8)])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    r = np.unique(np.concatenate([r, mids, mids + 1e-12, mids - 1e-12]))
    ours = formats.e2m1_magnitude_code(r)
    ref = np.array([_e2m1_code_by_round(float(x)) for x in r])
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# NVFP4 block encode
# ---------------------------------------------------------------------------

def _golden_vectors():
    cases = []
    with open(os.path.join(GOLDEN, "nvfp4_block_vectors.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, xs, s, data = [p.strip() for p in line.split("|")]
            x = [float(t) for t in xs.split()]
            cases.append((name, x, int(s, 16), [int(t, 16) for t in data.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_vectors(), ids=lambda c: c[0])
def test_block_vectors_golden(case):
    name, x, s_exp, data_exp = case
    bits = _bf16_bits(np.array(x, dtype=np.float64)).reshape(1, 1, 16)
    data, scale = nvfp4.quantize_rows(bits)
    assert int(scale[0, 0, 0]) == s_exp
    assert list(data[0, 0]) == data_exp


def test_round_trip_every_scale():
    """Blocks built as S * (E2M1 values including +-6) encode to S's own byte
    and decode back exactly, for every positive finite E4M3 scale."""
    rng = np.random.default_rng(0)
    for sb in range(1, 0x7F):
        S = formats.E4M3_VALUES[sb]
        codes = rng.integers(0, 16, size=16)
        codes[rng.integers(0, 16)] = 7 if rng.random() < 0.5 else 15   # amax = 6 S
        x = formats.E2M1_VALUES[codes] * S
        bits = _bf16_bits(x).reshape(1, 1, 16)
        data, scale = nvfp4.quantize_rows(bits)
        assert int(scale[0, 0, 0]) == sb
        back = nvfp4.dequant_rows(data, scale)
        assert np.array_equal(back.reshape(16), x)


def test_encode_is_nearest_by_brute_force():
    """Scale = nearest E4M3 to amax/6 and each code = nearest E2M1 to |x|/S,
    checked by exhaustive argmin over the candidates (ties to the even code)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2000, 16)).astype(np.float32)
    x[::7] *= 20.0
    x[::11] *= 1e-3
    bits = np.asarray(x).view(np.uint32)
    bits = ((bits.astype(np.uint64) + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    xv = nvfp4.bf16_to_f64(bits)
    data, scale = nvfp4.quantize_rows(bits.reshape(2000, 1, 16))
    codes = nvfp4.unpack_nibbles(data.reshape(2000, 8))
    e4 = formats.E4M3_VALUES[:127]
    e2 = formats.E2M1_VALUES[:8]
    for i in range(2000):
        target = np.max(np.abs(xv[i])) / 6.0
        dist = np.abs(e4 - target)
        best = np.flatnonzero(dist == dist.min())
        sb = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        if target > 448:
            sb = 0x7E
        assert scale[i, 0, 0] == sb
        S = e4[sb]
        for j in range(16):
            c = codes[i, j]
            assert (c >> 3) == (1 if math.copysign(1.0, xv[i, j]) < 0 else 0)
            if S == 0:
                assert (c & 7) == 0
                continue
            r = abs(xv[i, j]) / S
            dd = np.abs(e2 - r)
            cand = np.flatnonzero(dd == dd.min())
            want = cand[0] if len(cand) == 1 else [c2 for c2 in cand if c2 % 2 == 0][0]
            if r > 6:
                want = 7
            assert (c & 7) == want


def test_storage_ratio_golden():
    facts = {}
    with open(os.path.join(GOLDEN, "storage_ratio.txt")) as f:
        for line in f:
            if not line.startswith("#") and line.strip():
                k, v = line.split()
                facts[k] = float(v)
    for d in (64, 128):
        nv = nvfp4.storage_bytes(1000, 8, d)
        f8 = 1000 * 8 * d
        assert nv / f8 == facts["ratio"] == (facts["nvfp4_bytes_per_16"] / facts["fp8_bytes_per_16"])
        data, scale = nvfp4.empty_cache(10, 8, 16, d)
        assert (data.nbytes + scale.nbytes) / (10 * 8 * 16 * d) == facts["ratio"]
    assert round(1 / facts["ratio"], 2) == facts["capacity_gain_rounded"]


def test_nibble_order_and_cache_layout():
    assert list(nvfp4.pack_nibbles(np.array([1, 2, 0xF, 0x8], dtype=np.uint8))) == [0x21, 0x8F]
    rng = np.random.default_rng(2)
    P, H, d = 16, 2, 32
    x = _bf16_bits(formats.E2M1_VALUES[rng.integers(0, 16, size=(3, H, d))])
    data, scale = nvfp4.empty_cache(4, H, P, d, fill=0xAB)
    # a negative slot and one past the pool (4 pages * P) skip their rows, as the entry point does
    nvfp4.write_cache(data, scale, np.concatenate([x, x[:1]]), np.array([2 * P + 5, -1, 0 * P + 15, 4 * P]))
    rd, rs = nvfp4.quantize_rows(x)
    assert np.array_equal(data[2, :, 5], rd[0]) and np.array_equal(scale[2, :, 5], rs[0])
    assert np.array_equal(data[0, :, 15], rd[2]) and np.array_equal(scale[0, :, 15], rs[2])
    untouched = np.ones(data.shape[:3], bool)
    untouched[2, :, 5] = untouched[0, :, 15] = False
    assert np.all(data[untouched] == 0xAB) and np.all(scale[untouched] == 0xAB)


def test_planted_tie_mistake_is_caught():
    """A rounding mistake planted in the oracle (ties away from zero) must
    fail the golden vectors: the pins are sensitive to it."""
    orig = formats._rne_on_grid

    def ties_away(x, grid):
        x = np.asarray(x, dtype=np.float64)
        hi = np.minimum(np.searchsorted(grid, x, side="left"), len(grid) - 1)
        lo = np.maximum(hi - 1, 0)
        idx = np.where(grid[hi] - x <= x - grid[lo], hi, lo)
        return np.where(x >= grid[-1], len(grid) - 1, np.where(x == 0, 0, idx))

    formats._rne_on_grid = ties_away
    try:
        bad = 0
        for name, x, s_exp, data_exp in _golden_vectors():
            bits = _bf16_bits(np.array(x)).reshape(1, 1, 16)
            data, scale = nvfp4.quantize_rows(bits)
            bad += int(scale[0, 0, 0]) != s_exp or list(data[0, 0]) != data_exp
        assert bad > 0
    finally:
        formats._rne_on_grid = orig


# ---------------------------------------------------------------------------
# FP8 baseline
# ---------------------------------------------------------------------------

def test_fp8_rows_match_torch_cast():
    _, vals = _all_bf16_finite()
    x = vals[np.abs(vals) < 464]
    bits = _bf16_bits(x)
    ours = fp8.quantize_rows(bits)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    back = torch.from_numpy(ref).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(fp8.dequant_cache(ours), back)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _small_problem(seed=3, B=2, Hq=4, Hkv=2, d=32, P=16, lens=(37, 64)):
    rng = np.random.default_rng(seed)
    max_pages = max(-(-L // P) for L in lens)
    num_pages = B * max_pages + 3
    perm = rng.permutation(num_pages)
    bt = perm[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    k_hat = rng.standard_normal((num_pages, Hkv, P, d))
    v_hat = rng.standard_normal((num_pages, Hkv, P, d))
    q = _bf16_bits(np.round(rng.standard_normal((B, Hq, d)) * 64) / 64)
    return q, k_hat, v_hat, bt, np.array(lens, dtype=np.int32)


def test_attention_matches_torch_sdpa():
    q, k_hat, v_hat, bt, lens = _small_problem()
    sm = 1 / math.sqrt(q.shape[-1])
    out, mass = attention.paged_decode(q, k_hat, v_hat, bt, lens, sm)
    qf = nvfp4.bf16_to_f64(q)
    G = q.shape[1] // k_hat.shape[1]
    for b in range(q.shape[0]):
        k = attention.gather_tokens(k_hat, bt[b], lens[b])
        v = attention.gather_tokens(v_hat, bt[b], lens[b])
        kq = torch.from_numpy(np.repeat(k.transpose(1, 0, 2), G, axis=0))[None]
        vq = torch.from_numpy(np.repeat(v.transpose(1, 0, 2), G, axis=0))[None]
        qq = torch.from_numpy(qf[b])[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq, scale=sm)
        np.testing.assert_allclose(out[b], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    assert np.all(mass >= np.abs(out) - 1e-12)


def test_attention_brute_force_loops():
    q, k_hat, v_hat, bt, lens = _small_problem(seed=4, B=1, Hq=2, Hkv=1, d=8, P=4, lens=(9,))
    sm = 0.3
    out, _ = attention.paged_decode(q, k_hat, v_hat, bt, lens, sm)
    qf = nvfp4.bf16_to_f64(q)
    P = k_hat.shape[2]
    for h in range(2):
        logits = []
        for t in range(9):
            page = bt[0][t // P]
            s = 0.0
            for c in range(8):
                s += qf[0, h, c] * k_hat[page, 0, t % P, c]
            logits.append(s * sm)
        mx = max(logits)
        w = [math.exp(z - mx) for z in logits]
        for c in range(8):
            acc = sum(w[t] * v_hat[bt[0][t // P], 0, t % P, c] for t in range(9))
            assert abs(out[0, h, c] - acc / sum(w)) < 1e-13


def test_attention_special_cases():
    q, k_hat, v_hat, bt, lens = _small_problem(seed=5)
    sm = 0.2
    # L = 1: the output is the first value row
    one = np.array([1, 1], dtype=np.int32)
    out, _ = attention.paged_decode(q, k_hat, v_hat, bt, one, sm)
    G = 2
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b, h], v_hat[bt[b, 0], h // G, 0])
    # q = 0: uniform weights, the output is the mean value row
    z = np.zeros_like(q)
    out, _ = attention.paged_decode(z, k_hat, v_hat, bt, lens, sm)
    for b in range(2):
        v = attention.gather_tokens(v_hat, bt[b], lens[b])
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v[:, h // G].mean(axis=0), rtol=1e-12, atol=1e-13)
    # empty sequence: zeros
    out, _ = attention.paged_decode(q, k_hat, v_hat, bt, np.array([0, 5], np.int32), sm)
    assert np.all(out[0] == 0)


def test_attention_dominant_key_selects_its_value():
    d, P, L = 16, 8, 20
    k = np.zeros((4, 1, P, d))
    v = np.random.default_rng(6).standard_normal((4, 1, P, d))
    bt = np.array([[2, 0, 3]], np.int32)
    for t in range(L):                       # orthogonal one-hot keys
        k[bt[0, t // P], 0, t % P, t % d] = 1.0
    j = 13
    q = _bf16_bits(np.eye(d)[j % d][None, None, :] * 256.0)
    out, _ = attention.paged_decode(q, k, v, bt, np.array([L], np.int32), 1.0)
    # tokens j and j - d share the one-hot direction only if j >= d; j=13 < 16 is unique
    np.testing.assert_allclose(out[0, 0], v[bt[0, j // P], 0, j % P], atol=1e-100)


def test_attention_page_permutation_invariance():
    q, k_hat, v_hat, bt, lens = _small_problem(seed=7)
    out1, _ = attention.paged_decode(q, k_hat, v_hat, bt, lens, 0.25)
    perm = np.random.default_rng(8).permutation(k_hat.shape[0])
    inv = np.argsort(perm)
    out2, _ = attention.paged_decode(q, k_hat[perm], v_hat[perm], inv[bt].astype(np.int32), lens, 0.25)
    np.testing.assert_array_equal(out1, out2)


def test_gqa_group_one_is_mha():
    q, k_hat, v_hat, bt, lens = _small_problem(seed=9, Hq=2, Hkv=2)
    out, _ = attention.paged_decode(q, k_hat, v_hat, bt, lens, 0.3)
    for h in range(2):
        o1, _ = attention.paged_decode(q[:, h:h + 1], k_hat[:, h:h + 1], v_hat[:, h:h + 1], bt, lens, 0.3)
        np.testing.assert_allclose(out[:, h], o1[:, 0], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# extend-path workspace
# ---------------------------------------------------------------------------

def test_workspace_is_exact_bf16_of_dequantized_prefix():
    rng = np.random.default_rng(10)
    H, d, P, num_pages = 2, 32, 16, 12
    x = _bf16_bits(np.round(rng.standard_normal((num_pages * P, H, d)) * 16) / 16)
    data, scale = nvfp4.empty_cache(num_pages, H, P, d)
    slots = rng.permutation(num_pages * P)
    nvfp4.write_cache(data, scale, x, slots)
    hat = nvfp4.dequant_cache(data, scale)
    bt = rng.permutation(num_pages).astype(np.int32).reshape(3, 4)
    prefix = np.array([17, 0, 64], np.int32)
    offs = np.array([0, 20, 25, 100], np.int64)
    ws = attention.dequant_workspace(hat, bt, prefix, offs, 100, fill=0x7FC0)
    for b in range(3):
        got = nvfp4.bf16_to_f64(ws[offs[b]:offs[b] + prefix[b]])
        np.testing.assert_array_equal(got, attention.gather_tokens(hat, bt[b], prefix[b]))
    assert np.all(ws[17:20] == 0x7FC0) and np.all(ws[20:25] == 0x7FC0) and np.all(ws[89:] == 0x7FC0)
    # every E2M1 * E4M3 product is exact in bf16
    prod = np.outer(formats.E2M1_VALUES, formats.E4M3_VALUES[:127]).reshape(-1)
    attention.f64_to_bf16_exact(prod)


# ---------------------------------------------------------------------------
# calibrated global scale: the FP32 recipe
# ---------------------------------------------------------------------------

def _test_blocks(rng, n=4000):
    """bf16-valued blocks over many magnitudes, plus blocks built from exact midpoints."""
    mags = 2.0 ** rng.integers(-12, 14, size=(n, 1))
    x = (rng.standard_normal((n, 16)) * mags).astype(np.float32)
    x = nvfp4.bf16_to_f64(nvfp4.f32_to_bf16_rne(x))
    ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -1.75, -3.5, 0.0, 6.0, 3.0, 2.0, 1.0])
    return np.concatenate([x, ties[None, :] * 2.0 ** np.arange(-6, 7)[:, None]])


@pytest.mark.parametrize("gs", [1.0, 2.0, 0.5, 2.0 ** -8, 2.0 ** 6])
def test_fp32_recipe_is_the_exact_encode_at_power_of_two_scales(gs):
    """Two formulations: FP32 threshold compares vs division and nearest-even
    rounding in float64. At a power-of-two gs they must agree everywhere."""
    x = _test_blocks(np.random.default_rng(31))
    c1, s1 = nvfp4.encode_blocks(x, gs)
    c2, s2 = nvfp4.encode_blocks_fp32(x, gs)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)


@pytest.mark.parametrize("gs", [float(np.float32(1.0 / 3.0)), float(np.float32(0.1))])
def test_fp32_recipe_differs_from_real_arithmetic_only_at_rounding_boundaries(gs):
    """At a calibrated (non-power-of-two) gs the FP32 recipe rounds 6*gs, the
    scale quotient, S*gs and the thresholds. Wherever it disagrees with the
    real-number encode, the real quantity must sit within a few FP32 ulps of
    the boundary that decided it; anything else would be an arithmetic slip."""
    rng = np.random.default_rng(32)
    x = _test_blocks(rng, 20000)
    c_real, s_real = nvfp4.encode_blocks(x, gs)
    c_f32, s_f32 = nvfp4.encode_blocks_fp32(x, gs)
    # block scales: a disagreement means amax / (6 gs) is within 4 ulps of an E4M3 rounding boundary
    bad_s = np.nonzero(s_real != s_f32)[0]
    grid = formats.E4M3_VALUES[:127]
    mids = (grid[1:] + grid[:-1]) / 2
    for i in bad_s:
        q = np.abs(x[i]).max() / (6.0 * gs)
        dist = np.min(np.abs(mids - q))
        assert dist <= 4 * np.spacing(np.float32(q)), (i, q, dist)
    # element codes (same scale byte): a disagreement means |x| is within 4 ulps of a midpoint m * S * gs
    same = s_real == s_f32
    diff = np.argwhere((c_real != c_f32) & same[:, None])
    for i, e in diff:
        s = formats.E4M3_VALUES[s_real[i]] * gs
        a = abs(x[i, e])
        dist = min(abs(a - m * s) for m, _ in nvfp4.MIDPOINTS)
        assert dist <= 4 * np.spacing(np.float32(a)), (i, e, a, dist)
    assert 0 < len(bad_s) + len(diff) < 0.01 * x.size     # the rounding does matter, and only rarely


def test_calibrated_global_scale_recovers_the_dynamic_range():
    """The accuracy lever of the tensor scale: with gs = 1 a tensor whose
    blocks exceed 448 * 6 saturates and one below the E4M3 range flushes to
    zero; gs = amax / 2688 brings both back to NVFP4's ordinary error."""
    rng = np.random.default_rng(33)
    for mag in (3.0e4, 1.0e-5):
        x = rng.standard_normal((512, 16)) * mag
        x = nvfp4.bf16_to_f64(nvfp4.f32_to_bf16_rne(x.astype(np.float32)))
        gs_cal = float(np.float32(np.abs(x).max()) / np.float32(2688.0))
        errs = {}
        for gs in (1.0, gs_cal):
            c, s = (nvfp4.encode_blocks if gs == 1.0 else nvfp4.encode_blocks_fp32)(x, gs)
            xh = formats.E2M1_VALUES[c.astype(np.int64)] * (formats.E4M3_VALUES[s] * gs)[:, None]
            errs[gs] = np.sqrt(np.mean((xh - x) ** 2) / np.mean(x ** 2))
        assert errs[1.0] > 0.5, errs          # saturated or flushed
        assert errs[gs_cal] < 0.15, errs      # NVFP4's usual relative error


def test_workspace_bits_are_exact_at_power_of_two_scales():
    rng = np.random.default_rng(34)
    xb = nvfp4.f32_to_bf16_rne(rng.standard_normal((64, 2, 128)).astype(np.float32) * 3)
    for gs in (1.0, 0.25, 8.0):
        d, s = nvfp4.quantize_rows(xb, gs)
        assert np.array_equal(nvfp4.workspace_bits(d, s, gs), attention.f64_to_bf16_exact(nvfp4.dequant_rows(d, s, gs)))


# ---------------------------------------------------------------------------
# the pages' FP8 path-2 types: FP8 source, FP8 workspace
# ---------------------------------------------------------------------------

def test_fp8_workspace_rounds_exactly_the_non_e4m3_products():
    """Every product e2m1 * S (gs = ws_scale = 1) either is an E4M3 value and
    is stored exactly, or is stored as its nearest E4M3 value (ties to the
    even byte, saturating at 448). Checked against rational arithmetic and a
    linear search; 275 of the 1016 products are rounded, 63 of them saturate."""
    from fractions import Fraction
    grid = [(Fraction(formats.E4M3_VALUES[b]), b) for b in range(127)]
    codes = np.arange(8, dtype=np.uint8)
    data = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)            # the 8 magnitudes, one block half
    data = np.concatenate([data, data])                                  # 16 elements
    rounded = saturated = 0
    for sb in range(127):
        got = nvfp4.workspace_fp8_bytes(data[None, :], np.array([[sb]], np.uint8))[0]
        for c in range(8):
            exact = Fraction(formats.E2M1_VALUES[c]) * Fraction(formats.E4M3_VALUES[sb])
            if exact > 448:
                want, saturated = 0x7E, saturated + 1
            else:
                best = min(grid, key=lambda g: (abs(g[0] - exact), g[1] & 1))
                want = best[1]
            if Fraction(formats.E4M3_VALUES[want]) != exact:
                rounded += 1
            assert got[c] == want, (sb, c, got[c], want)
    assert (rounded, saturated) == (275, 63)


def test_fp8_source_rows_equal_the_bf16_route():
    """FP8 values are bf16 values (4 significant bits), so quantizing FP8 bytes
    at source scale 1 must equal quantizing their bf16 images."""
    rng = np.random.default_rng(35)
    b = rng.integers(0, 256, size=(64, 2, 128)).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x41                                          # no NaN bytes
    d1, s1 = nvfp4.quantize_rows_fp8(b)
    vals = formats.E4M3_VALUES[b.astype(np.int64)].astype(np.float32)
    d2, s2 = nvfp4.quantize_rows((vals.view(np.uint32) >> 16).astype(np.uint16))
    assert np.array_equal(d1, d2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------
# extend attention (path 2)
# ---------------------------------------------------------------------------

def test_extend_attention_pins():
    """A one-query chunk is decode over the prefix plus itself; later chunk
    keys never change earlier queries (causality); explicit loops on a tiny
    case agree with the vectorised routine."""
    rng = np.random.default_rng(36)
    Hq, Hkv, d, sm = 4, 2, 16, 0.25
    L, C = 5, 3
    q = rng.standard_normal((C, Hq, d))
    k = rng.standard_normal((L + C, Hkv, d))
    v = rng.standard_normal((L + C, Hkv, d))
    qo, wo, pl = np.array([0, C]), np.array([0, L + C]), np.array([L])
    out, _ = attention.extend_attention(q, k, v, qo, wo, pl, sm)
    # query 0 = decode over keys [0, L]
    ref0, _ = attention.decode_heads(q[0], k[:L + 1], v[:L + 1], sm)
    assert np.allclose(out[0], ref0, rtol=1e-13, atol=1e-13)
    # causality: perturb the last chunk key; queries 0 .. C-2 unchanged
    k2, v2 = k.copy(), v.copy()
    k2[-1] += 5.0
    v2[-1] -= 3.0
    out2, _ = attention.extend_attention(q, k2, v2, qo, wo, pl, sm)
    assert np.array_equal(out2[:C - 1], out[:C - 1]) and not np.allclose(out2[C - 1], out[C - 1])
    # explicit loops
    for i in range(C):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = [sm * sum(q[i, h, c] * k[j, g, c] for c in range(d)) for j in range(L + i + 1)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            o = [sum(w[j] * v[j, g, c] for j in range(L + i + 1)) / sum(w) for c in range(d)]
            assert np.allclose(out[i, h], o, rtol=1e-12, atol=1e-12)


def test_extend_attention_matches_torch_sdpa():
    """Ragged sequences (an empty prefix, a one-query chunk, spare workspace
    rows between sequences, GQA groups of 4): each sequence's chunk against
    torch's scaled_dot_product_attention in float64 with the causal mask
    shifted by the prefix length (query i sees keys j <= prefix + i)."""
    rng = np.random.default_rng(37)
    Hq, Hkv, d, sm = 8, 2, 32, -0.17
    G = Hq // Hkv
    prefix, chunk, spare = np.array([13, 0, 40]), np.array([7, 5, 1]), np.array([2, 0, 3])
    qo = np.concatenate([[0], np.cumsum(chunk)])
    wo = np.concatenate([[0], np.cumsum(prefix + chunk + spare)])
    q = rng.standard_normal((int(qo[-1]), Hq, d))
    k = rng.standard_normal((int(wo[-1]), Hkv, d))
    v = rng.standard_normal((int(wo[-1]), Hkv, d))
    out, mass = attention.extend_attention(q, k, v, qo, wo, prefix.astype(np.int32), sm)
    for b in range(len(prefix)):
        n, c = int(prefix[b] + chunk[b]), int(chunk[b])
        kb = k[wo[b]:wo[b] + n].transpose(1, 0, 2)                    # [Hkv][n][d]
        vb = v[wo[b]:wo[b] + n].transpose(1, 0, 2)
        kq = torch.from_numpy(np.repeat(kb, G, axis=0))[None]         # [1][Hq][n][d]
        vq = torch.from_numpy(np.repeat(vb, G, axis=0))[None]
        qq = torch.from_numpy(q[qo[b]:qo[b + 1]].transpose(1, 0, 2).copy())[None]   # [1][Hq][c][d]
        mask = torch.from_numpy(np.arange(n)[None, :] <= prefix[b] + np.arange(c)[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq, attn_mask=mask, scale=sm)
        np.testing.assert_allclose(out[qo[b]:qo[b + 1]], ref[0].numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
    assert np.all(mass >= np.abs(out) - 1e-12)


# ---------------------------------------------------------------------------
# bf16 rounding (the workspace at a calibrated scale, and the input generator)
# ---------------------------------------------------------------------------

def _bf16_rounding_cases(n_random=4_000_000):
    """float32 bit patterns that decide a bf16 rounding rule: every finite bf16
    value's exact halfway point to its upper neighbour (both signs), one f32
    ulp either side of it, the value itself, plus random finite patterns."""
    b = np.arange(1 << 15, dtype=np.uint32)                      # non-negative bf16 patterns
    b = b[(b & 0x7F80) != 0x7F80]                                 # finite only
    hi = np.concatenate([b, b | 0x8000]) << 16                    # both signs
    pats = np.concatenate([hi, hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi | 0x0001])
    rng = np.random.default_rng(40)
    r = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    r = r[(r & 0x7F800000) != 0x7F800000]
    return np.concatenate([pats, r]).astype(np.uint32).view(np.float32)


def _torch_bf16_bits(x):
    """torch's CPU float32 -> bfloat16 cast, an independent round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch():
    """oracle f32_to_bf16_rne (the last step of the workspace value at any
    calibrated scale) and the input generator's rounding, against torch's
    float32 -> bfloat16 cast on every halfway point and 4M random patterns."""
    x = _bf16_rounding_cases()
    want = _torch_bf16_bits(x)
    assert np.array_equal(nvfp4.f32_to_bf16_rne(x), want)
    import synth
    assert np.array_equal(synth.f32_to_bf16_bits(x), want)


def test_bf16_rounding_pin_catches_planted_mistakes():
    """Truncation, or ties rounded away from zero, must fail the torch pin."""
    x = _bf16_rounding_cases(n_random=0)
    want = _torch_bf16_bits(x)
    u = x.view(np.uint32).astype(np.uint64)
    truncate = (u >> 16).astype(np.uint16)
    ties_away = ((u + 0x8000) >> 16).astype(np.uint16)
    assert not np.array_equal(truncate, want)
    assert not np.array_equal(ties_away, want)


def test_workspace_bits_at_a_calibrated_scale_match_torch():
    """Every workspace value bf16(fl32(e2m1 * fl32(S * gs))) at gs = fl32(1/3):
    all 16 E2M1 codes under every finite E4M3 scale byte, against the same
    float32 products and bf16 cast done in torch from torch's own E4M3 decode."""
    gs = np.float32(1.0 / 3.0)
    e2m1 = np.loadtxt(os.path.join(GOLDEN, "e2m1_magnitudes.txt"), dtype=np.float32)
    e2m1 = np.concatenate([e2m1, -e2m1])                              # codes 0..15
    sbytes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    s_t = torch.from_numpy(sbytes).view(torch.float8_e4m3fn).float()
    prod = torch.from_numpy(e2m1)[None, :] * (s_t * torch.tensor(gs))[:, None]   # [scales][16]
    want = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes = np.arange(16, dtype=np.uint8)
    data = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), (sbytes.size, 1))  # [scales][8]
    got = nvfp4.workspace_bits(data, sbytes[:, None], float(gs))
    assert np.array_equal(got, want)
    assert np.count_nonzero(prod.numpy() != prod.to(torch.bfloat16).float().numpy()) > 0   # rounding happens


# ---------------------------------------------------------------------------
# non-finite elements under the FP32 recipe
# ---------------------------------------------------------------------------

def _nonfinite_vectors():
    cases = []
    with open(os.path.join(GOLDEN, "nvfp4_nonfinite_blocks.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, gs, xs, s, data = [p.strip() for p in line.split("|")]
            bits = np.array([int(t, 16) for t in xs.split()], np.uint16)
            cases.append((name, float(gs), bits, int(s, 16), [int(t, 16) for t in data.split()]))
    return cases


def _encode_golden_bits(bits, gs, enc=None):
    with np.errstate(invalid="ignore", over="ignore"):
        codes, s = (enc or nvfp4.encode_blocks_fp32)(nvfp4.bf16_to_f64(bits).reshape(1, 16), gs)
    return int(s[0]), list(nvfp4.pack_nibbles(codes)[0])


@pytest.mark.parametrize("case", _nonfinite_vectors(), ids=lambda c: c[0])
def test_nonfinite_blocks_golden(case):
    name, gs, bits, s_exp, data_exp = case
    assert np.float32(gs) == np.float32(1.0) or np.float32(gs) == np.float32(1.0 / 3.0)
    s, data = _encode_golden_bits(bits, gs)
    assert s == s_exp, (name, hex(s))
    assert data == data_exp, (name, [hex(v) for v in data])


def test_nonfinite_pin_catches_planted_mistakes():
    """Two plausible mistakes in the non-finite handling must fail the golden
    blocks: NaN taking the saturated code 7, and a block maximum that
    propagates NaN (np.max) instead of ignoring it."""
    cases = _nonfinite_vectors()

    def nan_code_seven(x, gs):
        c, s = nvfp4.encode_blocks_fp32(x, gs)
        return np.where(np.isnan(x), (c & 8) | 7, c).astype(np.uint8), s

    def nan_propagating_max(x, gs):
        c, s = nvfp4.encode_blocks_fp32(x, gs)
        amax = np.max(np.abs(x), axis=-1)
        s = np.where(np.isnan(amax), 0x7F, s).astype(np.uint8)
        return c, s

    for planted in (nan_code_seven, nan_propagating_max):
        bad = sum(_encode_golden_bits(bits, gs, planted) != (s_exp, data_exp)
                  for _, gs, bits, s_exp, data_exp in cases)
        assert bad > 0, planted.__name__
