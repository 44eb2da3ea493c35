"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before any HIP call (no GPU needed).

The pointers passed here are never dereferenced: validation runs on the
host and returns before anything is launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4kv.h")


@pytest.fixture(scope="module")
def L():
    import nvfp4_quantized_paged_amd as nk
    if not os.path.exists(nk.LIB_PATH):
        from nvfp4_quantized_paged_amd import build
        build.build()
    return nk


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:const\s+char\s*\*|int32_t|int|size_t|float)\s+(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("nvfp4_kv_quantize", "nvfp4_kv_dequant_workspace", "nvfp4_paged_decode_attn",
                     "fp8_paged_decode_attn", "fp8_kv_quantize", "nvfp4kv_lse_merge", "nvfp4_kv_absmax",
                     "nvfp4_global_scale_from_absmax"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert L.abi_version() == 1


def test_exported_symbols_are_only_the_abi(L):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.split()[-2] in ("T", "W")}
    ours = {n for n in exported if not n.startswith("_")}
    assert ours == set(declared_functions())


def test_split_heuristic_and_workspace_size(L):
    # at most 3072 items (at least one split), at most one split per 128 tokens of the longest sequence
    assert L.nvfp4_paged_decode_num_splits(44, 8, 512, 64) == 8
    assert L.nvfp4_paged_decode_num_splits(2, 8, 16384, 64) == 192
    assert L.nvfp4_paged_decode_num_splits(64, 8, 657, 16) == 6
    assert L.nvfp4_paged_decode_num_splits(10, 8, 2560, 64) == 38
    assert L.nvfp4_paged_decode_num_splits(512, 8, 64, 16) == 1
    assert L.nvfp4_paged_decode_num_splits(8, 8, 256, 16) == 32        # 4096 tokens: the 128-token cap
    assert L.nvfp4_paged_decode_num_splits(2, 1, 10, 16) == 2          # 160 tokens
    assert L.nvfp4_paged_decode_num_splits(1, 1, 16, 16) == 2
    assert L.nvfp4_paged_decode_workspace_bytes(44, 40, 128, 32) == 44 * 40 * 32 * (128 * 2 + 8)
    assert L.nvfp4_paged_decode_workspace_bytes(0, 40, 128, 32) == 0


FAKE = 0x100000  # aligned, never dereferenced


def _geom(L, pages=16, P=16, H=1, d=64):
    return L.Geom(pages, P, H, d)


def _nv(L, data=FAKE, scale=FAKE, gs=1.0):
    return L.NVFP4CacheDesc(data, scale, gs)


def _quant(L, g, k=FAKE, v=FAKE, stride=64, T=4, slots=FAKE, kc=None, vc=None):
    kc = kc or _nv(L)
    vc = vc or _nv(L)
    gp = ctypes.byref(g) if g is not None else None
    return L.lib().nvfp4_kv_quantize(gp, k, v, stride, T, slots, ctypes.byref(kc), ctypes.byref(vc), None)


def test_quantize_rejects_bad_arguments(L):
    assert _quant(L, None) == L.EINVAL
    assert _quant(L, _geom(L, d=96)) == L.EUNSUPPORTED
    assert _quant(L, _geom(L, d=80)) == L.EUNSUPPORTED
    assert _quant(L, _geom(L, P=8)) == L.EUNSUPPORTED
    assert _quant(L, _geom(L, pages=0)) == L.EINVAL
    assert _quant(L, _geom(L), T=-1) == L.EINVAL
    assert _quant(L, _geom(L), k=None) == L.EINVAL
    assert _quant(L, _geom(L), slots=None) == L.EINVAL
    assert _quant(L, _geom(L), stride=32) == L.EINVAL
    assert _quant(L, _geom(L), stride=68) == L.EALIGN
    assert _quant(L, _geom(L), k=FAKE + 2) == L.EALIGN
    assert _quant(L, _geom(L), kc=_nv(L, data=FAKE + 8)) == L.EALIGN
    assert _quant(L, _geom(L), vc=_nv(L, scale=None)) == L.EINVAL
    assert _quant(L, _geom(L), kc=_nv(L, gs=0.0)) == L.EINVAL
    assert _quant(L, _geom(L), kc=_nv(L, gs=float("nan"))) == L.EINVAL
    assert "global_scale" in L.last_error()
    # zero tokens: accepted, nothing launched
    assert _quant(L, _geom(L), T=0, k=None, v=None, slots=None) == L.OK


def _decode(L, g, q=FAKE, bt=FAKE, maxp=16, sl=FAKE, B=1, Hq=4, sm=0.125, S=1, ws=FAKE,
            ws_bytes=1 << 20, out=FAKE, fn="nvfp4_paged_decode_attn"):
    kc, vc = _nv(L), _nv(L)
    return getattr(L.lib(), fn)(ctypes.byref(g), q, ctypes.byref(kc), ctypes.byref(vc), bt, maxp, sl, B, Hq,
                                sm, S, ws, ws_bytes, out, None)


def test_decode_rejects_bad_arguments(L):
    g = _geom(L)
    assert _decode(L, g, q=None) == L.EINVAL
    assert _decode(L, g, q=FAKE + 4) == L.EALIGN
    assert _decode(L, g, out=FAKE + 2) == L.EALIGN
    assert _decode(L, g, out=None) == L.EINVAL
    assert _decode(L, g, B=-1) == L.EINVAL
    assert _decode(L, g, maxp=0) == L.EINVAL
    assert _decode(L, g, maxp=(1 << 31) // 16) == L.EINVAL     # max_pages * page_size past 2^31 - 1
    assert "2^31" in L.last_error()
    assert _decode(L, _geom(L, H=2), Hq=3) == L.EINVAL
    assert _decode(L, g, Hq=32) == L.EUNSUPPORTED
    assert _decode(L, g, S=5000) == L.EINVAL
    assert _decode(L, g, S=-1) == L.EINVAL
    assert _decode(L, g, sm=float("inf")) == L.EINVAL
    assert _decode(L, g, ws_bytes=100) == L.EWORKSPACE
    assert "workspace" in L.last_error()
    assert _decode(L, g, ws=None) == L.EINVAL
    # batch 0 needs no workspace and launches nothing
    assert _decode(L, g, B=0, ws=None, ws_bytes=0) == L.OK


def _shared(L, g, B=1, Hq=4, maxp=16, shared=16, sp=0, sr=0, ws_bytes=1 << 20, out=FAKE, ws=FAKE):
    kc, vc = _nv(L), _nv(L)
    return L.lib().nvfp4_paged_decode_attn_shared_prefix(ctypes.byref(g), FAKE, ctypes.byref(kc), ctypes.byref(vc),
                                                          FAKE, maxp, FAKE, B, Hq, 0.125, shared, sp, sr, ws,
                                                          ws_bytes, out, None)


def test_shared_prefix_decode_checks_its_arguments(L):
    """The shared-prefix decode validates the prefix length (whole pages within
    the table's reach), the split counts and the grid on the host, and sizes
    its workspace as the partials of prefix + further splits."""
    g = _geom(L, P=16, H=2, d=128)
    f = L.lib().nvfp4_paged_decode_shared_prefix_workspace_bytes
    assert f(ctypes.byref(g), 16, 13, 8, 96, 2, 3) == 13 * 8 * 5 * (128 * 2 + 8)
    # automatic counts: the plain decode's count past the prefix; prefix items at least as long
    rest = L.nvfp4_paged_decode_num_splits(13, 2, 16 - 96 // 16, 16)
    span = -(-(16 * 16 - 96) // rest)
    pref = min(max(96 // span, 1), 96 // 16)
    assert f(ctypes.byref(g), 16, 13, 8, 96, 0, 0) == 13 * 8 * (pref + rest) * (128 * 2 + 8)
    assert f(ctypes.byref(g), 16, 13, 8, 0, 0, 3) == 13 * 8 * 3 * (128 * 2 + 8)   # no prefix items
    for bad in (8, -16, 16 * 16 + 16):                                      # not whole pages, negative, past the reach
        assert f(ctypes.byref(g), 16, 13, 8, bad, 0, 0) == 0
        assert _shared(L, g, shared=bad) == L.EINVAL
    assert "shared_len" in L.last_error()
    assert f(ctypes.byref(g), 16, 13, 8, 96, 5000, 0) == 0
    assert _shared(L, g, sp=5000) == L.EINVAL
    assert _shared(L, g, sp=4000, sr=200) == L.EINVAL                    # more than 4096 slots in all
    assert _shared(L, g, B=40000, sp=1, sr=2) == L.EUNSUPPORTED            # grid past 65535 items per KV head
    assert _shared(L, g, ws_bytes=16) == L.EWORKSPACE
    assert _shared(L, g, out=None) == L.EINVAL
    assert _shared(L, g, Hq=2 * 17) == L.EUNSUPPORTED                      # query group above 16
    assert _shared(L, g, B=0, ws=None, ws_bytes=0) == L.OK                 # nothing to do, nothing launched


def _noalloc(L, g, B=1, Hq=4, S=1, q=FAKE, out=FAKE, maxp=16):
    kc, vc = _nv(L), _nv(L)
    return L.lib().nvfp4_paged_decode_attn_noalloc(ctypes.byref(g), q, ctypes.byref(kc), ctypes.byref(vc), FAKE,
                                                   maxp, FAKE, B, Hq, 0.125, S, out, None)


def test_noalloc_decode_rejects_partials_past_its_static_scratch(L):
    """The allocation-free decode keeps its partials in a 32 MiB static array:
    explicit split counts whose partials exceed it, and shapes where even one
    split does not fit, are rejected on the host (no HIP call)."""
    assert L.lib().nvfp4_paged_decode_noalloc_scratch_bytes() == 32 << 20
    g = _geom(L, H=1, d=64)
    per_split = 100 * 16 * (64 * 2 + 8)                      # batch 100, 16 query heads
    S = (32 << 20) // per_split + 1
    assert _noalloc(L, g, B=100, Hq=16, S=S) == L.EWORKSPACE
    assert "static scratch" in L.last_error()
    assert _noalloc(L, g, B=65535, Hq=16, S=1) == L.EWORKSPACE            # one split is 143 MB
    assert _noalloc(L, g, B=65535, Hq=16, S=0) == L.EWORKSPACE            # auto cannot lower below one
    assert _noalloc(L, g, out=None) == L.EINVAL
    assert _noalloc(L, g, out=FAKE + 2) == L.EALIGN
    assert _noalloc(L, g, q=None) == L.EINVAL
    assert _noalloc(L, g, S=5000) == L.EINVAL
    assert _noalloc(L, g, B=0) == L.OK                                   # nothing to do, nothing launched


def _append(L, g, fp8=False, knew=FAKE, vnew=FAKE, stride=64, B=1, S=1, out=FAKE, ws_bytes=1 << 20, partial=False):
    name = ("fp8" if fp8 else "nvfp4") + ("_paged_decode_append_partial" if partial else "_paged_decode_append_attn")
    f = getattr(L.lib(), name)
    if fp8:
        kc, vc = L.FP8CacheDesc(FAKE, 1.0), L.FP8CacheDesc(FAKE, 1.0)
    else:
        kc, vc = _nv(L), _nv(L)
    args = [ctypes.byref(g), FAKE, knew, vnew, stride, ctypes.byref(kc), ctypes.byref(vc), FAKE, 16, FAKE, B, 4,
            0.125, S, FAKE, ws_bytes]
    return f(*(args if partial else args + [out]), None)


def test_append_decode_rejects_bad_new_tokens(L):
    """The decode step with the new token validates the new-token rows on the
    host (no HIP call): present, 16-byte aligned, rows at least Hkv * d
    elements apart and a multiple of 8."""
    g = _geom(L, H=1, d=64)
    for fp8 in (False, True):
        assert _append(L, g, fp8, knew=None) == L.EINVAL
        assert _append(L, g, fp8, vnew=None) == L.EINVAL
        assert _append(L, g, fp8, knew=FAKE + 2) == L.EALIGN
        assert _append(L, g, fp8, stride=63) == L.EINVAL                # below Hkv * d
        assert _append(L, g, fp8, stride=68) == L.EINVAL                # not a multiple of 8
        assert "new_stride" in L.last_error()
        assert _append(L, g, fp8, out=None) == L.EINVAL
        assert _append(L, g, fp8, S=5000) == L.EINVAL
        assert _append(L, g, fp8, ws_bytes=16) == L.EWORKSPACE
        assert _append(L, g, fp8, B=0, knew=None, vnew=None) == L.OK   # nothing to do, nothing launched


def test_append_partial_rejects_bad_arguments(L):
    """The append step without the merge checks what the full step checks,
    except the output, and needs an explicit split count."""
    g = _geom(L, H=1, d=64)
    for fp8 in (False, True):
        assert _append(L, g, fp8, partial=True, S=0) == L.EINVAL
        assert _append(L, g, fp8, partial=True, knew=None) == L.EINVAL
        assert _append(L, g, fp8, partial=True, vnew=FAKE + 8) == L.EALIGN
        assert _append(L, g, fp8, partial=True, stride=68) == L.EINVAL
        assert _append(L, g, fp8, partial=True, ws_bytes=16) == L.EWORKSPACE
        assert _append(L, g, fp8, partial=True, B=0, knew=None, vnew=None) == L.OK


def test_partial_rejects_bad_variant_and_auto_splits(L):
    g = _geom(L)
    kc, vc = _nv(L), _nv(L)
    f = L.lib().nvfp4_paged_decode_partial
    args = lambda S, variant: (ctypes.byref(g), FAKE, ctypes.byref(kc), ctypes.byref(vc), FAKE, 16, FAKE, 1, 4,
                               0.125, S, variant, FAKE, 1 << 20, None)
    assert f(*args(1, 7)) == L.EINVAL
    assert f(*args(1, 4)) == L.EINVAL
    assert f(*args(1, -1)) == L.EINVAL
    assert f(*args(0, 0)) == L.EINVAL      # the partial call needs an explicit split count


def test_merge_rejects_bad_arguments(L):
    f = L.lib().nvfp4kv_lse_merge
    assert f(FAKE, 1 << 20, 1, 4, 96, 1, 1.0, FAKE, None) == L.EUNSUPPORTED
    assert f(FAKE, 1 << 20, 1, 4, 64, 0, 1.0, FAKE, None) == L.EINVAL
    assert f(FAKE, 10, 1, 4, 64, 1, 1.0, FAKE, None) == L.EWORKSPACE
    assert f(None, 1 << 20, 1, 4, 64, 1, 1.0, FAKE, None) == L.EINVAL
    assert f(FAKE, 1 << 20, 1, 4, 64, 1, float("nan"), FAKE, None) == L.EINVAL
    assert f(FAKE, 0, 0, 4, 64, 1, 1.0, None, None) == L.OK


def test_workspace_dequant_rejects_bad_arguments(L):
    g = _geom(L)
    kc, vc = _nv(L), _nv(L)
    f = L.lib().nvfp4_kv_dequant_workspace
    ok = dict(bt=FAKE, maxp=16, pl=FAKE, offs=FAKE, B=2, kw=FAKE, vw=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(g), ctypes.byref(kc), ctypes.byref(vc), a["bt"], a["maxp"], a["pl"], a["offs"],
                 a["B"], a["kw"], a["vw"], None)

    assert call(B=-1) == L.EINVAL
    assert call(bt=None) == L.EINVAL
    assert call(offs=None) == L.EINVAL
    assert call(maxp=0) == L.EINVAL
    assert call(maxp=1 << 30) == L.EINVAL                           # 2^30 pages of 16 tokens: beyond int32 positions
    assert call(kw=FAKE + 2) == L.EALIGN
    assert call(B=0, bt=None, pl=None, offs=None, kw=None, vw=None) == L.OK


def test_fp8_entry_points_validate(L):
    g = _geom(L)
    kc = L.FP8CacheDesc(FAKE, 1.0)
    bad = L.FP8CacheDesc(FAKE, -1.0)
    f = L.lib().fp8_kv_quantize
    assert f(ctypes.byref(g), FAKE, FAKE, 64, 4, FAKE, ctypes.byref(kc), ctypes.byref(bad), None) == L.EINVAL
    assert f(ctypes.byref(g), FAKE, FAKE, 64, 0, FAKE, ctypes.byref(kc), ctypes.byref(kc), None) == L.OK
    d = L.lib().fp8_paged_decode_attn
    assert d(ctypes.byref(g), FAKE, ctypes.byref(kc), ctypes.byref(kc), FAKE, 16, FAKE, 1, 4, 0.125, 1, FAKE, 8,
             FAKE, None) == L.EWORKSPACE


def test_absmax_rejects_bad_arguments(L):
    f = L.lib().nvfp4_kv_absmax
    FAKE16, FAKE4 = 1 << 20, (1 << 20) + 4
    assert f(FAKE16, 1024, 0, 8, 128, None, None) == L.OK            # no tokens: nothing to do
    assert f(FAKE16, 1024, -1, 8, 128, FAKE4, None) == L.EINVAL
    assert f(FAKE16, 1024, 4, 0, 128, FAKE4, None) == L.EINVAL
    assert f(FAKE16, 1024, 4, 8, 96, FAKE4, None) == L.EUNSUPPORTED
    assert f(None, 1024, 4, 8, 128, FAKE4, None) == L.EINVAL
    assert f(FAKE16, 1024, 4, 8, 128, None, None) == L.EINVAL
    assert f(FAKE16, 1000, 4, 8, 128, FAKE4, None) == L.EINVAL     # stride below a token row
    assert f(FAKE16 + 2, 1024, 4, 8, 128, FAKE4, None) == L.EALIGN
    assert f(FAKE16, 1028, 4, 8, 128, FAKE4, None) == L.EALIGN
    assert f(FAKE16, 1024, 4, 8, 128, FAKE4 + 1, None) == L.EALIGN


def test_extend_rejects_bad_arguments(L):
    f = L.lib().nvfp4_extend_attn
    F = 1 << 20
    ok = dict(batch=2, hq=8, hkv=2, d=128, mc=64, sm=0.088)

    def call(q=F, qo=F, k=F, v=F, wo=F, pl=F, out=F, **kw):
        a = dict(ok, **kw)
        return f(q, qo, k, v, wo, pl, a["batch"], a["hq"], a["hkv"], a["d"], a["mc"], a["sm"], out, None)

    assert call(batch=0) == L.OK and call(mc=0) == L.OK            # nothing to do
    assert call(batch=-1) == L.EINVAL
    assert call(mc=-1) == L.EINVAL
    assert call(hkv=0) == L.EINVAL
    assert call(hq=6, hkv=4) == L.EINVAL                            # not a multiple
    assert call(hq=6, hkv=2) == L.EUNSUPPORTED                      # group 3
    assert call(hq=64, hkv=2) == L.EUNSUPPORTED                     # group 32
    assert call(d=96) == L.EUNSUPPORTED
    assert call(sm=float("nan")) == L.EINVAL and call(sm=float("inf")) == L.EINVAL
    assert call(batch=1 << 20, hkv=1024, hq=1024, mc=1 << 12) == L.EINVAL   # grid above 2^31 - 1
    assert call(hkv=1 << 17, hq=1 << 17) == L.EINVAL               # 64-row block above 2 GiB
    assert call(q=None) == L.EINVAL and call(pl=None) == L.EINVAL and call(out=None) == L.EINVAL
    assert call(q=F + 2) == L.EALIGN and call(k=F + 8) == L.EALIGN and call(out=F + 4) == L.EALIGN


def test_extend_fp8_rejects_bad_arguments(L):
    f = L.lib().nvfp4_extend_attn_fp8
    F = 1 << 20
    ok = dict(batch=2, hq=8, hkv=2, d=128, mc=64, sm=0.088, ks=0.5, vs=2.0)

    def call(q=F, qo=F, k=F, v=F, wo=F, pl=F, out=F, **kw):
        a = dict(ok, **kw)
        return f(q, qo, k, v, wo, pl, a["batch"], a["hq"], a["hkv"], a["d"], a["mc"], a["sm"], a["ks"], a["vs"],
                 out, None)

    assert call(batch=0) == L.OK and call(mc=0) == L.OK            # nothing to do
    assert call(batch=-1) == L.EINVAL and call(mc=-1) == L.EINVAL
    assert call(hq=6, hkv=2) == L.EUNSUPPORTED and call(d=96) == L.EUNSUPPORTED
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(ks=bad) == L.EINVAL and call(vs=bad) == L.EINVAL
        assert call(ks=bad, batch=0) == L.EINVAL                  # scales are checked before the no-op
    assert call(sm=1e30, ks=1e30) == L.EINVAL                       # logit scale overflows FP32
    assert call(sm=float("nan")) == L.EINVAL
    assert call(k=None) == L.EINVAL and call(v=None) == L.EINVAL
    assert call(k=F + 8) == L.EALIGN and call(v=F + 4) == L.EALIGN and call(q=F + 2) == L.EALIGN


def test_read_probe_rejects_bad_arguments(L):
    f = L.lib().nvfp4kv_hbm_read_probe
    FAKE16, FAKE4 = 1 << 20, (1 << 20) + 4
    assert f(FAKE16, 0, 64, 1, FAKE4, None) == L.OK                 # nothing to read
    assert f(FAKE16, -16, 64, 1, FAKE4, None) == L.EINVAL
    assert f(FAKE16, 1000, 64, 1, FAKE4, None) == L.EINVAL           # not a multiple of 16
    assert f(FAKE16, 1024, 0, 1, FAKE4, None) == L.EINVAL
    assert f(None, 1024, 64, 1, FAKE4, None) == L.EINVAL
    assert f(FAKE16, 1024, 64, 1, None, None) == L.EINVAL
    assert f(FAKE16 + 8, 1024, 64, 1, FAKE4, None) == L.EALIGN
    assert f(FAKE16, 1024, 64, 1, FAKE4 + 2, None) == L.EALIGN
    assert f(FAKE16, 1024, 64, 4, FAKE4, None) == L.EINVAL           # unknown flag


def test_global_scale_from_absmax(L):
    g = L.nvfp4_global_scale_from_absmax
    assert g(2688.0) == 1.0                       # 448 * 6: the largest block maps onto scale 448, element 6
    assert g(1344.0) == 0.5
    assert g(0.0) == 1.0 and g(-3.0) == 1.0 and g(float("inf")) == 1.0 and g(float("nan")) == 1.0
    import numpy as np
    for a in (1.0, 3.14159, 1e-20, 6.5e4, 1e30):
        assert g(a) == float(np.float32(a) / np.float32(2688.0))


def test_fp8_path2_entry_points_validate(L):
    g = _geom(L)
    kc, vc = _nv(L), _nv(L)
    q = L.lib().nvfp4_kv_quantize_fp8
    ok = dict(k=FAKE, v=FAKE, stride=64, T=4, slots=FAKE, ks=1.0, vs=1.0, rows=None, kw=None, vw=None)

    def quant(**kw):
        a = dict(ok, **kw)
        return q(ctypes.byref(g), a["k"], a["v"], a["stride"], a["T"], a["slots"], a["ks"], a["vs"],
                 ctypes.byref(kc), ctypes.byref(vc), a["rows"], a["kw"], a["vw"], None)

    assert quant(T=0, k=None, v=None, slots=None) == L.OK
    assert quant(ks=0.0) == L.EINVAL and quant(vs=float("nan")) == L.EINVAL
    assert quant(stride=72) == L.EALIGN                 # FP8 rows are read 16 bytes at a time
    assert quant(stride=32) == L.EINVAL                 # below a token row (1 x 64)
    assert quant(rows=FAKE) == L.EINVAL                 # a copy needs both workspaces
    assert quant(rows=FAKE, kw=FAKE + 8, vw=FAKE) == L.EALIGN
    d = L.lib().nvfp4_kv_dequant_workspace_fp8
    okd = dict(bt=FAKE, maxp=16, pl=FAKE, offs=FAKE, B=2, ks=1.0, vs=1.0, kw=FAKE, vw=FAKE)

    def deq(**kw):
        a = dict(okd, **kw)
        return d(ctypes.byref(g), ctypes.byref(kc), ctypes.byref(vc), a["bt"], a["maxp"], a["pl"], a["offs"],
                 a["B"], a["ks"], a["vs"], a["kw"], a["vw"], None)

    assert deq(ks=-1.0) == L.EINVAL and deq(vs=float("inf")) == L.EINVAL
    assert deq(bt=None) == L.EINVAL
    assert deq(kw=FAKE + 8) == L.EALIGN
    assert deq(B=0, bt=None, pl=None, offs=None, kw=None, vw=None) == L.OK


def test_binding_fails_loudly_without_the_library(L, monkeypatch, tmp_path):
    """No silent fallback: with the native library absent, every entry point raises."""
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libnvfp4kv.so"))
    monkeypatch.setattr(L, "_lib_handle", None)
    with pytest.raises(ImportError):
        L.lib()
    with pytest.raises(ImportError):
        L.nvfp4_global_scale_from_absmax(1.0)
    with pytest.raises(ImportError):
        L.nvfp4_paged_decode_num_splits(1, 1, 16, 16)


def test_binding_rejects_tensors_smaller_than_the_sizes_it_passes(L):
    """The C ABI cannot see tensor sizes; the binding compares every tensor with
    the sizes it passes, so a short V, slot mapping, table, pool or output raises
    before anything is launched (CPU tensors: the checks look at shapes only)."""
    import torch
    nk = L
    T, H, P, d, pages, B = 5, 2, 16, 64, 4, 3
    pool = lambda n=pages, h=H: nk.NVFP4Pool(torch.empty((n, h, P, d // 2), dtype=torch.uint8),
                                             torch.empty((n, h, P, d // 16), dtype=torch.uint8))
    kp, vp = pool(), pool()
    k = torch.empty((T, H, d), dtype=torch.bfloat16)
    slots = torch.empty(T, dtype=torch.int64)
    assert nk._check_quantize_shapes(k, k.clone(), slots, kp, vp).num_pages == pages
    with pytest.raises(ValueError, match="v must have shape"):
        nk._check_quantize_shapes(k, k[:T - 1], slots, kp, vp)
    with pytest.raises(ValueError, match="slot_mapping"):
        nk._check_quantize_shapes(k, k, slots[:T - 1], kp, vp)
    with pytest.raises(ValueError, match="k must have shape"):
        nk._check_quantize_shapes(torch.empty((T, H, 2 * d), dtype=torch.bfloat16), k, slots, kp, vp)
    with pytest.raises(ValueError, match="same geometry"):
        nk._check_quantize_shapes(k, k, slots, kp, pool(n=pages - 1))

    bt = torch.empty((B, 8), dtype=torch.int32)
    ws = torch.empty((40, H, d), dtype=torch.bfloat16)
    pl, offs = torch.empty(B, dtype=torch.int32), torch.empty(B + 1, dtype=torch.int64)
    nk._check_workspace_shapes(kp, vp, bt, pl, offs, ws, ws.clone())
    with pytest.raises(ValueError, match="prefix_lens"):
        nk._check_workspace_shapes(kp, vp, bt, pl[:B - 1], offs, ws, ws)
    with pytest.raises(ValueError, match="ws_row_offsets"):
        nk._check_workspace_shapes(kp, vp, bt, pl, offs[:B], ws, ws)
    with pytest.raises(ValueError, match="v_ws"):
        nk._check_workspace_shapes(kp, vp, bt, pl, offs, ws, ws[:10])
    with pytest.raises(ValueError, match="k_ws"):
        nk._check_workspace_shapes(kp, vp, bt, pl, offs, torch.empty((40, H + 1, d), dtype=torch.bfloat16), ws)

    q = torch.empty((B, 4 * H, d), dtype=torch.bfloat16)
    sl = torch.empty(B, dtype=torch.int32)
    nk._check_decode_shapes(q, kp, vp, bt, sl, q.clone())
    with pytest.raises(ValueError, match="seq_lens"):
        nk._check_decode_shapes(q, kp, vp, bt, sl[:B - 1])
    with pytest.raises(ValueError, match="block_tables"):
        nk._check_decode_shapes(q, kp, vp, bt[:B - 1], sl)
    with pytest.raises(ValueError, match="out"):
        nk._check_decode_shapes(q, kp, vp, bt, sl, q[:B - 1])
    with pytest.raises(ValueError, match="q must be"):
        nk._check_decode_shapes(torch.empty((B, 4 * H, 2 * d), dtype=torch.bfloat16), kp, vp, bt, sl)
    with pytest.raises(ValueError, match="same geometry"):
        nk._check_decode_shapes(q, kp, pool(h=H + 1), bt, sl)

    rows = torch.empty((12, 4 * H, d), dtype=torch.bfloat16)
    qo = torch.empty(B + 1, dtype=torch.int64)
    nk._check_extend_shapes(rows, qo, ws, ws, offs, pl, rows.clone())
    with pytest.raises(ValueError, match="q_row_offsets"):
        nk._check_extend_shapes(rows, qo[:B], ws, ws, offs, pl)
    with pytest.raises(ValueError, match="share d"):
        nk._check_extend_shapes(rows, qo, torch.empty((40, H, 2 * d), dtype=torch.bfloat16), ws, offs, pl)
    with pytest.raises(ValueError, match="v_ws"):
        nk._check_extend_shapes(rows, qo, ws, ws[:39], offs, pl)

    bad_scale = nk.NVFP4Pool(torch.empty((pages, H, P, d // 2), dtype=torch.uint8),
                             torch.empty((pages, H, P, d // 32), dtype=torch.uint8))
    with pytest.raises(ValueError, match="pool scale"):
        nk._shape(bad_scale.scale, tuple(bad_scale.data.shape[:3]) + (bad_scale.data.shape[3] // 8,), "pool scale")
