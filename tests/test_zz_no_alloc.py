"""The allocation-free decode entry point against the workspace one.

nvfp4_paged_decode_attn_noalloc runs the same partial and merge kernels as
nvfp4_paged_decode_attn with the partials in the library's static scratch
array instead of a caller workspace. Two calls in a row on one GPU, the
second smaller than the first (the array keeps the first call's partials),
each compared bit for bit with the workspace entry point at the same split
count, and with the oracle at the decode tolerance.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import nvfp4 as onv

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 2e-3


@pytest.fixture(scope="module")
def nk():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import nvfp4_quantized_paged_amd as m
    m.lib()
    return m


def _problem(nk, wl, lens):
    inp = synth.host_uniform_decode(wl)
    inp.seq_lens[:] = np.asarray(lens, np.int32)
    H, P, d = wl.num_kv_heads, wl.page_size, wl.head_dim
    kp = nk.NVFP4Pool.empty(inp.num_pages, H, P, d)
    vp = nk.NVFP4Pool.empty(inp.num_pages, H, P, d)
    nk.nvfp4_kv_quantize(synth.to_device_bf16(inp.k), synth.to_device_bf16(inp.v), synth.to_device(inp.slot_mapping),
                         kp, vp)
    kd, ks = onv.empty_cache(inp.num_pages, H, P, d)
    vd, vs = onv.empty_cache(inp.num_pages, H, P, d)
    onv.write_cache(kd, ks, inp.k, inp.slot_mapping)
    onv.write_cache(vd, vs, inp.v, inp.slot_mapping)
    ref, mass = oatt.paged_decode(inp.q, onv.dequant_cache(kd, ks), onv.dequant_cache(vd, vs), inp.block_tables,
                                  inp.seq_lens, wl.sm_scale)
    return inp, kp, vp, ref, mass


def _check(out, ref, mass, what):
    got = out.float().cpu().numpy().astype(np.float64)
    e = np.abs(got - ref) / np.maximum(1.0, mass)
    print(f"  {what}: max e {e.max():.3e} mean e {e.mean():.3e}", flush=True)
    assert np.all(np.isfinite(got)) and e.max() <= TOL_MAX and e.mean() <= TOL_MEAN, what


def test_noalloc_decode_matches_the_workspace_entry_point(nk):
    assert nk.nvfp4_paged_decode_noalloc_scratch_bytes() == 32 << 20
    cases = [
        # large first: 6 sequences, 40 / 8 heads, ragged lengths, the library's split count
        (synth.Workload(300, "noalloc-large", 6, 40, 8, 128, 64, 3000, True, 0), [3000, 2999, 1, 0, 1500, 2048], 0),
        # then smaller: fewer sequences, heads, channels and splits than the call before
        (synth.Workload(301, "noalloc-small", 2, 8, 2, 64, 16, 500, False, 3), [500, 77], 3),
    ]
    for wl, lens, splits in cases:
        print(f"case noalloc decode: {wl.name} B {wl.batch} Hq {wl.num_q_heads} Hkv {wl.num_kv_heads} "
              f"d {wl.head_dim} P {wl.page_size} lens {lens} splits {splits}", flush=True)
        inp, kp, vp, ref, mass = _problem(nk, wl, lens)
        q, bt, sl = synth.to_device_bf16(inp.q), synth.to_device(inp.block_tables), synth.to_device(inp.seq_lens)
        S = splits or nk.nvfp4_paged_decode_num_splits(wl.batch, wl.num_kv_heads, bt.shape[1], wl.page_size)
        need = nk.nvfp4_paged_decode_workspace_bytes(wl.batch, wl.num_q_heads, wl.head_dim, S)
        assert need <= nk.nvfp4_paged_decode_noalloc_scratch_bytes()
        out_ws = nk.nvfp4_paged_decode_attn(q, kp, vp, bt, sl, wl.sm_scale, num_splits=S)
        out_na = torch.full_like(q, float("nan"))
        nk.nvfp4_paged_decode_attn_noalloc(q, kp, vp, bt, sl, wl.sm_scale, out_na, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), f"{wl.name}: differs from workspace call"
        _check(out_na, ref, mass, wl.name)
