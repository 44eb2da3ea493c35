"""Determinism and structure of the seeded synthetic inputs."""
import numpy as np

import synth


def test_uniform_decode_is_deterministic_and_well_formed():
    wl = synth.WORKLOADS[1]
    a = synth.host_uniform_decode(wl)
    b = synth.host_uniform_decode(wl)
    for name in ("k", "v", "q", "block_tables", "slot_mapping"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert a.k.shape == (256, 1, 64) and a.q.shape == (1, 4, 64)
    assert sorted(a.block_tables.reshape(-1).tolist()) == list(range(16))
    assert len(set(a.slot_mapping.tolist())) == 256


def test_outlier_channels():
    wl = synth.WORKLOADS[2]
    inp = synth.host_uniform_decode(wl, context=64, batch=2)
    x = synth.bf16_bits_to_f64(inp.k).reshape(-1, 8 * 128)
    big = np.abs(x).max(axis=0) > 8
    assert 15 <= big.sum() <= 20        # 20 channels scaled by 20


def test_agentic_shared_prefix_structure():
    wl = synth.WORKLOADS[5]
    a = synth.host_agentic(wl, batch=6, len_min=40, len_max=90, shared_prefix=32, chunk=10)
    P = wl.page_size
    n_shared = 32 // P
    for b in range(6):
        assert np.array_equal(a.block_tables[b, :n_shared], a.shared_pages)
    shared = set(a.shared_pages.tolist())
    assert not any(int(s) // P in shared for s in a.slot_chunk)
    assert a.k_cached.shape[0] == 32 + int((a.cached_lens - 32).sum())
    assert a.k_chunk.shape[0] == 6 * 10
    assert np.array_equal(np.diff(a.ws_row_offsets), a.seq_lens.astype(np.int64))
    used = set()
    for b in range(6):
        npg = -(-int(a.seq_lens[b]) // P)
        used.update(a.block_tables[b, :npg].tolist())
    assert len(used) == a.num_pages
