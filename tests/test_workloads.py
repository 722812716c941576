"""Seeded input generators: determinism, pool sizing, table structure, sharing, bf16 rounding."""

import numpy as np
import pytest
import torch

from workloads import bf16_bits_from_f32, make_config, config_prefix, config_decode
from workloads.synth import _bulk_normal


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0, 1e-40], np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bulk_fill_independent_of_threads():
    a = _bulk_normal(123, (3, 1 << 21), "bf16", threads=1)
    b = _bulk_normal(123, (3, 1 << 21), "bf16", threads=8)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["decode", "mixed", "spec", "prefix"])
def test_small_configs_structure(name):
    w1 = make_config(name, "small")
    w2 = make_config(name, "small")
    st = w1.steps[0]
    assert np.array_equal(w1.k_pool, w2.k_pool) and np.array_equal(st.q, w2.steps[0].q)
    L = st.context_lens.astype(np.int64)
    n = np.diff(st.query_start_loc)
    assert np.all(n <= L) and st.query_start_loc[0] == 0
    nblk = -(-L // w1.block_size)
    shared = w1.shared_prefix_blocks
    in_use = shared + int(np.sum(nblk - shared))
    assert w1.num_blocks == int(np.ceil(1.25 * in_use))
    used = []
    for s in range(w1.num_seqs):
        row = w1.block_tables[s]
        assert np.all(row[:nblk[s]] >= 0) and np.all(row[nblk[s]:] == -1)
        assert np.array_equal(row[:shared], w1.block_tables[0][:shared])
        used.extend(row[shared:nblk[s]].tolist())
    used.extend(w1.block_tables[0][:shared].tolist())
    assert len(set(used)) == len(used) == in_use  # no block owned twice
    # each new token's slot is inside the sequence's own last blocks, and slots are distinct
    assert len(set(st.slot_mapping.tolist())) == len(st.slot_mapping)
    for s in range(w1.num_seqs):
        for t in range(st.query_start_loc[s], st.query_start_loc[s + 1]):
            pos = L[s] - n[s] + (t - st.query_start_loc[s])
            blk, off = divmod(int(st.slot_mapping[t]), w1.block_size)
            assert blk == w1.block_tables[s][pos // w1.block_size] and off == pos % w1.block_size


def test_full_config_metadata_only():
    # lengths and tables of the full workloads without drawing the big pools twice
    w = config_decode()
    L = w.steps[0].context_lens
    assert w.num_seqs == 64 and L.min() >= 512 and L.max() <= 4096
    assert w.k_pool.shape == (w.num_blocks, 16, 8, 128) and w.k_pool.dtype == np.uint16
    p = config_prefix(num_seqs=16)
    assert np.all(p.block_tables[:, :128] == p.block_tables[0, :128])
    assert np.all(p.steps[0].context_lens >= 2048 + 64)
