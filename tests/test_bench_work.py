"""The algorithmic work bench.py prices its rooflines with, checked against independent counts on small
workloads: causal (query, key) pairs by brute force over the bottom-right mask, unique K/V bytes as the set of
physical (block, row) positions some sequence reads (shared blocks count once by construction), logical bytes
per sequence, Q/O and block-table bytes, and the rows the slot mapping writes."""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import config_tiny, make_config  # noqa: E402


def independent_counts(w):
    st = w.steps[0]
    e, hq, hkv, d, bs = w.elem_bytes, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    row = hkv * d * e
    pairs = 0
    rows_read = set()
    logical = 0
    for s in range(w.num_seqs):
        L = int(st.context_lens[s])
        n = int(st.query_start_loc[s + 1] - st.query_start_loc[s])
        for i in range(n):
            for p in range(L):
                if p <= L - n + i:
                    pairs += 1
        for p in range(L):
            rows_read.add((int(w.block_tables[s, p // bs]), p % bs))
        logical += 2 * row * L
    total_q = int(st.query_start_loc[-1])
    qo = 2 * total_q * hq * d * e
    tables = sum(4 * (-(-int(L) // bs)) for L in st.context_lens)
    writes = sum(1 for x in st.slot_mapping if x >= 0)
    return dict(pairs=pairs, flops=4 * d * hq * pairs, unique=2 * row * len(rows_read) + qo + tables,
                logical=logical + qo + tables, write_bytes=2 * 2 * writes * row, total_q=total_q)


@pytest.mark.parametrize("make", [lambda: config_tiny(shared_write="skip"), lambda: config_tiny(shared_write="rewrite"),
                                  lambda: make_config("prefix", "small"), lambda: make_config("mixed", "small")],
                         ids=["tiny-skip", "tiny-rewrite", "prefix-small", "mixed-small"])
def test_algorithmic_work_matches_independent_counts(make):
    w = make()
    got = bench.algorithmic_work(w)
    ref = independent_counts(w)
    assert got["pairs"] == ref["pairs"]
    assert got["flops"] == ref["flops"]
    assert got["attn_bytes_unique"] == ref["unique"]
    assert got["attn_bytes_logical"] == ref["logical"]
    assert got["write_bytes"] == ref["write_bytes"]
    assert got["total_q"] == ref["total_q"]
