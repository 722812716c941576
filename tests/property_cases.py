"""Hypothesis strategies for random paged-attention cases (the property tier of the tests).

A case is a set of lengths and a geometry; the inputs themselves come from ``workloads.build_workload``
with a drawn seed (random block permutation, N(0,1) values).  Sequences may share their first blocks
(prefix caching, "Paged Attention 基础 – 原理与实现进度", §2 figure: two sequences starting with one
physical block); a sharer's new tokens then always lie after the shared blocks, so no slot is written
twice in one step.
"""

from __future__ import annotations

import numpy as np
from hypothesis import strategies as st

from workloads import build_workload


@st.composite
def lengths(draw, max_seqs: int, max_prior: int, q_len_choices, shared_max: int, block_size: int):
    """(q_lens, context_lens, shared_blocks): every context holds its q_len new tokens, and when blocks
    are shared every sequence's prior context covers them."""
    nseq = draw(st.integers(1, max_seqs))
    shared = draw(st.integers(0, shared_max))
    q_lens, ctx = [], []
    for _ in range(nseq):
        n = draw(q_len_choices)
        prior = draw(st.integers(shared * block_size, max(shared * block_size, max_prior)))
        q_lens.append(n)
        ctx.append(prior + n)
    return q_lens, ctx, shared


@st.composite
def gpu_case(draw, dtype: str):
    """Geometry and lengths at the library's supported sizes: groups {1, 2, 4, 8, 32}, block sizes
    {16, 32}, head_dim {64, 128}; decode, speculative and chunk-sized q_lens (0 included)."""
    group = draw(st.sampled_from([1, 2, 4, 8, 32]))
    hkv = draw(st.sampled_from([1, 2, 4] if group <= 8 else [1, 2]))
    bs = draw(st.sampled_from([16, 32]))
    d = draw(st.sampled_from([64, 128]))
    q_len = st.one_of(st.integers(0, 2), st.integers(1, 9), st.integers(1, 300))
    q_lens, ctx, shared = draw(lengths(6, 1500, q_len, 3, bs))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    w = build_workload(np.random.default_rng(seed), name="property", dtype=dtype, num_q_heads=group * hkv,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, q_lens=q_lens, context_lens=ctx,
                       shared_prefix_blocks=shared)
    w.description = (f"seed={seed} G={group} Hkv={hkv} D={d} bs={bs} shared={shared} "
                     f"q_lens={q_lens} ctx={ctx}")
    return w


@st.composite
def long_case(draw, dtype: str):
    """Few sequences over long contexts (3 K - 9 K keys) with decode-like and speculative q_lens (small row
    tiles), at the supported geometry: with a small work-item target the partitions are long and every split
    tile ends on late pieces."""
    group = draw(st.sampled_from([1, 2, 4, 8]))
    hkv = draw(st.sampled_from([1, 2]))
    bs = draw(st.sampled_from([16, 32]))
    d = draw(st.sampled_from([64, 128]))
    q_lens, ctx, shared = draw(lengths(4, 9000, st.integers(1, 8), 2, bs))
    ctx = [max(c, 3000 + n) for c, n in zip(ctx, q_lens)]
    seed = draw(st.integers(0, 2 ** 32 - 1))
    w = build_workload(np.random.default_rng(seed), name="property-long", dtype=dtype, num_q_heads=group * hkv,
                       num_kv_heads=hkv, head_dim=d, block_size=bs, q_lens=q_lens, context_lens=ctx,
                       shared_prefix_blocks=shared)
    w.description = (f"seed={seed} G={group} Hkv={hkv} D={d} bs={bs} shared={shared} "
                     f"q_lens={q_lens} ctx={ctx}")
    return w


@st.composite
def tiny_case(draw, dtype: str):
    """Tiny geometry for scalar brute force: head_dim 2..8, block sizes 1..8, contexts up to 30."""
    group = draw(st.sampled_from([1, 2, 3, 4]))
    hkv = draw(st.sampled_from([1, 2]))
    bs = draw(st.sampled_from([1, 2, 4, 8]))
    d = draw(st.integers(2, 8))
    q_len = st.integers(0, 6)
    q_lens, ctx, shared = draw(lengths(3, 24, q_len, 2, bs))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    w = build_workload(np.random.default_rng(seed), name="property-tiny", dtype=dtype,
                       num_q_heads=group * hkv, num_kv_heads=hkv, head_dim=d, block_size=bs, q_lens=q_lens,
                       context_lens=ctx, shared_prefix_blocks=shared)
    w.description = f"seed={seed} G={group} Hkv={hkv} D={d} bs={bs} shared={shared} q_lens={q_lens} ctx={ctx}"
    return w
