"""Seeded synthetic paged-attention workloads.

Every array here is an *input*: lengths, block tables, slot mappings, the pool contents that stand for
earlier context, and this step's new K/V and Q.  The draw order per workload is fixed: lengths, then the
physical-block permutation, then pool contents, then new K/V, then Q.  bf16 tensors are carried as
uint16 bit patterns (numpy has no bfloat16); fp32 tensors as float32.

Geometry follows the pages: a pool of fixed-size physical blocks, one row per token slot, laid out
``[num_blocks, block_size, num_kv_heads, head_dim]`` per layer ("Paged Attention 基础 – 原理与实现进度",
§4 comparison table, memory-layout row, with the layer axis taken out as ADR 004 "Paged Attention
Serving Integration", Decision item 4, slices ``k_cache[i]`` per layer); block tables
``[num_seqs, max_blocks_per_seq]`` ("Paged Attention 基础", §3.1 C, block-table row); a slot is the
row index ``physical_block * block_size + offset`` into the pool viewed as ``[num_blocks*block_size, ...]``.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
FP32 = "fp32"

# Values per independently seeded chunk of a bulk normal fill.  Fixed, so that the drawn values do not
# depend on how many threads fill them.
_FILL_CHUNK = 1 << 22


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the uint16 bit patterns.

    Inputs must be finite (they are N(0,1) draws here).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> 16) & 1
    r += 0x7FFF
    r += b
    r >>= 16
    return r.astype(np.uint16)


def _storage_dtype(dtype: str):
    if dtype == BF16:
        return np.uint16
    if dtype == FP32:
        return np.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Small N(0,1) draw from ``rng`` in the storage type of ``dtype``."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_bits_from_f32(x).reshape(shape) if dtype == BF16 else x


def _bulk_normal(entropy: int, shape, dtype: str, threads: int | None = None) -> np.ndarray:
    """Large N(0,1) fill: chunk c of ``_FILL_CHUNK`` values comes from Philox seeded by child c of
    ``SeedSequence(entropy)``.  Filled by a thread pool; the values depend only on ``entropy``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=_storage_dtype(dtype))
    nchunks = max(1, -(-n // _FILL_CHUNK))
    children = np.random.SeedSequence(entropy).spawn(nchunks)

    def fill(c: int) -> None:
        lo = c * _FILL_CHUNK
        hi = min(n, lo + _FILL_CHUNK)
        g = np.random.Generator(np.random.Philox(children[c]))
        x = g.standard_normal(size=hi - lo, dtype=np.float32)
        out[lo:hi] = bf16_bits_from_f32(x) if dtype == BF16 else x

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nchunks == 1 or threads <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Step:
    """One write + attend step: new K/V go to ``slot_mapping``, then every sequence attends."""

    q: np.ndarray  # [total_q, H_q, D]
    k_new: np.ndarray  # [T, H_kv, D] (T == total_q here: one new row per query token)
    v_new: np.ndarray  # [T, H_kv, D]
    slot_mapping: np.ndarray  # [T] int32, -1 = no write
    context_lens: np.ndarray  # [N] int32, counts this step's tokens
    query_start_loc: np.ndarray  # [N+1] int32

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc)


@dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    block_tables: np.ndarray  # [N, max_blocks_per_seq] int32, -1 past each sequence's blocks
    k_pool: np.ndarray  # [num_blocks, block_size, H_kv, D], contents before the first step
    v_pool: np.ndarray
    steps: list = field(default_factory=list)
    scale: float = 0.0
    shared_prefix_blocks: int = 0
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4


def _slots_for(table_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Slot of each position of one sequence: its physical block's first row plus the offset."""
    return (table_row[positions // block_size].astype(np.int64) * block_size
            + positions % block_size).astype(np.int32)


def build_workload(rng: np.random.Generator, *, name: str, dtype: str, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, block_size: int, q_lens, context_lens,
                   shared_prefix_blocks: int = 0, pool_factor: float = 1.25,
                   description: str = "") -> Workload:
    """Tables, pool and one step for the given (already drawn) lengths.

    The pool holds ``ceil(pool_factor * blocks in use)`` blocks.  Block ids are the first ones of a
    random permutation of the pool, the shared prefix ids first, then each sequence's own ids dealt in
    order.  Every sequence's last ``q_len`` positions are this step's new tokens.
    """
    q_lens = np.asarray(q_lens, dtype=np.int64)
    context_lens = np.asarray(context_lens, dtype=np.int64)
    assert q_lens.shape == context_lens.shape
    assert np.all(q_lens >= 0) and np.all(q_lens <= context_lens)
    n_seqs = len(q_lens)
    bs = block_size
    nblk = -(-context_lens // bs)
    shared = int(shared_prefix_blocks)
    assert np.all(nblk >= shared)
    in_use = shared + int(np.sum(nblk - shared))
    num_blocks = max(1, int(math.ceil(pool_factor * in_use)))
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_nb = max(1, int(nblk.max(initial=1)))
    tables = np.full((n_seqs, max_nb), -1, dtype=np.int32)
    cursor = shared
    for s in range(n_seqs):
        own = int(nblk[s]) - shared
        tables[s, :shared] = perm[:shared]
        tables[s, shared:shared + own] = perm[cursor:cursor + own]
        cursor += own

    pool_shape = (num_blocks, bs, num_kv_heads, head_dim)
    k_pool = _bulk_normal(int(rng.integers(1 << 62)), pool_shape, dtype)
    v_pool = _bulk_normal(int(rng.integers(1 << 62)), pool_shape, dtype)

    total_q = int(q_lens.sum())
    k_new = _normal(rng, (total_q, num_kv_heads, head_dim), dtype)
    v_new = _normal(rng, (total_q, num_kv_heads, head_dim), dtype)
    q = _normal(rng, (total_q, num_q_heads, head_dim), dtype)

    qsl = np.zeros(n_seqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    slots = np.empty(total_q, dtype=np.int32)
    for s in range(n_seqs):
        pos = np.arange(context_lens[s] - q_lens[s], context_lens[s], dtype=np.int64)
        slots[qsl[s]:qsl[s + 1]] = _slots_for(tables[s], pos, bs)

    step = Step(q=q, k_new=k_new, v_new=v_new, slot_mapping=slots,
                context_lens=context_lens.astype(np.int32), query_start_loc=qsl)
    return Workload(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=bs, num_blocks=num_blocks, block_tables=tables,
                    k_pool=k_pool, v_pool=v_pool, steps=[step], scale=1.0 / math.sqrt(head_dim),
                    shared_prefix_blocks=shared, description=description)


# --------------------------------------------------------------------------------------------------
# The five workloads.  Seeds are 229000 + workload number.  "small" variants keep the geometry
# (heads, head_dim, block_size, dtype, sharing) and shrink counts and lengths so that the fp64 oracle
# finishes in seconds while still spanning several tiles, partitions and a ragged last block.
# --------------------------------------------------------------------------------------------------

def config_tiny(seed: int = 229001, shared_write: str = "skip") -> Workload:
    """The pages' worked example ("Paged Attention 基础", §2 block-table figure): block_size 16,
    sequence A on physical blocks [7, 3] and B on [7, 9] (block 7 shared as a prefix), 24 tokens each.
    Pool of 16 blocks, 4 q heads / 2 kv heads, head_dim 64, fp32.  Step 0 is the full causal prefill of
    both sequences (q_len 24 each); step 1 writes one more token per sequence and decodes it.

    ``shared_write`` says how B's prefill treats its first 16 tokens, which live in A's block 7:
    ``"skip"`` marks them slot -1 (a prefix hit), ``"rewrite"`` writes the identical rows again.
    """
    assert shared_write in ("skip", "rewrite")
    rng = np.random.default_rng(seed)
    bs, hq, hkv, d = 16, 4, 2, 64
    num_blocks = 16
    tables = np.array([[7, 3], [7, 9]], dtype=np.int32)
    pool_shape = (num_blocks, bs, hkv, d)
    k_pool = _normal(rng, pool_shape, FP32)
    v_pool = _normal(rng, pool_shape, FP32)

    # Prefill: A's 24 rows, then B's 8 own rows; B's first 16 rows are A's (same prompt prefix).
    ka = _normal(rng, (24, hkv, d), FP32)
    va = _normal(rng, (24, hkv, d), FP32)
    kb_own = _normal(rng, (8, hkv, d), FP32)
    vb_own = _normal(rng, (8, hkv, d), FP32)
    k_new = np.concatenate([ka, ka[:16], kb_own])
    v_new = np.concatenate([va, va[:16], vb_own])
    slots_a = np.concatenate([7 * bs + np.arange(16), 3 * bs + np.arange(8)])
    if shared_write == "skip":
        slots_b_prefix = np.full(16, -1)
    else:
        slots_b_prefix = 7 * bs + np.arange(16)
    slots_b = np.concatenate([slots_b_prefix, 9 * bs + np.arange(8)])
    q0 = _normal(rng, (48, hq, d), FP32)
    step0 = Step(q=q0, k_new=k_new, v_new=v_new,
                 slot_mapping=np.concatenate([slots_a, slots_b]).astype(np.int32),
                 context_lens=np.array([24, 24], dtype=np.int32),
                 query_start_loc=np.array([0, 24, 48], dtype=np.int32))

    # Decode: token 24 of each sequence lands in offset 8 of its second block.
    k1 = _normal(rng, (2, hkv, d), FP32)
    v1 = _normal(rng, (2, hkv, d), FP32)
    q1 = _normal(rng, (2, hq, d), FP32)
    step1 = Step(q=q1, k_new=k1, v_new=v1,
                 slot_mapping=np.array([3 * bs + 8, 9 * bs + 8], dtype=np.int32),
                 context_lens=np.array([25, 25], dtype=np.int32),
                 query_start_loc=np.array([0, 1, 2], dtype=np.int32))
    return Workload(name="tiny", dtype=FP32, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    block_size=bs, num_blocks=num_blocks, block_tables=tables, k_pool=k_pool,
                    v_pool=v_pool, steps=[step0, step1], scale=1.0 / math.sqrt(d),
                    shared_prefix_blocks=1,
                    description="worked example: A on [7,3], B on [7,9], bs 16, fp32, prefill 24 + decode 1")


def config_decode(seed: int = 229002, num_seqs: int = 64, ctx_range=(512, 4096),
                  dtype: str = BF16, block_size: int = 16) -> Workload:
    """Decode batch: q_len 1, context uniform in ``ctx_range``, 32 q / 8 kv heads, head_dim 128."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_range[0], ctx_range[1], size=num_seqs, endpoint=True)
    return build_workload(rng, name="decode", dtype=dtype, num_q_heads=32, num_kv_heads=8,
                          head_dim=128, block_size=block_size, q_lens=np.ones(num_seqs, np.int64),
                          context_lens=ctx,
                          description=f"decode {num_seqs} seqs q_len 1 ctx U{list(ctx_range)} GQA 32/8 D128 bs{block_size} {dtype}")


def config_mixed(seed: int = 229003, num_chunks: int = 8, chunk_len: int = 512,
                 prior_range=(0, 2048), num_decode: int = 56, decode_range=(1024, 8192),
                 dtype: str = BF16) -> Workload:
    """Chunked-prefill step: ``num_chunks`` chunks of ``chunk_len`` new tokens over a prior context
    uniform in ``prior_range``, then ``num_decode`` single-token sequences with context uniform in
    ``decode_range``.  32 q / 8 kv heads, head_dim 128, block_size 16."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(prior_range[0], prior_range[1], size=num_chunks, endpoint=True)
    dctx = rng.integers(decode_range[0], decode_range[1], size=num_decode, endpoint=True)
    q_lens = np.concatenate([np.full(num_chunks, chunk_len), np.ones(num_decode, np.int64)])
    ctx = np.concatenate([prior + chunk_len, dctx])
    return build_workload(rng, name="mixed", dtype=dtype, num_q_heads=32, num_kv_heads=8,
                          head_dim=128, block_size=16, q_lens=q_lens, context_lens=ctx,
                          description=f"mixed {num_chunks}x{chunk_len}-token chunks prior U{list(prior_range)} + {num_decode} decode ctx U{list(decode_range)} GQA 32/8 D128 bs16 {dtype}")


def config_spec(seed: int = 229004, num_seqs: int = 32, qlen_range=(4, 8),
                ctx_range=(8192, 32768), dtype: str = BF16) -> Workload:
    """Speculative multi-token decode: q_len uniform in ``qlen_range``, context uniform in
    ``ctx_range``, 64 q / 8 kv heads, head_dim 128, block_size 32."""
    rng = np.random.default_rng(seed)
    qlen = rng.integers(qlen_range[0], qlen_range[1], size=num_seqs, endpoint=True)
    ctx = rng.integers(ctx_range[0], ctx_range[1], size=num_seqs, endpoint=True)
    return build_workload(rng, name="spec", dtype=dtype, num_q_heads=64, num_kv_heads=8,
                          head_dim=128, block_size=32, q_lens=qlen, context_lens=ctx,
                          description=f"spec decode {num_seqs} seqs q_len U{list(qlen_range)} ctx U{list(ctx_range)} GQA 64/8 D128 bs32 {dtype}")


def config_prefix(seed: int = 229005, num_seqs: int = 256, shared_blocks: int = 128,
                  suffix_range=(64, 1024), dtype: str = BF16) -> Workload:
    """Prefix-sharing decode: every table starts with the same ``shared_blocks`` physical blocks
    (block_size 16), then a unique suffix of length uniform in ``suffix_range``.  q_len 1, MQA
    32 q / 1 kv head, head_dim 128.  The new token is the last suffix position."""
    rng = np.random.default_rng(seed)
    suffix = rng.integers(suffix_range[0], suffix_range[1], size=num_seqs, endpoint=True)
    ctx = shared_blocks * 16 + suffix
    return build_workload(rng, name="prefix", dtype=dtype, num_q_heads=32, num_kv_heads=1,
                          head_dim=128, block_size=16, q_lens=np.ones(num_seqs, np.int64),
                          context_lens=ctx, shared_prefix_blocks=shared_blocks,
                          description=f"prefix-sharing decode {num_seqs} seqs, {shared_blocks} shared blocks + suffix U{list(suffix_range)}, MQA 32/1 D128 bs16 {dtype}")


CONFIG_NAMES = ("tiny", "decode", "mixed", "spec", "prefix")


def make_config(name: str, size: str = "full", dtype: str | None = None) -> Workload:
    """Named workload at full size or at the small size the oracle finishes in seconds."""
    kw = {} if dtype is None else {"dtype": dtype}
    if name == "tiny":
        return config_tiny()
    if size == "full":
        return {"decode": config_decode, "mixed": config_mixed, "spec": config_spec,
                "prefix": config_prefix}[name](**kw)
    if size != "small":
        raise ValueError(size)
    if name == "decode":
        return config_decode(seed=229102, num_seqs=6, ctx_range=(1, 900), **kw)
    if name == "mixed":
        return config_mixed(seed=229103, num_chunks=2, chunk_len=70, prior_range=(0, 300),
                            num_decode=5, decode_range=(100, 1500), **kw)
    if name == "spec":
        return config_spec(seed=229104, num_seqs=4, ctx_range=(300, 2500), **kw)
    if name == "prefix":
        return config_prefix(seed=229105, num_seqs=12, shared_blocks=8, suffix_range=(1, 300), **kw)
    raise ValueError(name)


def subset_workload(w: Workload, seqs) -> Workload:
    """The same pool and step restricted to the sequences `seqs` (in that order): their table rows,
    lengths, query rows, new K/V rows and slots.  Used to time the prefill or decode part of a mixed step
    on its own."""
    seqs = [int(s) for s in seqs]
    out_steps = []
    for st in w.steps:
        qsl = st.query_start_loc
        rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs]).astype(np.int64)
        q_lens = np.array([qsl[s + 1] - qsl[s] for s in seqs], dtype=np.int64)
        new_qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
        new_qsl[1:] = np.cumsum(q_lens)
        out_steps.append(Step(q=st.q[rows], k_new=st.k_new[rows], v_new=st.v_new[rows],
                              slot_mapping=st.slot_mapping[rows], context_lens=st.context_lens[seqs],
                              query_start_loc=new_qsl))
    return Workload(name=w.name, dtype=w.dtype, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                    head_dim=w.head_dim, block_size=w.block_size, num_blocks=w.num_blocks,
                    block_tables=w.block_tables[seqs], k_pool=w.k_pool, v_pool=w.v_pool, steps=out_steps,
                    scale=w.scale, shared_prefix_blocks=w.shared_prefix_blocks,
                    description=w.description)
