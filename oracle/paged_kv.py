"""CPU oracle for paged KV-cache writes and paged attention (float64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and its binding) never calls
it, and it shares no code with that path.

What it computes, step by step, in the pages' order:

* Write.  Each new K/V row goes to the pool row named by its slot; a slot is a physical block index
  times the block size plus the offset inside the block ("Paged Attention 基础 – 原理与实现进度", §3.2
  status table: block tables, slot mapping and context lengths are the per-step metadata; "Any plan for
  support paged attention?", tridao's comment: prefill K/V come out of the projections as one
  contiguous blob that is then copied into blocks; ADR 004 "Paged Attention Serving Integration",
  Consequences: one ``update`` call covers a fresh allocation and the extension of a sequence).
* Gather.  A sequence's K/V is the concatenation, in block-table order, of the physical blocks its
  table lists, cut to its context length ("Paged Attention 基础", §2: block-table figure and attention
  steps 1 to 4 for token q = 23 of sequence A on blocks [7, 3]).
* Attend.  ``softmax(Q K^T * scale) V`` with a causal mask over the concatenated keys ("Paged Attention
  基础", §2, step 5; the scale is the softmax_scale in zhaoyang-star's comment on the flash-attention
  issue).  Several query tokens per sequence are allowed (ADR 004, Consequences: prefill and decode
  share one call; flash-attention issue, donglinz: speculative decoding needs several tokens per
  sequence).  Grouped heads map query head h to kv head h // (H_q / H_kv) (zhaoyang-star: MQA/GQA).

Readings where the pages are silent (each is listed with its reason in the design notes):

* ``context_lens[s]`` counts every cached token including this step's new ones (write first, then
  attend: ADR 004, Decision 4 writes K/V, then reads through the paged call).
* The ``n`` query tokens of a sequence are its last ``n`` positions; query i sees keys
  ``0 .. L - n + i`` (bottom-right causal alignment; the worked example is the n = L case).
* A negative slot means "no write".  Block-table entries past ``ceil(L / block_size)`` are never read.
* The softmax uses the natural exponential; results are in float64.
"""

from __future__ import annotations

import math

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64.  bf16 values are stored as uint16 bit patterns: the
    value is the float32 whose upper 16 bits are those bits and whose lower 16 bits are zero."""
    if dtype == BF16:
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == FP32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------------------------- write

def slot_to_block_offset(slot: int, block_size: int) -> tuple[int, int]:
    """Physical block and row inside it for a slot (slot = block * block_size + offset)."""
    return slot // block_size, slot % block_size


def kv_write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             slot_mapping: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Copies of the pools ``[num_blocks, block_size, H_kv, D]`` with row t of ``k_new``/``v_new``
    ``[T, H_kv, D]`` stored at ``slot_mapping[t]``; negative slots are skipped.  Values are copied in
    their stored type, bit for bit.  Tokens are applied in order, so with repeated slots the last one
    stays (repeated slots in one write are outside the supported inputs)."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    block_size = k_pool.shape[1]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = slot_to_block_offset(slot, block_size)
        k_out[blk, off] = k_new[t]
        v_out[blk, off] = v_new[t]
    return k_out, v_out


# --------------------------------------------------------------------------------------------- gather

def logical_block_count(context_len: int, block_size: int) -> int:
    """Blocks a sequence of ``context_len`` tokens occupies: the last one may be partly filled."""
    return -(-context_len // block_size)


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, context_len: int) -> np.ndarray:
    """One sequence's cached rows ``[context_len, H_kv, D]``, in position order: the physical blocks
    listed in its block table, concatenated in table order and cut to ``context_len`` rows."""
    block_size = pool.shape[1]
    nb = logical_block_count(context_len, block_size)
    if nb == 0:
        return pool[:0, 0]
    blocks = [pool[int(table_row[j])] for j in range(nb)]
    return np.concatenate(blocks, axis=0)[:context_len]


# --------------------------------------------------------------------------------------------- attend

def kv_head_of(q_head: int, group: int) -> int:
    """kv head read by a query head when ``group`` query heads share one kv head."""
    return q_head // group


def last_visible_key(i: int, n: int, context_len: int) -> int:
    """Position of the last key query i (of n new tokens) may attend: the new tokens are the last n
    positions, so query i sits at ``context_len - n + i`` and sees every key up to it."""
    return context_len - n + i


def causal_mask(n: int, context_len: int) -> np.ndarray:
    """Boolean ``[n, context_len]``: True where query i may attend key p."""
    mask = np.zeros((n, context_len), dtype=bool)
    for i in range(n):
        mask[i, :last_visible_key(i, n, context_len) + 1] = True
    return mask


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of scores that may hold -inf (each row has at least one finite entry)."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)


def head_scores(qh: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """Scaled dot products ``[n, L]`` of one head's query rows ``[n, D]`` with its keys ``[L, D]``."""
    return (qh @ kh.T) * scale


def attend_head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, mask: np.ndarray,
                scale: float) -> np.ndarray:
    """One head: masked scores, row softmax, weighted sum of the value rows.  ``[n, D]``."""
    scores = np.where(mask, head_scores(qh, kh, scale), -np.inf)
    return softmax_rows(scores) @ vh


def attend_sequence(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Causal attention of one sequence's ``n`` new query rows ``[n, H_q, D]`` over its ``L`` cached
    rows ``keys``/``values`` ``[L, H_kv, D]`` (float64).  Returns ``[n, H_q, D]``."""
    n, num_q_heads, _ = q.shape
    context_len, num_kv_heads, _ = keys.shape
    assert 0 <= n <= context_len
    group = num_q_heads // num_kv_heads
    out = np.zeros(q.shape, dtype=np.float64)
    if n == 0:
        return out
    mask = causal_mask(n, context_len)
    for h in range(num_q_heads):
        g = kv_head_of(h, group)
        out[:, h, :] = attend_head(q[:, h, :], keys[:, g, :], values[:, g, :], mask, scale)
    return out


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
                    context_lens: np.ndarray, query_start_loc: np.ndarray, scale: float, dtype: str,
                    seqs=None) -> np.ndarray:
    """Paged attention for every sequence (or only ``seqs``).

    ``q`` ``[total_q, H_q, D]`` packs each sequence's new query rows at
    ``query_start_loc[s] : query_start_loc[s+1]``; ``k_pool``/``v_pool`` ``[num_blocks, block_size,
    H_kv, D]`` hold the cache after this step's write; ``block_tables[s]`` lists sequence s's physical
    blocks; ``context_lens[s]`` is its cached length.  Returns float64 ``[total_q, H_q, D]``; rows of
    sequences not in ``seqs`` stay zero."""
    num_q_heads = q.shape[1]
    num_kv_heads = k_pool.shape[2]
    if num_q_heads % num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    out = np.zeros(q.shape, dtype=np.float64)
    which = range(len(context_lens)) if seqs is None else seqs
    for s in which:
        lo, hi = int(query_start_loc[s]), int(query_start_loc[s + 1])
        length = int(context_lens[s])
        if hi == lo:
            continue
        keys = to_float64(gather_sequence(k_pool, block_tables[s], length), dtype)
        values = to_float64(gather_sequence(v_pool, block_tables[s], length), dtype)
        out[lo:hi] = attend_sequence(to_float64(q[lo:hi], dtype), keys, values, scale)
    return out


def run_step(k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray, step, scale: float,
             dtype: str, seqs=None):
    """One write-then-attend step; ``step`` carries ``k_new, v_new, slot_mapping, q, context_lens,
    query_start_loc``.  Returns ``(k_pool', v_pool', out_f64)``."""
    k2, v2 = kv_write(k_pool, v_pool, step.k_new, step.v_new, step.slot_mapping)
    out = paged_attention(step.q, k2, v2, block_tables, step.context_lens, step.query_start_loc,
                          scale, dtype, seqs=seqs)
    return k2, v2, out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
