"""CPU oracle for the paged cache manager: block allocator, block tables, slot mapping, shared blocks.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` (and ``bench.py``'s CPU-baseline leg) may import this module.
The product's manager is C++ inside the HIP library; the two share no code.

What the pages fix, and where:

* The pool is a set of fixed-size physical blocks; a sequence owns a list of them (its block table) and
  grows by taking one more block when its last one is full, with no data movement ("Paged Attention 基础
  – 原理与实现进度", §1 problems 1 and 2; §3.1 A names the block allocator, the block table and the slot
  mapping; §3.2 the block manager's allocate/free).
* Several tables may list the same physical block: prefix caching (same page, §1 problem 3 and the §2
  figure, where sequences A and B both start with block 7).
* One ``update`` call serves both a fresh sequence and the extension of an existing one, block tables are
  kept per sequence id and released by ``free(seq_id)``, and prefix reuse goes through ``add_prefix`` /
  ``try_get_prefix_blocks`` (ADR 004 "Paged Attention Serving Integration", Decision 5 and Consequences).
* A paged kernel needs a cache manager that copies and updates the pages ("Any plan for support paged
  attention?", tridao's and curry-zzl's comments).

Readings where the pages are silent (listed in the design notes):

* A slot is ``physical_block * block_size + offset`` (the attention oracle's reading).
* Allocation takes the lowest-numbered free block, so that the allocation sequence is a pure function of
  the operations (any policy is valid; this one is easy to state and to compare).
* A block is shared by reference counting: every sequence and every registered prefix listing it holds
  one reference; it returns to the free set when the count reaches zero.
* Appending into a last block that is partly filled and shared first copies that block to a fresh one
  (copy on write), so the other owners never see the new rows.  At most one copy per append: only the
  last block of a sequence can be partly filled.
* Operations that cannot complete (no free block, unknown sequence, ...) raise and change nothing.
"""

from __future__ import annotations

import numpy as np


class CacheError(Exception):
    """An operation the manager refuses; the manager's state is unchanged."""


class BlockManagerOracle:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise CacheError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free = set(range(num_blocks))
        self.seqs: dict[int, dict] = {}
        self.prefixes: dict[int, dict] = {}

    # -- allocation primitives ------------------------------------------------------------------------
    def _take(self) -> int:
        b = min(self.free)
        self.free.remove(b)
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.add(b)

    def num_free(self) -> int:
        return len(self.free)

    def seq_len(self, seq_id: int) -> int:
        return self.seqs[seq_id]["len"] if seq_id in self.seqs else -1

    # -- the update call: fresh sequence or extension ------------------------------------------------
    def append(self, seq_id: int, n: int):
        """Add ``n`` tokens at the end of ``seq_id`` (created if new).  Returns (slots, cow) where slots
        are the pool rows of the new positions, in order, and cow is None or (src_block, dst_block), the
        copy the caller must make before writing the slots."""
        if n < 0:
            raise CacheError("negative token count")
        seq = self.seqs.get(seq_id, {"blocks": [], "len": 0})
        blocks, length, bs = list(seq["blocks"]), seq["len"], self.block_size
        blocks_after = -(-(length + n) // bs)
        need = blocks_after - len(blocks)
        cow_needed = n > 0 and length % bs != 0 and self.ref[blocks[-1]] > 1
        if need + int(cow_needed) > len(self.free):
            raise CacheError("out of blocks")
        cow = None
        if cow_needed:
            src = blocks[-1]
            dst = self._take()
            self._release(src)
            blocks[-1] = dst
            cow = (src, dst)
        for _ in range(need):
            blocks.append(self._take())
        slots = [blocks[p // bs] * bs + p % bs for p in range(length, length + n)]
        self.seqs[seq_id] = {"blocks": blocks, "len": length + n}
        return slots, cow

    def free_seq(self, seq_id: int) -> None:
        if seq_id not in self.seqs:
            raise CacheError("unknown sequence")
        for b in self.seqs.pop(seq_id)["blocks"]:
            self._release(b)

    def fork(self, parent: int, child: int) -> None:
        """``child`` starts as a copy of ``parent`` that shares every block."""
        if parent not in self.seqs or child in self.seqs:
            raise CacheError("fork needs a known parent and a new child")
        p = self.seqs[parent]
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs[child] = {"blocks": list(p["blocks"]), "len": p["len"]}

    # -- prefix registry ------------------------------------------------------------------------------
    def add_prefix(self, key: int, seq_id: int, tokens: int) -> None:
        """Register the blocks holding the first ``tokens`` tokens of ``seq_id`` under ``key``; the
        registry keeps its own reference, so they outlive the sequence."""
        if key in self.prefixes or seq_id not in self.seqs:
            raise CacheError("prefix key taken or unknown sequence")
        seq = self.seqs[seq_id]
        if tokens <= 0 or tokens > seq["len"]:
            raise CacheError("prefix longer than the sequence")
        blocks = seq["blocks"][: -(-tokens // self.block_size)]
        for b in blocks:
            self.ref[b] += 1
        self.prefixes[key] = {"blocks": list(blocks), "tokens": tokens}

    def attach_prefix(self, key: int, seq_id: int) -> int:
        """A new sequence starts with the registered prefix's blocks (shared).  Returns the number of
        tokens it now holds; 0 when the key is unknown (nothing changes)."""
        if seq_id in self.seqs:
            raise CacheError("the sequence already exists")
        pre = self.prefixes.get(key)
        if pre is None:
            return 0
        for b in pre["blocks"]:
            self.ref[b] += 1
        self.seqs[seq_id] = {"blocks": list(pre["blocks"]), "len": pre["tokens"]}
        return pre["tokens"]

    def drop_prefix(self, key: int) -> None:
        if key not in self.prefixes:
            raise CacheError("unknown prefix")
        for b in self.prefixes.pop(key)["blocks"]:
            self._release(b)

    # -- per-step metadata ----------------------------------------------------------------------------
    def build_tables(self, seq_ids, max_blocks_per_seq: int):
        """Block-table rows (padded with -1) and context lengths for a batch of sequences."""
        tables = np.full((len(seq_ids), max_blocks_per_seq), -1, dtype=np.int32)
        lens = np.zeros(len(seq_ids), dtype=np.int32)
        for i, sid in enumerate(seq_ids):
            if sid not in self.seqs:
                raise CacheError("unknown sequence")
            blocks = self.seqs[sid]["blocks"]
            if len(blocks) > max_blocks_per_seq:
                raise CacheError("table row too short")
            tables[i, : len(blocks)] = blocks
            lens[i] = self.seqs[sid]["len"]
        return tables, lens


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs) -> tuple[np.ndarray, np.ndarray]:
    """The copy-on-write step on the pools: block dst takes the contents of block src, pair by pair in
    order (whole blocks, every row and head, bit for bit)."""
    k, v = k_pool.copy(), v_pool.copy()
    for src, dst in pairs:
        k[dst] = k[src]
        v[dst] = v[src]
    return k, v
