"""Pins of the cache-manager oracle (oracle/block_manager.py) against things other than itself:

* the sharing structure of the pages' worked example ("Paged Attention 基础", §2: A on [7, 3], B on
  [7, 9], block 7 shared), with block ids up to renaming;
* a brute-force paged store: every appended token gets a unique id written at the slot the manager
  returns (after its copy-on-write copy, if any); after every operation each sequence must read back,
  through its block table, exactly the ids it holds, and each registered prefix its own ids;
* reference counts recomputed from the owners, the free set, block counts per length;
* all-or-nothing failures; everything returns to the free set at the end;
* planted mistakes in the oracle (no copy on write, an off-by-one slot, releasing shared blocks, sharing
  without references) each break a pin.
"""

import random

import numpy as np
import pytest

from oracle.block_manager import BlockManagerOracle, CacheError, copy_blocks


class PagedStore:
    """A pool of token ids driven by a manager; the reference for what each sequence must read."""

    def __init__(self, mgr):
        self.m = mgr
        self.bs = mgr.block_size
        self.pool = np.full(mgr.num_blocks * self.bs, -1, dtype=np.int64)
        self.expect = {}
        self.expect_prefix = {}
        self.next_id = 0

    def append(self, sid, n):
        slots, cow = self.m.append(sid, n)
        if cow is not None:
            src, dst = cow
            self.pool[dst * self.bs:(dst + 1) * self.bs] = self.pool[src * self.bs:(src + 1) * self.bs]
        ids = list(range(self.next_id, self.next_id + n))
        self.next_id += n
        assert len(slots) == n and len(set(slots)) == n
        self.pool[np.asarray(slots, dtype=np.int64)] = ids
        self.expect[sid] = self.expect.get(sid, []) + ids
        return slots, cow

    def fork(self, parent, child):
        self.m.fork(parent, child)
        self.expect[child] = list(self.expect[parent])

    def free(self, sid):
        self.m.free_seq(sid)
        del self.expect[sid]

    def add_prefix(self, key, sid, tokens):
        self.m.add_prefix(key, sid, tokens)
        self.expect_prefix[key] = self.expect[sid][:tokens]

    def attach(self, key, sid):
        got = self.m.attach_prefix(key, sid)
        if got:
            self.expect[sid] = list(self.expect_prefix[key])
        return got

    def drop_prefix(self, key):
        self.m.drop_prefix(key)
        del self.expect_prefix[key]

    def rows(self, blocks, length):
        return [blocks[p // self.bs] * self.bs + p % self.bs for p in range(length)]

    def check(self):
        m = self.m
        owners = [0] * m.num_blocks
        for sid, seq in m.seqs.items():
            assert len(seq["blocks"]) == -(-seq["len"] // self.bs)
            got = self.pool[np.asarray(self.rows(seq["blocks"], seq["len"]), dtype=np.int64)].tolist()
            assert got == self.expect[sid], f"sequence {sid} reads {got[:8]}... expected {self.expect[sid][:8]}..."
            for b in seq["blocks"]:
                owners[b] += 1
        for key, pre in m.prefixes.items():
            got = self.pool[np.asarray(self.rows(pre["blocks"], pre["tokens"]), dtype=np.int64)].tolist()
            assert got == self.expect_prefix[key]
            for b in pre["blocks"]:
                owners[b] += 1
        assert owners == m.ref
        assert m.free == {b for b in range(m.num_blocks) if owners[b] == 0}


def test_worked_example_structure():
    """bs 16: A holds 24 tokens on two blocks; B starts with A's first block (registered as a 16-token
    prefix) and adds 8 tokens in a block of its own; decoding one token each lands at offset 8 of each
    sequence's second block."""
    st = PagedStore(BlockManagerOracle(16, 16))
    st.append("A", 24)
    st.add_prefix(1, "A", 16)
    assert st.attach(1, "B") == 16
    slots_b, cow = st.append("B", 8)
    assert cow is None  # the shared block is full: nothing to copy
    tables, lens = st.m.build_tables(["A", "B"], 4)
    assert tables[0, 0] == tables[1, 0] and tables[0, 1] != tables[1, 1]
    assert list(lens) == [24, 24]
    assert slots_b == [tables[1, 1] * 16 + i for i in range(8)]
    sa, _ = st.append("A", 1)
    sb, _ = st.append("B", 1)
    assert sa == [tables[0, 1] * 16 + 8] and sb == [tables[1, 1] * 16 + 8]
    st.check()


def test_copy_on_write():
    """A fork shares a partly filled block; the first append to either side copies it first."""
    st = PagedStore(BlockManagerOracle(8, 4))
    st.append(0, 6)                      # blocks b0 (full), b1 (2 of 4)
    st.fork(0, 1)
    st.check()
    before = st.m.build_tables([0], 4)[0].copy()
    slots, cow = st.append(1, 1)         # child writes into the shared partly filled block
    assert cow is not None and cow[0] == before[0, 1]
    assert st.m.build_tables([0], 4)[0].tolist() == before.tolist()  # parent unchanged
    st.check()
    slots, cow = st.append(0, 2)         # the parent's block is now its own: no copy
    assert cow is None
    st.check()


def test_failures_change_nothing():
    m = BlockManagerOracle(3, 4)
    m.append(0, 8)
    snapshot = (list(m.ref), set(m.free), {k: dict(v) for k, v in m.seqs.items()})
    with pytest.raises(CacheError):
        m.append(1, 9)   # needs 3 blocks, 1 free
    with pytest.raises(CacheError):
        m.free_seq(7)
    with pytest.raises(CacheError):
        m.fork(0, 0)
    with pytest.raises(CacheError):
        m.add_prefix(5, 0, 9)
    with pytest.raises(CacheError):
        m.build_tables([0], 1)
    assert (list(m.ref), set(m.free), {k: dict(v) for k, v in m.seqs.items()}) == snapshot
    assert m.attach_prefix(99, 3) == 0 and 3 not in m.seqs


def random_ops(st, rng, steps):
    live = []
    keys = []
    next_sid = 0
    for _ in range(steps):
        op = rng.random()
        try:
            if op < 0.45 or not live:
                if live and rng.random() < 0.7:
                    sid = rng.choice(live)
                else:
                    sid = next_sid
                    next_sid += 1
                st.append(sid, rng.randint(0, 2 * st.bs + 3))
                if sid not in live:
                    live.append(sid)
            elif op < 0.6:
                sid = rng.choice(live)
                st.free(sid)
                live.remove(sid)
            elif op < 0.72:
                st.fork(rng.choice(live), next_sid)
                live.append(next_sid)
                next_sid += 1
            elif op < 0.82:
                sid = rng.choice(live)
                if st.m.seq_len(sid) > 0:
                    key = 1000 + len(keys)
                    st.add_prefix(key, sid, rng.randint(1, st.m.seq_len(sid)))
                    keys.append(key)
            elif op < 0.92 and keys:
                if st.attach(rng.choice(keys), next_sid):
                    live.append(next_sid)
                next_sid += 1
            elif keys:
                key = rng.choice(keys)
                st.drop_prefix(key)
                keys.remove(key)
        except CacheError:
            pass
        st.check()
    return live, keys


@pytest.mark.parametrize("seed,bs,nb", [(1, 4, 24), (2, 16, 40), (3, 1, 30), (4, 8, 12)])
def test_random_operations_read_back(seed, bs, nb):
    st = PagedStore(BlockManagerOracle(nb, bs))
    live, keys = random_ops(st, random.Random(seed), 400)
    for sid in list(live):
        st.free(sid)
    for key in list(keys):
        st.drop_prefix(key)
    st.check()
    assert st.m.num_free() == nb


def test_copy_blocks_pool():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    v = rng.standard_normal((6, 4, 2, 8)).astype(np.float32)
    k2, v2 = copy_blocks(k, v, [(1, 4), (2, 5)])
    assert np.array_equal(k2[4], k[1]) and np.array_equal(v2[5], v[2])
    assert np.array_equal(k2[[0, 1, 2, 3]], k[[0, 1, 2, 3]])


# --- planted mistakes: each must break a pin --------------------------------------------------------

class NoCopyOnWrite(BlockManagerOracle):
    def append(self, seq_id, n):
        seq = self.seqs.get(seq_id)
        if seq and seq["len"] % self.block_size and seq["blocks"]:
            saved = self.ref[seq["blocks"][-1]]
            self.ref[seq["blocks"][-1]] = 1  # pretend the shared block is private
            try:
                return super().append(seq_id, n)
            finally:
                self.ref[seq["blocks"][-1]] = saved
        return super().append(seq_id, n)


class OffByOneSlot(BlockManagerOracle):
    def append(self, seq_id, n):
        slots, cow = super().append(seq_id, n)
        return [s + 1 if s % self.block_size == 0 else s for s in slots], cow


class ReleaseIgnoresSharing(BlockManagerOracle):
    def _release(self, b):
        self.ref[b] = 0
        self.free.add(b)


class ForkWithoutReference(BlockManagerOracle):
    def fork(self, parent, child):
        super().fork(parent, child)
        for b in self.seqs[child]["blocks"]:
            self.ref[b] -= 1


@pytest.mark.parametrize("cls", [NoCopyOnWrite, OffByOneSlot, ReleaseIgnoresSharing, ForkWithoutReference])
def test_planted_mistakes_are_caught(cls):
    caught = False
    for seed in range(6):
        st = PagedStore(cls(20, 4))
        try:
            random_ops(st, random.Random(seed), 300)
        except AssertionError:
            caught = True
            break
    assert caught, f"{cls.__name__} passed every pin"
