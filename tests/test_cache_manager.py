"""The library's C++ cache manager (pkv_cm_*) against the cache-manager oracle: on the same random
operation sequences every result must be identical (slots, copy-on-write pairs, refusals, free counts,
tables).  Host only: no GPU."""

import random

import numpy as np
import pytest

import paged_kv_cache_229_amd as pkv
from paged_kv_cache_229_amd import _native as N
from oracle.block_manager import BlockManagerOracle, CacheError


def same_state(cm, om, live, max_blocks):
    assert cm.num_free() == om.num_free()
    for sid in live:
        assert cm.seq_len(sid) == om.seq_len(sid)
    if live:
        t1, l1 = cm.build_tables(live, max_blocks)
        t2, l2 = om.build_tables(live, max_blocks)
        assert np.array_equal(t1, t2) and np.array_equal(l1, l2)


def both(fn_c, fn_o):
    """Run one operation on both; they must agree on success/failure and on the result."""
    try:
        r_o = fn_o()
        ok_o = True
    except CacheError:
        ok_o = False
    try:
        r_c = fn_c()
        ok_c = True
    except pkv.PagedKVError:
        ok_c = False
    assert ok_c == ok_o
    return (r_c, r_o) if ok_o else (None, None)


@pytest.mark.parametrize("seed,nb,bs", [(0, 30, 4), (1, 64, 16), (2, 12, 8), (3, 40, 1), (4, 200, 32)])
def test_random_operations_match_oracle(seed, nb, bs):
    rng = random.Random(seed)
    cm, om = pkv.CacheManager(nb, bs), BlockManagerOracle(nb, bs)
    live, keys, next_sid = [], [], 0
    max_blocks = nb
    for _ in range(500):
        op = rng.random()
        if op < 0.45 or not live:
            sid = rng.choice(live) if live and rng.random() < 0.7 else next_sid
            n = rng.randint(0, 3 * bs + 2)
            r_c, r_o = both(lambda: cm.append(sid, n), lambda: om.append(sid, n))
            if r_o is not None:
                assert r_c[0].tolist() == r_o[0] and r_c[1] == r_o[1]
                if sid not in live:
                    live.append(sid)
            if sid == next_sid:
                next_sid += 1
        elif op < 0.58:
            sid = rng.choice(live + [10**9])
            r_c, r_o = both(lambda: cm.free(sid), lambda: om.free_seq(sid))
            if sid in live:
                live.remove(sid)
        elif op < 0.7:
            child = rng.choice([next_sid, rng.choice(live)])
            parent = rng.choice(live)
            both(lambda: cm.fork(parent, child), lambda: om.fork(parent, child))
            if child == next_sid:
                if child in om.seqs:
                    live.append(child)
                next_sid += 1
        elif op < 0.8:
            sid = rng.choice(live)
            key = 5000 + len(keys) if rng.random() < 0.9 or not keys else rng.choice(keys)
            tokens = rng.randint(0, om.seq_len(sid) + 1)
            both(lambda: cm.add_prefix(key, sid, tokens), lambda: om.add_prefix(key, sid, tokens))
            if key in om.prefixes and key not in keys:
                keys.append(key)
        elif op < 0.9:
            key = rng.choice(keys + [777])
            sid = rng.choice([next_sid, rng.choice(live)])
            r_c, r_o = both(lambda: cm.attach_prefix(key, sid), lambda: om.attach_prefix(key, sid))
            if r_o is not None:
                assert r_c == r_o
            if sid == next_sid:
                if sid in om.seqs:
                    live.append(sid)
                next_sid += 1
        else:
            key = rng.choice(keys + [888])
            both(lambda: cm.drop_prefix(key), lambda: om.drop_prefix(key))
            if key in keys and key not in om.prefixes:
                keys.remove(key)
        same_state(cm, om, live, max_blocks)
    for sid in live:
        cm.free(sid)
        om.free_seq(sid)
    for key in keys:
        cm.drop_prefix(key)
        om.drop_prefix(key)
    assert cm.num_free() == om.num_free() == nb
    cm.close()


def test_errors_and_codes():
    cm = pkv.CacheManager(4, 16)
    cm.append(1, 50)                      # 4 blocks
    with pytest.raises(pkv.PagedKVError) as e:
        cm.append(2, 1)
    assert e.value.status == N.PKV_ERR_NO_BLOCKS
    assert cm.num_free() == 0 and cm.seq_len(2) == -1
    with pytest.raises(pkv.PagedKVError):
        cm.build_tables([1], 3)           # 4 blocks do not fit a 3-entry row
    with pytest.raises(pkv.PagedKVError):
        cm.free(9)
    assert cm.attach_prefix(123, 5) == 0 and cm.seq_len(5) == -1
    with pytest.raises(pkv.PagedKVError):
        pkv.CacheManager(0, 16)
    with pytest.raises(pkv.PagedKVError):
        pkv.CacheManager(1 << 28, 256)     # slots would not fit int32
    lib = N.lib()
    assert lib.pkv_cm_num_free(None) == -1 and lib.pkv_cm_seq_len(None, 1) == -1
    assert lib.pkv_cm_free(None, 1) == N.PKV_ERR_INVALID_ARG
    cm.close()
