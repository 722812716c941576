"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function raises (AssertionError or any error) when the oracle is wrong.  They are run
as ordinary tests by ``test_oracle.py`` and, with mistakes planted into the oracle, by
``test_oracle_mutants.py``, which requires every planted mistake to be caught by at least one pin.

Sources of truth used here:

* the pages' worked example, as indices only (``tests/golden/worked_example.json``: "Paged Attention
  基础 – 原理与实现进度", §2 block-table figure and the attention steps for token q = 23);
* brute force: scalar Python loops that read each key straight from its (block, offset) slot;
* a library routine: ``torch.nn.functional.scaled_dot_product_attention`` in float64 on the CPU over
  contiguous K/V, with an explicit causal mask and ``enable_gqa``;
* closed forms: uniform weights give the mean of the visible values; a single visible key returns its
  value; a strongly planted key returns its value;
* invariances: physical block ids, sharing a block versus a private copy, garbage outside the context,
  a chunk of a prefill versus the whole prefill.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.paged_kv as O
from workloads import FP32, BF16, build_workload, config_tiny

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


def _expected_rows(g, seq):
    """(physical block, offset) of every token of a golden sequence, from the fixture's ranges."""
    rows = []
    for rng_ in g["token_to_physical"][seq]:
        for t in range(rng_["first_token"], rng_["last_token"] + 1):
            rows.append((rng_["physical_block"], rng_["first_offset"] + t - rng_["first_token"]))
    return rows


def _position_coded_pool(num_blocks, bs, hkv, d):
    """Pool whose every element names its own (block, offset, head, dim)."""
    b, o, h, e = np.meshgrid(np.arange(num_blocks), np.arange(bs), np.arange(hkv), np.arange(d),
                             indexing="ij")
    return (b * 1_000_000 + o * 10_000 + h * 100 + e).astype(np.float64)


def _small_case(seed, hq, hkv, d, bs, q_lens, ctx_lens, dtype=FP32, shared=0):
    rng = np.random.default_rng(seed)
    return build_workload(rng, name="pin", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=d, block_size=bs, q_lens=q_lens, context_lens=ctx_lens,
                          shared_prefix_blocks=shared)


def _oracle_out(w, step_idx=0, k_pool=None, v_pool=None, scale=None):
    st = w.steps[step_idx]
    kp = w.k_pool if k_pool is None else k_pool
    vp = w.v_pool if v_pool is None else v_pool
    kp, vp = O.kv_write(kp, vp, st.k_new, st.v_new, st.slot_mapping)
    return O.paged_attention(st.q, kp, vp, w.block_tables, st.context_lens, st.query_start_loc,
                             w.scale if scale is None else scale, w.dtype), kp, vp


# ------------------------------------------------------------------------------------ worked example

def pin_worked_example_gather():
    """Sequence A's rows are block 7 rows 0..15 then block 3 rows 0..7; B's are block 7 then block 9;
    both share block 7's rows."""
    g = _golden()
    bs = g["block_size"]
    pool = _position_coded_pool(16, bs, 2, 4)
    gathered = {}
    for seq, info in g["sequences"].items():
        table = np.array(info["block_table"], dtype=np.int32)
        got = O.gather_sequence(pool, table, info["num_tokens"])
        exp = np.stack([pool[b, o] for (b, o) in _expected_rows(g, seq)])
        assert got.shape == exp.shape, (seq, got.shape, exp.shape)
        assert np.array_equal(got, exp), seq
        gathered[seq] = got
    assert np.array_equal(gathered["A"][:16], gathered["B"][:16])
    assert g["slots_used_in_last_block"]["A"] == 24 - 16


def pin_worked_example_query23():
    """Query token 23 of A depends on exactly A's 24 cached rows (block 7 rows 0..15, block 3 rows
    0..7) and on nothing else in the pool."""
    g = _golden()
    w = config_tiny()
    out0, kp, vp = _oracle_out(w)
    qrow = g["query_token"]  # A's rows come first in the packed batch
    base = out0[qrow]
    visible = set(_expected_rows(g, "A"))
    assert len(visible) == g["query_sees_tokens"][1] - g["query_sees_tokens"][0] + 1
    st = w.steps[0]
    for blk in range(w.num_blocks):
        for off in range(w.block_size):
            vp2 = vp.copy()
            vp2[blk, off] += 1.0
            kp2 = kp.copy()
            kp2[blk, off] += 1.0
            out = O.paged_attention(st.q, kp2, vp2, w.block_tables, st.context_lens,
                                    st.query_start_loc, w.scale, w.dtype)
            changed = not np.array_equal(out[qrow], base)
            assert changed == ((blk, off) in visible), (blk, off)


def pin_write_worked_example():
    """Both prefills, then both decodes, land exactly where the worked example puts the tokens:
    A on blocks 7 and 3, B's own tokens on block 9, the decode tokens at offset 8 of blocks 3 and 9.
    Both ways of treating B's shared prefix give the same pool; every other row is untouched."""
    g = _golden()
    pools = []
    for mode in ("skip", "rewrite"):
        w = config_tiny(shared_write=mode)
        st0, st1 = w.steps
        k1, v1 = O.kv_write(w.k_pool, w.v_pool, st0.k_new, st0.v_new, st0.slot_mapping)
        exp_k = w.k_pool.copy()
        exp_v = w.v_pool.copy()
        for t, (b, o) in enumerate(_expected_rows(g, "A")):
            exp_k[b, o] = st0.k_new[t]
            exp_v[b, o] = st0.v_new[t]
        for t, (b, o) in enumerate(_expected_rows(g, "B")):
            if t >= 16:  # B's own tokens; its first 16 are A's rows in the shared block
                exp_k[b, o] = st0.k_new[24 + t]
                exp_v[b, o] = st0.v_new[24 + t]
        assert np.array_equal(k1.view(np.uint32), exp_k.view(np.uint32)), mode
        assert np.array_equal(v1.view(np.uint32), exp_v.view(np.uint32)), mode
        k2, v2 = O.kv_write(k1, v1, st1.k_new, st1.v_new, st1.slot_mapping)
        exp_k[3, 8] = st1.k_new[0]
        exp_v[3, 8] = st1.v_new[0]
        exp_k[9, 8] = st1.k_new[1]
        exp_v[9, 8] = st1.v_new[1]
        assert np.array_equal(k2.view(np.uint32), exp_k.view(np.uint32)), mode
        assert np.array_equal(v2.view(np.uint32), exp_v.view(np.uint32)), mode
        pools.append((k2, v2))
    assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])


def pin_write_bf16_bits_and_skip():
    """bf16 rows are copied bit for bit (including NaN payloads and -0); slot -1 writes nothing."""
    nb, bs, h, d = 4, 8, 2, 3
    rng = np.random.default_rng(7)
    kp = rng.integers(0, 1 << 16, size=(nb, bs, h, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(nb, bs, h, d), dtype=np.uint16)
    kn = np.array([[[0x7FC1, 0x8000, 0x0001]] * h, [[0x1234, 0xFFFF, 0x7F80]] * h,
                   [[0x4242, 0x4243, 0x4244]] * h], dtype=np.uint16)
    vn = kn[::-1].copy()
    slots = np.array([2 * bs + 5, -1, 3 * bs + 0], dtype=np.int32)
    k2, v2 = O.kv_write(kp, vp, kn, vn, slots)
    ek, ev = kp.copy(), vp.copy()
    ek[2, 5], ev[2, 5] = kn[0], vn[0]
    ek[3, 0], ev[3, 0] = kn[2], vn[2]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert k2.dtype == np.uint16


# -------------------------------------------------------------------------------------- brute force

def _brute_force(w, k_pool, v_pool, st, scale):
    """Scalar loops: every key is read from its own slot; exp via math.exp."""
    hq, hkv, d, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    grp = hq // hkv
    q = O.to_float64(st.q, w.dtype) if w.dtype == BF16 else st.q.astype(np.float64)
    kp = k_pool.astype(np.float64) if w.dtype == FP32 else O.to_float64(k_pool, w.dtype)
    vp = v_pool.astype(np.float64) if w.dtype == FP32 else O.to_float64(v_pool, w.dtype)
    out = np.zeros(q.shape)
    for s in range(w.num_seqs):
        lo, hi = int(st.query_start_loc[s]), int(st.query_start_loc[s + 1])
        length = int(st.context_lens[s])
        n = hi - lo
        for i in range(n):
            pos = length - n + i
            for h in range(hq):
                g = h // grp
                scores = []
                for p in range(pos + 1):
                    blk = int(w.block_tables[s][p // bs])
                    off = p % bs
                    acc = 0.0
                    for e in range(d):
                        acc += float(q[lo + i, h, e]) * float(kp[blk, off, g, e])
                    scores.append(acc * scale)
                mx = max(scores)
                wts = [math.exp(x - mx) for x in scores]
                tot = sum(wts)
                for e in range(d):
                    acc = 0.0
                    for p in range(pos + 1):
                        blk = int(w.block_tables[s][p // bs])
                        acc += wts[p] * float(vp[blk, p % bs, g, e])
                    out[lo + i, h, e] = acc / tot
    return out


def pin_brute_force():
    """Random tiny shapes (MHA, GQA, MQA; block sizes 2..8; ragged tails) against scalar loops."""
    cases = [
        dict(seed=1, hq=2, hkv=2, d=4, bs=4, q_lens=[3, 1], ctx_lens=[9, 6]),
        dict(seed=2, hq=4, hkv=2, d=5, bs=8, q_lens=[5, 2, 1], ctx_lens=[5, 17, 1]),
        dict(seed=3, hq=4, hkv=1, d=3, bs=2, q_lens=[4, 0, 2], ctx_lens=[11, 3, 2]),
        dict(seed=4, hq=6, hkv=3, d=8, bs=4, q_lens=[7], ctx_lens=[23]),
    ]
    for dtype in (FP32, BF16):
        for c in cases:
            w = _small_case(c["seed"], c["hq"], c["hkv"], c["d"], c["bs"], c["q_lens"],
                            c["ctx_lens"], dtype=dtype)
            out, kp, vp = _oracle_out(w)
            ref = _brute_force(w, kp, vp, w.steps[0], w.scale)
            assert np.max(np.abs(out - ref)) <= 1e-12, (dtype, c)


# ------------------------------------------------------------------------------------ library routine

def _contiguous_to_pool(seqs_kv, bs, num_blocks, tables):
    """Lay each sequence's contiguous ``[L, H, D]`` rows into the physical blocks its table names."""
    h, d = seqs_kv[0].shape[1:]
    pool = np.full((num_blocks, bs, h, d), np.nan)
    for s, kv in enumerate(seqs_kv):
        for j in range(-(-kv.shape[0] // bs)):
            rows = kv[j * bs:(j + 1) * bs]
            pool[tables[s][j], :rows.shape[0]] = rows
    return pool


def pin_sdpa_library():
    """Paged oracle on a randomly permuted pool == torch SDPA (float64, CPU) on contiguous K/V with a
    bottom-right causal mask and grouped heads."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(11)
    for (hq, hkv, d, bs) in [(8, 2, 16, 4), (4, 4, 8, 8), (6, 1, 12, 16)]:
        q_lens = [1, 5, 9, 0, 3]
        ctx = [7, 5, 40, 3, 33]
        nblk = [-(-c // bs) for c in ctx]
        num_blocks = sum(nblk) + 5
        perm = rng.permutation(num_blocks)
        tables = np.full((len(ctx), max(nblk)), -1, dtype=np.int32)
        cur = 0
        for s, nb in enumerate(nblk):
            tables[s, :nb] = perm[cur:cur + nb]
            cur += nb
        ks = [rng.standard_normal((c, hkv, d)) for c in ctx]
        vs = [rng.standard_normal((c, hkv, d)) for c in ctx]
        kp = _contiguous_to_pool(ks, bs, num_blocks, tables)
        vp = _contiguous_to_pool(vs, bs, num_blocks, tables)
        qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        q = rng.standard_normal((int(qsl[-1]), hq, d))
        scale = 0.37
        # The oracle widens float32 storage; keep values representable by rounding through float32.
        q32, kp32, vp32 = q.astype(np.float32), kp.astype(np.float32), vp.astype(np.float32)
        out = O.paged_attention(q32, kp32, vp32, tables, np.array(ctx, np.int32), qsl, scale, FP32)
        for s in range(len(ctx)):
            n, length = q_lens[s], ctx[s]
            if n == 0:
                continue
            qt = torch.from_numpy(q32[qsl[s]:qsl[s + 1]].astype(np.float64)).permute(1, 0, 2)[None]
            kt = torch.from_numpy(ks[s].astype(np.float32).astype(np.float64)).permute(1, 0, 2)[None]
            vt = torch.from_numpy(vs[s].astype(np.float32).astype(np.float64)).permute(1, 0, 2)[None]
            mask = torch.ones(n, length, dtype=torch.bool).tril(diagonal=length - n)
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                                 enable_gqa=True)
            ref = ref[0].permute(1, 0, 2).numpy()
            assert np.max(np.abs(out[qsl[s]:qsl[s + 1]] - ref)) <= 1e-12, (hq, hkv, s)


# ------------------------------------------------------------------------------------- closed forms

def pin_uniform_weights_mean():
    """With scale 0 every visible key weighs the same; with position-coded values V[p] = p the output
    of query i is exactly the mean of 0 .. L-n+i, i.e. (L-n+i)/2."""
    w = _small_case(21, 4, 2, 6, 4, [5, 1, 3], [13, 9, 3])
    st = w.steps[0]
    kp, vp = O.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
    vp = vp.copy()
    for s in range(w.num_seqs):
        for p in range(int(st.context_lens[s])):
            vp[w.block_tables[s][p // w.block_size], p % w.block_size] = p
    out = O.paged_attention(st.q, kp, vp, w.block_tables, st.context_lens, st.query_start_loc, 0.0,
                            w.dtype)
    for s in range(w.num_seqs):
        lo, hi = int(st.query_start_loc[s]), int(st.query_start_loc[s + 1])
        length, n = int(st.context_lens[s]), hi - lo
        for i in range(n):
            assert np.max(np.abs(out[lo + i] - (length - n + i) / 2.0)) <= 1e-12, (s, i)


def pin_single_visible_key():
    """A one-token sequence (n = L = 1) and the first query of a full prefill see only key 0: the
    output is exactly that value row."""
    w = _small_case(22, 4, 2, 6, 4, [1, 6], [1, 6])
    out, kp, vp = _oracle_out(w)
    st = w.steps[0]
    grp = w.num_q_heads // w.num_kv_heads
    for s, row in ((0, 0), (1, 1)):
        v0 = vp[w.block_tables[s][0], 0].astype(np.float64)  # [H_kv, D]
        for h in range(w.num_q_heads):
            assert np.array_equal(out[row, h], v0[h // grp]), (s, h)


def pin_planted_key():
    """Planting ``K[p*] = 40 * q`` for one query makes its output the value at p* (to 1e-9): the
    exact slot of every visible position is read, and no other."""
    w = _small_case(23, 2, 1, 8, 4, [3], [14])
    st = w.steps[0]
    kp0, vp0 = O.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
    n, length = 3, 14
    for i in range(n):
        for target in range(length - n + i + 1):
            kp = kp0.copy()
            blk, off = w.block_tables[0][target // 4], target % 4
            kp[blk, off, 0] = 40.0 * st.q[i, 0]
            for p in range(length):  # keep every other key far weaker
                if p != target:
                    kp[w.block_tables[0][p // 4], p % 4, 0] *= 0.01
            out = O.paged_attention(st.q, kp, vp0, w.block_tables, st.context_lens,
                                    st.query_start_loc, 1.0, w.dtype)
            assert np.max(np.abs(out[i, 0] - vp0[blk, off, 0])) <= 1e-9, (i, target)


# ------------------------------------------------------------------------------------- invariances

def pin_paging_invariance():
    """The same logical K/V laid out in a randomly permuted pool or in consecutive blocks (a contiguous
    per-sequence cache) gives bit-identical output."""
    for dtype in (FP32, BF16):
        w = _small_case(31, 8, 2, 16, 8, [4, 1, 6, 2], [30, 17, 6, 45], dtype=dtype)
        out_perm, kp, vp = _oracle_out(w)
        nblk = [-(-int(c) // w.block_size) for c in w.steps[0].context_lens]
        tables = np.full_like(w.block_tables, -1)
        kc = np.zeros_like(kp)
        vc = np.zeros_like(vp)
        cur = 0
        for s, nb in enumerate(nblk):
            for j in range(nb):
                tables[s, j] = cur
                kc[cur] = kp[w.block_tables[s, j]]
                vc[cur] = vp[w.block_tables[s, j]]
                cur += 1
        st = w.steps[0]
        out_contig = O.paged_attention(st.q, kc, vc, tables, st.context_lens, st.query_start_loc,
                                       w.scale, dtype)
        assert np.array_equal(out_perm, out_contig), dtype


def pin_gqa_equals_repeated_heads():
    """Grouped heads equal plain multi-head attention with each kv head repeated for its group."""
    w = _small_case(32, 8, 2, 8, 4, [3, 2], [10, 7])
    out, kp, vp = _oracle_out(w)
    grp = 4
    kr = np.repeat(kp, grp, axis=2)
    vr = np.repeat(vp, grp, axis=2)
    st = w.steps[0]
    out_rep = O.paged_attention(st.q, kr, vr, w.block_tables, st.context_lens, st.query_start_loc,
                                w.scale, w.dtype)
    assert np.max(np.abs(out - out_rep)) <= 1e-13


def pin_chunk_consistency():
    """Worked example, sequence B: the last 8 tokens attended as a chunk over the 24 cached tokens equal
    rows 16..23 of the full 24-token prefill; the decode step at L = 25 equals row 24 of a 25-token
    prefill over the same cache."""
    w = config_tiny()
    st0, st1 = w.steps
    out0, kp, vp = _oracle_out(w)
    qb = st0.q[24:48]
    chunk = O.paged_attention(qb[16:], kp, vp, w.block_tables[1:], np.array([24], np.int32),
                              np.array([0, 8], np.int32), w.scale, w.dtype)
    assert np.max(np.abs(chunk - out0[24 + 16:48])) <= 1e-12
    kp2, vp2 = O.kv_write(kp, vp, st1.k_new, st1.v_new, st1.slot_mapping)
    dec = O.paged_attention(st1.q, kp2, vp2, w.block_tables, st1.context_lens, st1.query_start_loc,
                            w.scale, w.dtype)
    q_full = np.concatenate([st0.q[:24], st1.q[:1]])
    full = O.paged_attention(q_full, kp2, vp2, w.block_tables[:1], np.array([25], np.int32),
                             np.array([0, 25], np.int32), w.scale, w.dtype)
    assert np.max(np.abs(full[24] - dec[0])) <= 1e-12


def pin_shared_block_equals_private_copy():
    """Sequence B reading the shared block 7 equals B reading a private copy of it in a spare block."""
    w = config_tiny()
    out0, kp, vp = _oracle_out(w)
    st = w.steps[0]
    spare = 12
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[spare], vp2[spare] = kp[7], vp[7]
    tables = w.block_tables.copy()
    tables[1, 0] = spare
    out1 = O.paged_attention(st.q, kp2, vp2, tables, st.context_lens, st.query_start_loc, w.scale,
                             w.dtype)
    assert np.array_equal(out0, out1)


def pin_garbage_invariance():
    """NaN in blocks no table uses and in rows past each sequence's length changes nothing."""
    w = _small_case(33, 4, 2, 8, 8, [2, 1, 3], [11, 16, 21])
    out0, kp, vp = _oracle_out(w)
    st = w.steps[0]
    kp2, vp2 = kp.copy(), vp.copy()
    used = np.zeros((w.num_blocks, w.block_size), dtype=bool)
    for s in range(w.num_seqs):
        for p in range(int(st.context_lens[s])):
            used[w.block_tables[s][p // w.block_size], p % w.block_size] = True
    kp2[~used] = np.nan
    vp2[~used] = np.nan
    tables = w.block_tables.copy()
    tables[tables < 0] = 10 ** 6  # entries past a sequence's blocks are never read
    out1 = O.paged_attention(st.q, kp2, vp2, tables, st.context_lens, st.query_start_loc, w.scale,
                             w.dtype)
    assert np.all(np.isfinite(out1)) and np.array_equal(out0, out1)


# ------------------------------------------------------------------------------------ small helpers

def pin_softmax_rows_values():
    s = np.array([[0.0, math.log(2.0), -np.inf], [5.0, 5.0, 5.0]])
    p = O.softmax_rows(s)
    assert np.allclose(p, [[1 / 3, 2 / 3, 0.0], [1 / 3, 1 / 3, 1 / 3]], rtol=0, atol=1e-15)


def pin_bf16_widening():
    """bf16 bit patterns widen to their exact values."""
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x8000, 0x4049], dtype=np.uint16)
    vals = O.to_float64(bits, BF16)
    exp = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, np.inf, 0.0, 3.140625]
    assert np.array_equal(vals, np.array(exp))
    assert math.copysign(1.0, vals[5]) == -1.0


def pin_causal_mask_shape():
    """Bottom-right alignment: the last query sees every key; the first sees L - n + 1 keys."""
    m = O.causal_mask(3, 7)
    assert m.tolist() == [[True] * 5 + [False] * 2, [True] * 6 + [False], [True] * 7]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
