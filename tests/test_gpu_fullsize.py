"""Full-size workloads, in the launch configuration bench.py times (default tuning): every new K/V row
is checked bit for bit at its slot, a sample of other pool rows is checked untouched, and the attention
output of sampled sequences (shortest, longest, first, last and two random ones) is checked against the
oracle, which computes those sequences one by one."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_229_amd as pkv
from gpu_util import DeviceWorkload, check_close, log, out_f64
from workloads import BF16, make_config, subset_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode", "mixed", "spec", "prefix"])
def test_full_size_sampled(name):
    pkv.set_tuning(0, 0, 0)
    w = make_config(name, "full")
    st = w.steps[0]
    log(f"full {name}: {w.description}, pool {w.num_blocks} blocks")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    torch.cuda.synchronize()

    # K/V write: the new rows, bit for bit, and untouched rows elsewhere.
    bs = w.block_size
    slots = st.slot_mapping[st.slot_mapping >= 0].astype(np.int64)
    blk = torch.from_numpy(slots // bs).to(dw.k_pool.device)
    off = torch.from_numpy(slots % bs).to(dw.k_pool.device)
    got_k = dw.k_pool[blk, off].view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = dw.v_pool[blk, off].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, st.k_new[st.slot_mapping >= 0])
    assert np.array_equal(got_v, st.v_new[st.slot_mapping >= 0])
    rng = np.random.default_rng(0)
    cand = rng.integers(0, w.num_blocks * bs, size=4000)
    cand = np.setdiff1d(cand, slots)
    cb = torch.from_numpy(cand // bs).to(dw.k_pool.device)
    co = torch.from_numpy(cand % bs).to(dw.k_pool.device)
    assert np.array_equal(dw.k_pool[cb, co].view(torch.int16).cpu().numpy().view(np.uint16),
                          w.k_pool[cand // bs, cand % bs])

    # Attention on sampled sequences.
    L = st.context_lens
    seqs = sorted(set([int(np.argmin(L)), int(np.argmax(L)), 0, w.num_seqs - 1]
                      + rng.choice(w.num_seqs, 2, replace=False).tolist()))
    k2, v2 = oracle.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
    ref = oracle.paged_attention(st.q, k2, v2, w.block_tables, st.context_lens, st.query_start_loc,
                                 w.scale, w.dtype, seqs=seqs)
    rows = np.concatenate([np.arange(st.query_start_loc[s], st.query_start_loc[s + 1]) for s in seqs])
    got = out_f64(out)
    check_close(got[rows], ref[rows], BF16, f"full {name} seqs {seqs}")


def test_full_size_prefix_pass_sampled():
    """The prefix-sharing batch at full size through paged_attention_forward_prefix (the configuration
    bench.py --prefix-pass times): all 256 sequences share 128 blocks; sampled sequences against the oracle,
    and the whole output against the ordinary entry point's."""
    pkv.set_tuning(0, 0, 0)
    w = make_config("prefix", "full")
    st = w.steps[0]
    log(f"full prefix, shared-prefix pass: {w.description}")
    dw = DeviceWorkload(w)
    out_plain = dw.run_step(0).clone()  # writes this step's K/V, then the ordinary computation
    s = dw.steps[0]
    out = pkv.paged_attention_forward_prefix(s["q"], dw.k_pool, dw.v_pool, dw.block_tables, s["context_lens"],
                                             s["query_start_loc"], 0, w.num_seqs,
                                             w.shared_prefix_blocks * w.block_size, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    L = st.context_lens
    seqs = sorted(set([int(np.argmin(L)), int(np.argmax(L)), 0, w.num_seqs - 1]
                      + rng.choice(w.num_seqs, 2, replace=False).tolist()))
    k2, v2 = oracle.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
    ref = oracle.paged_attention(st.q, k2, v2, w.block_tables, st.context_lens, st.query_start_loc,
                                 w.scale, w.dtype, seqs=seqs)
    rows = np.concatenate([np.arange(st.query_start_loc[q], st.query_start_loc[q + 1]) for q in seqs])
    check_close(out_f64(out)[rows], ref[rows], BF16, f"full prefix pass seqs {seqs}")
    # every row: the two entry points differ only by float32 summation order and bf16 rounding
    diff = (out.float() - out_plain.float()).abs()
    assert float(diff.max()) <= 2e-2 and float(diff.mean()) <= 2e-3, (float(diff.max()), float(diff.mean()))


def test_full_size_prefill_chunks_sampled():
    """The 8 prefill chunks of the mixed step alone, in the launch `bench.py --workload mixed --subset
    prefill` times (512-token chunks over up to 2048 prior tokens, 256-row tiles, automatic plan): the
    chunks with the shortest and the longest context against the oracle, every row."""
    pkv.set_tuning(0, 0, 0)
    full = make_config("mixed", "full")
    keep = np.nonzero(np.diff(full.steps[0].query_start_loc) > 1)[0]
    w = subset_workload(full, keep)
    st = w.steps[0]
    log(f"full prefill chunks: {w.num_seqs} sequences, contexts {st.context_lens.tolist()}")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    torch.cuda.synchronize()
    L = st.context_lens
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L))})
    k2, v2 = oracle.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
    ref = oracle.paged_attention(st.q, k2, v2, w.block_tables, st.context_lens, st.query_start_loc,
                                 w.scale, w.dtype, seqs=seqs)
    rows = np.concatenate([np.arange(st.query_start_loc[s], st.query_start_loc[s + 1]) for s in seqs])
    check_close(out_f64(out)[rows], ref[rows], BF16, f"full prefill chunks seqs {seqs}")
