"""paged_attention_forward_noalloc (no workspace argument; the library's fixed per-GPU scratch) through the
C-ABI against paged_attention_forward with a caller's workspace and against the oracle, on consecutive
calls that reuse the scratch: a larger batch, then a smaller one (whose plan must not depend on what the
first left behind), then a batch whose forced short partitions need more partial rows than the scratch
holds (the plan lengthens them), then float32.  Run last: it shares the GPU's scratch with nothing else."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_229_amd as pkv
from gpu_util import DeviceWorkload, check_close, log, out_f64
from workloads import BF16, FP32, build_workload, make_config

pytestmark = pytest.mark.gpu


def _compare(w, what, partition=0):
    pkv.set_tuning(partition, 0, 0)
    try:
        dw = DeviceWorkload(w)
        s = dw.steps[0]
        pkv.paged_kv_write(s["k_new"], s["v_new"], s["slot_mapping"], dw.k_pool, dw.v_pool)
        ref = pkv.paged_attention_forward(s["q"], dw.k_pool, dw.v_pool, dw.block_tables, s["context_lens"],
                                          s["query_start_loc"], scale=w.scale, max_q_len=s["max_q_len"])
        out = torch.full_like(s["q"], float("nan"))
        pkv.paged_attention_forward_noalloc(s["q"], dw.k_pool, dw.v_pool, dw.block_tables, s["context_lens"],
                                            s["query_start_loc"], out, scale=w.scale, max_q_len=s["max_q_len"])
        torch.cuda.synchronize()
    finally:
        pkv.set_tuning(0, 0, 0)
    got, want = out_f64(out), out_f64(ref)
    assert np.all(np.isfinite(got)), what
    if w.dtype == BF16:
        diff = np.abs(got - want)
        log(f"{what}: no-alloc vs workspace max {diff.max():.3e} mean {diff.mean():.3e}")
        assert diff.max() <= 2e-2 and diff.mean() <= 2e-3, what
    else:
        assert np.array_equal(got, want), what  # same plan-free kernel, same order
    _, _, orc = oracle.run_step(w.k_pool, w.v_pool, w.block_tables, w.steps[0], w.scale, w.dtype)
    check_close(got, orc, w.dtype, f"{what}: no-alloc vs oracle")


def test_noalloc_matches_the_workspace_entry_point():
    _compare(make_config("decode", "full"), "decode batch (64 sequences, contexts 512-4096)")
    _compare(make_config("spec", "small"), "smaller batch after it (4 speculative sequences)")
    # Two 16-token chunks (128 rows per kv head) over 50K-60K keys with 256-key partitions want ~480K partial
    # rows: the workspace plan lengthens the partitions to 1024 keys (120K rows), the scratch's smaller
    # budget (~64K rows at head_dim 128) to 2048.
    long = build_workload(np.random.default_rng(47), name="long", dtype=BF16, num_q_heads=64, num_kv_heads=8,
                          head_dim=128, block_size=16, q_lens=[16, 16], context_lens=[60000, 50000])
    _compare(long, "256-key partitions, more partial rows than the scratch holds", partition=256)
    _compare(make_config("decode", "small", dtype=FP32), "float32")
