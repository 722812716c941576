"""paged_attention_run (and paged_attention_run_prefix): the layers of a model step after the first run on
the work plan the first layer's paged_attention_forward (_prefix) left in the workspace (same metadata, each
layer its own pools, queries and new K/V).  Every layer's output is bit-identical to paged_attention_forward's on that layer and within tolerance of the
oracle; a workspace without a plan for the call's shape gives an all-NaN output; rejected sequences still
get NaN rows on a run; the float32 path (no plan) runs as paged_attention_forward."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_229_amd as pkv
from gpu_util import check_close, log, out_f64, to_torch
from workloads import BF16, FP32, build_workload, make_config

pytestmark = pytest.mark.gpu

LAYERS = 3


def _layer(w, st, l):
    """Layer l's pools and step: the workload's, with pool blocks, query heads and new K/V rows rotated by l
    (the same metadata; other values)."""
    if l == 0:
        return w.k_pool, w.v_pool, st
    kp = np.roll(w.k_pool, 3 * l, axis=0)
    vp = np.roll(w.v_pool, 5 * l, axis=0)
    st_l = dataclasses.replace(st, q=np.roll(st.q, l, axis=1), k_new=np.roll(st.k_new, l, axis=0),
                               v_new=np.roll(st.v_new, 2 * l, axis=0))
    return kp, vp, st_l


def _device_step(w, st):
    return dict(q=to_torch(st.q, w.dtype), k_new=to_torch(st.k_new, w.dtype), v_new=to_torch(st.v_new, w.dtype),
                slot_mapping=to_torch(st.slot_mapping, None), context_lens=to_torch(st.context_lens, None),
                query_start_loc=to_torch(st.query_start_loc, None),
                max_q_len=int(np.max(np.diff(st.query_start_loc), initial=0)))


def _run_layers(w, ctx=None, prefix_tokens=0):
    """Forward on layer 0, run on layers 1..LAYERS-1, and a fresh forward on every layer (own workspace) for
    comparison; with prefix_tokens, the shared-prefix entry points over all sequences.  Returns [(run or
    layer-0 output, fresh forward output, layer pools and step)]."""
    st = w.steps[0]
    if ctx is not None:
        st = dataclasses.replace(st, context_lens=ctx)
    bt = to_torch(w.block_tables, None)
    s0 = _device_step(w, st)
    need = pkv.workspace_size(w.num_seqs, s0["q"].shape[0], w.num_q_heads, w.num_kv_heads, w.head_dim,
                              s0["q"].dtype, s0["max_q_len"])
    if prefix_tokens:
        need = pkv.prefix_workspace_size(w.num_seqs, s0["q"].shape[0], w.num_q_heads, w.num_kv_heads, w.head_dim,
                                         s0["q"].dtype)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=s0["q"].device)
    ws_fresh = torch.zeros_like(ws)
    res = []
    for l in range(LAYERS):
        kp_h, vp_h, st_l = _layer(w, st, l)
        s = _device_step(w, st_l)
        kp, vp = to_torch(kp_h, w.dtype), to_torch(vp_h, w.dtype)
        pkv.paged_kv_write(s["k_new"], s["v_new"], s["slot_mapping"], kp, vp)
        args = (s["q"], kp, vp, bt, s["context_lens"], s["query_start_loc"])
        if prefix_tokens:
            pre = (0, w.num_seqs, prefix_tokens)
            call = pkv.paged_attention_forward_prefix if l == 0 else pkv.paged_attention_run_prefix
            out = call(*args, *pre, scale=w.scale, workspace=ws)
            fresh = pkv.paged_attention_forward_prefix(*args, *pre, scale=w.scale, workspace=ws_fresh)
        else:
            call = pkv.paged_attention_forward if l == 0 else pkv.paged_attention_run
            out = call(*args, scale=w.scale, workspace=ws, max_q_len=s["max_q_len"])
            fresh = pkv.paged_attention_forward(*args, scale=w.scale, workspace=ws_fresh, max_q_len=s["max_q_len"])
        res.append((out, fresh, kp_h, vp_h, st_l))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name", ["decode", "spec", "mixed", "prefix"])
def test_layers_reuse_the_first_plan(name):
    w = make_config(name, "small")
    log(f"plan reuse over {LAYERS} layers: small {name}")
    for l, (out, fresh, kp_h, vp_h, st_l) in enumerate(_run_layers(w)):
        got = out_f64(out)
        assert np.array_equal(got, out_f64(fresh)), f"{name} layer {l}: run differs from a fresh forward"
        if l == LAYERS - 1:
            _, _, ref = oracle.run_step(kp_h, vp_h, w.block_tables, st_l, w.scale, w.dtype)
            check_close(got, ref, w.dtype, f"{name} layer {l} (run) vs oracle")


def test_layers_reuse_the_shared_prefix_plan():
    """paged_attention_run_prefix on the plan paged_attention_forward_prefix made for the first layer: every
    layer bit-identical to a fresh paged_attention_forward_prefix and, on the last, to the oracle."""
    w = make_config("prefix", "small")
    prefix_tokens = w.shared_prefix_blocks * w.block_size
    assert prefix_tokens > 0
    log(f"shared-prefix plan reuse over {LAYERS} layers: small prefix, {prefix_tokens} shared tokens")
    for l, (out, fresh, kp_h, vp_h, st_l) in enumerate(_run_layers(w, prefix_tokens=prefix_tokens)):
        got = out_f64(out)
        assert np.array_equal(got, out_f64(fresh)), f"prefix layer {l}: run differs from a fresh forward"
        if l == LAYERS - 1:
            _, _, ref = oracle.run_step(kp_h, vp_h, w.block_tables, st_l, w.scale, w.dtype)
            check_close(got, ref, w.dtype, f"prefix layer {l} (run_prefix) vs oracle")


def test_forced_partitions_and_tile_kinds():
    """Split contexts (partial rows merged by the reduce on every run) under both row-tile kinds."""
    w = make_config("spec", "small")
    for kind in (1, 2):
        pkv.set_tuning(256, 0, kind)
        try:
            log(f"plan reuse, small spec, partition 256, tile kind {kind}")
            for l, (out, fresh, *_rest) in enumerate(_run_layers(w)):
                assert np.array_equal(out_f64(out), out_f64(fresh)), f"kind {kind} layer {l}"
        finally:
            pkv.set_tuning(0, 0, 0)


def _small(seed, q_lens, ctx, dtype=BF16, hq=8, hkv=2, d=128):
    return build_workload(np.random.default_rng(seed), name="reuse", dtype=dtype, num_q_heads=hq,
                          num_kv_heads=hkv, head_dim=d, block_size=16, q_lens=q_lens, context_lens=ctx)


def test_no_plan_for_the_shape_gives_nan():
    """A run on a zeroed workspace, on a plan for another batch shape, and on a plan the shared-prefix entry
    point made, and a shared-prefix run on a zeroed workspace, a plain forward's plan and another prefix
    range's plan: every output element NaN, nothing else written."""
    w = _small(61, [1, 3, 2], [40, 70, 33])
    w2 = _small(62, [1, 1, 2, 1], [40, 70, 33, 90])
    s, s2 = _device_step(w, w.steps[0]), _device_step(w2, w2.steps[0])
    kp, vp = to_torch(w.k_pool, w.dtype), to_torch(w.v_pool, w.dtype)
    kp2, vp2 = to_torch(w2.k_pool, w2.dtype), to_torch(w2.v_pool, w2.dtype)
    bt, bt2 = to_torch(w.block_tables, None), to_torch(w2.block_tables, None)
    need = max(pkv.workspace_size(w.num_seqs, s["q"].shape[0], 8, 2, 128, s["q"].dtype, None),
               pkv.prefix_workspace_size(w.num_seqs, s["q"].shape[0], 8, 2, 128, s["q"].dtype),
               pkv.workspace_size(w2.num_seqs, s2["q"].shape[0], 8, 2, 128, s2["q"].dtype, None))
    args = (s["q"], kp, vp, bt, s["context_lens"], s["query_start_loc"])
    for what in ("zeroed workspace", "plan for another batch", "shared-prefix plan"):
        ws = torch.zeros(need, dtype=torch.uint8, device=s["q"].device)
        if what == "plan for another batch":
            pkv.paged_attention_forward(s2["q"], kp2, vp2, bt2, s2["context_lens"], s2["query_start_loc"],
                                        scale=w2.scale, workspace=ws)
        elif what == "shared-prefix plan":
            pkv.paged_attention_forward_prefix(*args, 0, w.num_seqs, 16, scale=w.scale, workspace=ws)
        log(f"run without a plan for its shape: {what}")
        out = torch.zeros_like(s["q"])
        pkv.paged_attention_run(*args, scale=w.scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isnan(out.float()).all().item(), what
    for what in ("zeroed workspace", "plan of a plain forward", "plan for another prefix range"):
        ws = torch.zeros(need, dtype=torch.uint8, device=s["q"].device)
        if what == "plan of a plain forward":
            pkv.paged_attention_forward(*args, scale=w.scale, workspace=ws)
        elif what == "plan for another prefix range":
            pkv.paged_attention_forward_prefix(*args, 0, w.num_seqs - 1, 16, scale=w.scale, workspace=ws)
        log(f"shared-prefix run without a plan for its range: {what}")
        out = torch.zeros_like(s["q"])
        pkv.paged_attention_run_prefix(*args, 0, w.num_seqs, 16, scale=w.scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isnan(out.float()).all().item(), what


def test_rejected_sequences_on_a_run():
    """The reduce kernel, which every run launches, fills the rejected sequences' rows with NaN."""
    w = _small(63, [3, 2, 1, 4, 1], [40, 30, 60, 20, 9])
    ctx = w.steps[0].context_lens.copy()
    ctx[1] = 1                                              # q_len 2 > context 1
    ctx[3] = -5                                             # negative context
    ctx[4] = w.block_tables.shape[1] * w.block_size + 1     # past the table
    log("plan reuse with rejected sequences")
    res = _run_layers(w, ctx=ctx)
    qsl = w.steps[0].query_start_loc
    for l, (out, fresh, kp_h, vp_h, st_l) in enumerate(res):
        got = out_f64(out)
        for s in (1, 3, 4):
            assert np.all(np.isnan(got[qsl[s]:qsl[s + 1]])), (l, s)
        good = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in (0, 2)])
        assert np.array_equal(got[good], out_f64(fresh)[good]), l
    _, _, ref = oracle.run_step(kp_h, vp_h, w.block_tables, st_l, w.scale, w.dtype, seqs=[0, 2])
    check_close(got[good], ref[good], BF16, "valid rows beside rejected ones on a run")


def test_float32_runs_as_forward():
    w = _small(64, [1, 2, 1], [100, 80, 120], dtype=FP32, hq=4, d=64)
    log("float32 plan reuse (no plan)")
    for l, (out, fresh, kp_h, vp_h, st_l) in enumerate(_run_layers(w)):
        assert np.array_equal(out_f64(out), out_f64(fresh)), l
    _, _, ref = oracle.run_step(kp_h, vp_h, w.block_tables, st_l, w.scale, w.dtype)
    check_close(out_f64(out), ref, FP32, "float32 run vs oracle")
