#!/usr/bin/env python3
"""Benchmark: one step = paged_kv_write of the step's new K/V + paged_attention_forward, on one GPU.

    python bench.py [--workload spec|decode|mixed|prefix] [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  Inputs are seeded synthetic workloads (workloads/), resident in HBM before the
timed region.  The timed region runs exactly K steps between device synchronisations; each step uses the
next of several pool copies so the K/V stream comes from HBM, not from a cache warmed by the last step.
The attention kernel's own duration is read from HIP events the library records around it, and gives
the roofline fraction (algorithmic bytes per launch / average launch time vs 8 TB/s).  The CPU oracle is
timed on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16, 256 CU x 2.4 GHz x 4096 flop/clk
METRIC = "paged decode HBM GB/s (% peak) + prefill TFLOP/s (% MFMA peak), tokens/s"


def algorithmic_work(w) -> dict:
    """Bytes and flops the step must move/compute at minimum: tokens (not whole blocks) of K and V,
    Q read and O written once, block-table entries; causal (query, key) pairs only.  Shared prefix
    blocks count once for "unique" bytes and per sequence for "logical" bytes."""
    import numpy as np
    st = w.steps[0]
    e = w.elem_bytes
    L = st.context_lens.astype(np.int64)
    n = np.diff(st.query_start_loc).astype(np.int64)
    hq, hkv, d, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    row = hkv * d * e
    kv_logical = int(2 * row * L.sum())
    shared_tokens = w.shared_prefix_blocks * bs
    kv_unique = kv_logical - int(2 * row * shared_tokens * max(0, w.num_seqs - 1))
    total_q = int(n.sum())
    qo = 2 * total_q * hq * d * e
    tables = int(4 * (-(-L // bs)).sum())
    pairs = int(np.sum(n * (L - n) + n * (n + 1) // 2))
    flops = 4 * d * hq * pairs
    write_bytes = 2 * 2 * int(np.count_nonzero(st.slot_mapping >= 0)) * row
    # prefill subset (sequences with more than one new token) for the mixed workload
    pre = n > 1
    pairs_pre = int(np.sum(n[pre] * (L[pre] - n[pre]) + n[pre] * (n[pre] + 1) // 2))
    return dict(attn_bytes_unique=kv_unique + qo + tables, attn_bytes_logical=kv_logical + qo + tables,
                write_bytes=write_bytes, flops=flops, total_q=total_q, pairs=pairs,
                prefill_flops=4 * d * hq * pairs_pre)


def recorded_traffic(workload: str):
    """HBM bytes per launch of the attention kernel (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy
    calibration) as recorded in profiles/attn_traffic.json, or None when the kernel source has changed
    since those counters were taken (or none were taken for this workload)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec.get("sources", []):
        path = os.path.join(ROOT, src)
        if not os.path.exists(path):  # a source the counters covered is gone: the record is stale
            return None
        with open(path, "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec.get("kernel_source_sha256"):
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else int(w["read_bytes"] + w["write_bytes"])


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch already loaded (same soname)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.rt.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        self.rt.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def destroy(self, ev: int) -> None:
        self.rt.hipEventDestroy(ctypes.c_void_p(ev))


def _to_device(dev, a, is_data=True):
    import numpy as np
    import torch
    if is_data and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def time_steps(dev, w, steps: int, warmup: int, copies: int, layers: int = 1, prefix_pass: bool = False,
               graph: bool = False, reuse: bool = False, fused: bool = False) -> dict:
    """Warm up, then time exactly ``steps`` steps (paged_kv_write + paged_attention_forward of the workload's
    step, each on the next of ``copies`` pool copies) between two device synchronisations, with nothing else
    on the stream.  The same number of steps then runs again with events on the launch stream, for the
    attention kernel alone (HIP events the library records around it) and the whole attention call (plan +
    attention + split reduce: torch events around the call).  reuse: the pool copies stand for the layers
    of a model step, which share the metadata: the call on copy 0 plans (paged_attention_forward, or
    paged_attention_forward_prefix with prefix_pass), the calls on the other copies run on its plan
    (paged_attention_run, paged_attention_run_prefix).  fused: each step is one paged_attention_write_forward
    call (the write and the plan share a launch); the call events then also cover the write."""
    import numpy as np
    import torch

    import paged_kv_cache_229_amd as pkv

    st = w.steps[0]
    k0, v0 = _to_device(dev, w.k_pool), _to_device(dev, w.v_pool)
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(max(0, copies - 1))]
    if layers > 1:
        # Layer inside the block: each block holds every layer's rows; the attended layer's pool is a
        # strided view (block_stride = layers * block_size * H_kv * D elements).
        def inside(x):
            big = torch.zeros((x.shape[0], layers) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
            big[:, layers - 1] = x
            return big[:, layers - 1]
        pools = [(inside(k), inside(v)) for k, v in pools]
    del k0, v0
    bt = _to_device(dev, w.block_tables, False)
    q, kn, vn = _to_device(dev, st.q), _to_device(dev, st.k_new), _to_device(dev, st.v_new)
    sm = _to_device(dev, st.slot_mapping, False)
    cl, qsl = _to_device(dev, st.context_lens, False), _to_device(dev, st.query_start_loc, False)
    max_q = int(np.diff(st.query_start_loc).max())
    out = torch.empty_like(q)
    prefix_tokens = w.shared_prefix_blocks * w.block_size if prefix_pass else 0
    if prefix_tokens:
        need = pkv.prefix_workspace_size(w.num_seqs, q.shape[0], w.num_q_heads, w.num_kv_heads, w.head_dim,
                                         q.dtype)
    else:
        need = pkv.workspace_size(w.num_seqs, q.shape[0], w.num_q_heads, w.num_kv_heads, w.head_dim, q.dtype,
                                  max_q)
    ws = torch.empty(max(256, need), dtype=torch.uint8, device=dev)
    call_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]

    def step(i, timed=None):
        kp, vp = pools[i % len(pools)]
        if fused:
            if timed is not None:
                call_ev[timed][0].record()
            pkv.paged_attention_write_forward(kn, vn, sm, q, kp, vp, bt, cl, qsl, scale=w.scale, out=out,
                                              workspace=ws, max_q_len=max_q)
            if timed is not None:
                call_ev[timed][1].record()
            return
        pkv.paged_kv_write(kn, vn, sm, kp, vp)
        if timed is not None:
            call_ev[timed][0].record()
        if prefix_tokens and reuse and i % len(pools) != 0:
            pkv.paged_attention_run_prefix(q, kp, vp, bt, cl, qsl, 0, w.num_seqs, prefix_tokens,
                                           scale=w.scale, out=out, workspace=ws)
        elif prefix_tokens:
            pkv.paged_attention_forward_prefix(q, kp, vp, bt, cl, qsl, 0, w.num_seqs, prefix_tokens,
                                               scale=w.scale, out=out, workspace=ws)
        elif reuse and i % len(pools) != 0:
            pkv.paged_attention_run(q, kp, vp, bt, cl, qsl, scale=w.scale, out=out, workspace=ws,
                                    max_q_len=max_q)
        else:
            pkv.paged_attention_forward(q, kp, vp, bt, cl, qsl, scale=w.scale, out=out, workspace=ws,
                                        max_q_len=max_q)
        if timed is not None:
            call_ev[timed][1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    # graph: one HIP graph per pool copy (the same kernels as an eager step), captured once and replayed back
    # to back, as a serving loop replays its captured decode step.  Default: every step launched from the host.
    graphs = []
    if graph:
        try:
            for i in range(min(steps, len(pools))):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(warmup + i)
                graphs.append(g)
            for g in graphs:  # the first replay of each graph also uploads it
                g.replay()
            torch.cuda.synchronize()
        except Exception as exc:  # noqa: BLE001 - any capture failure falls back to eager launches
            pkv.set_profile_events(None, None)
            print(f"[bench] graph capture unavailable ({exc}); timing eager launches", file=sys.stderr, flush=True)
            graphs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for i in range(steps):
            graphs[i % len(graphs)].replay()
    else:
        for i in range(steps):
            step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Kernel and call durations: the same steps again, eagerly, with events on the launch stream (events
    # recorded by graph nodes cannot be timed, and events between the kernels would add to the wall clock).
    for i in range(steps):
        pkv.set_profile_events(*pairs[i])
        step(warmup + i, timed=i)
    pkv.set_profile_events(None, None)
    torch.cuda.synchronize()
    kernel_ms = np.array([ev.elapsed_ms(a, b) for a, b in pairs])
    call_ms = np.array([a.elapsed_time(b) for a, b in call_ev])
    launch = "hip_graph" if graphs else "eager"
    del graphs
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)

    def summary(x):
        return {"mean": round(float(np.mean(x)), 5), "p10": round(float(np.percentile(x, 10)), 5),
                "p90": round(float(np.percentile(x, 90)), 5)}

    return {"ms_per_step": elapsed * 1e3 / steps, "kernel_ms": float(np.mean(kernel_ms)),
            "call_ms": float(np.mean(call_ms)), "kernel": summary(kernel_ms), "call": summary(call_ms),
            "launch": launch,
            "pool_copies": len(pools)}


def kernel_name_for(w, tile_kind: int = 0, prefix_pass: bool = False) -> str:
    """The attention kernel that runs the workload's work items (one kernel; each item runs the 16-row or the
    32-row body its sequence's tile kind selects)."""
    return "attn_kernel"


def hbm_view(dev, name: str, steps: int, warmup: int, copies: int) -> dict:
    """Another HBM-bound workload of the metric at full size (the decode batch), with the same per-launch
    figures as the headline: kernel-only and whole-call fractions of the 8 TB/s peak."""
    from workloads import make_config

    w = make_config(name, "full")
    work = algorithmic_work(w)
    t = time_steps(dev, w, steps, warmup, copies)
    kgbs = work["attn_bytes_unique"] / (t["kernel_ms"] * 1e-3) / 1e9
    cgbs = work["attn_bytes_unique"] / (t["call_ms"] * 1e-3) / 1e9
    sgbs = (work["attn_bytes_unique"] + work["write_bytes"]) / (t["ms_per_step"] * 1e-3) / 1e9
    return {"workload": w.description, "kernel": kernel_name_for(w), "bound": "hbm",
            "bytes_per_launch": work["attn_bytes_unique"],
            "attention_kernel_ms": t["kernel"], "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
            "attention_call_ms": t["call"], "call_frac": round(cgbs / HBM_PEAK_GBS, 4),
            "ms_per_step": round(t["ms_per_step"], 4), "step_frac": round(sgbs / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(w.name), "tokens_per_s": round(work["total_q"] / (t["ms_per_step"] * 1e-3), 1)}


def plan_reuse_view(dev, name: str, steps: int, warmup: int, copies: int) -> dict:
    """The workload's step as one layer of a model step whose layers share the metadata: every ``copies``-th
    call plans (paged_attention_forward), the others run on that plan (paged_attention_run).  Per-layer wall
    time and whole-call time, beside the plain step's."""
    from workloads import make_config

    w = make_config(name, "full")
    work = algorithmic_work(w)
    t = time_steps(dev, w, steps, warmup, copies, reuse=True)
    sgbs = (work["attn_bytes_unique"] + work["write_bytes"]) / (t["ms_per_step"] * 1e-3) / 1e9
    cgbs = work["attn_bytes_unique"] / (t["call_ms"] * 1e-3) / 1e9
    return {"workload": w.name, "layers_per_plan": copies, "ms_per_layer": round(t["ms_per_step"], 4),
            "layer_frac": round(sgbs / HBM_PEAK_GBS, 4), "attention_call_ms": t["call"],
            "attention_call_frac": round(cgbs / HBM_PEAK_GBS, 4)}


def fused_step_view(dev, name: str, steps: int, warmup: int, copies: int) -> dict:
    """The workload's step through paged_attention_write_forward: the K/V write and the work plan share one
    launch, so a step is three launches instead of four.  Wall time per step, beside the plain step's."""
    from workloads import make_config

    w = make_config(name, "full")
    work = algorithmic_work(w)
    t = time_steps(dev, w, steps, warmup, copies, fused=True)
    sgbs = (work["attn_bytes_unique"] + work["write_bytes"]) / (t["ms_per_step"] * 1e-3) / 1e9
    return {"workload": w.name, "ms_per_step": round(t["ms_per_step"], 4),
            "step_frac": round(sgbs / HBM_PEAK_GBS, 4), "write_and_call_ms": t["call"]}


def prefill_view(dev, steps: int, warmup: int, copies: int) -> dict:
    """The other half of the metric: the chunked-prefill step's 8 prefill chunks alone (512 tokens each over a
    prior context U[0, 2048], the launch `--workload mixed --subset prefill` times), with the attention kernel
    timed by the library's HIP events and priced against the dense bf16 MFMA peak."""
    import numpy as np

    from workloads import make_config, subset_workload

    w = make_config("mixed", "full")
    keep = np.nonzero(np.diff(w.steps[0].query_start_loc) > 1)[0]
    w = subset_workload(w, keep)
    w.description += f" [prefill sequences only: {len(keep)}]"
    work = algorithmic_work(w)
    t = time_steps(dev, w, steps, warmup, copies)
    tflops = work["flops"] / (t["kernel_ms"] * 1e-3) / 1e12
    call_tflops = work["flops"] / (t["call_ms"] * 1e-3) / 1e12
    return {"workload": w.description, "kernel": kernel_name_for(w), "bound": "mfma",
            "attention_kernel_ms": t["kernel"], "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": work["flops"],
            "attention_call_ms": t["call"], "call_frac": round(call_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": recorded_traffic("mixed:prefill"),
            "tokens_per_s": round(work["total_q"] / (t["kernel_ms"] * 1e-3), 1)}


def cpu_baseline(w, work, budget_s: float) -> dict:
    """The oracle as it stands, on the host cores, over the workload's step (K/V write, then attention one
    sequence at a time), repeated until at least min(10 s, budget_s) of work and stopped mid-step once
    ``budget_s`` is spent.  Reported in the same GB/s unit."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    st = w.steps[0]
    qsl = st.query_start_loc
    L = st.context_lens.astype(np.int64)
    e = w.elem_bytes
    row = w.num_kv_heads * w.head_dim * e
    n = np.diff(qsl).astype(np.int64)
    secs = 0.0
    bytes_total = 0
    passes = 0
    partial = 0
    while True:
        t0 = time.perf_counter()
        k2, v2 = oracle.kv_write(w.k_pool, w.v_pool, st.k_new, st.v_new, st.slot_mapping)
        secs += time.perf_counter() - t0
        bytes_total += work["write_bytes"]
        partial = 0
        for s in range(w.num_seqs):
            t1 = time.perf_counter()
            oracle.paged_attention(st.q, k2, v2, w.block_tables, st.context_lens, qsl, w.scale, w.dtype,
                                   seqs=[s])
            secs += time.perf_counter() - t1
            bytes_total += int(2 * row * L[s] + 2 * n[s] * w.num_q_heads * w.head_dim * e)
            partial += 1
            if secs >= budget_s:
                break
        if partial == w.num_seqs:
            passes += 1
            partial = 0
        if secs >= min(10.0, budget_s):
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    what = f"{passes} whole step(s)" + (f" plus the first {partial} of {w.num_seqs} sequences" if partial else "")
    return {"value": round(bytes_total / secs / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 numpy oracle, K/V write then attention per sequence: {what} "
                      f"({secs:.1f} s, {os.cpu_count()} host cores visible, BLAS threads {threads})"}


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="spec", choices=["decode", "mixed", "spec", "prefix"],
                    help="headline workload (default: the long-context speculative decode batch)")
    ap.add_argument("--copies", type=int, default=4, help="pool copies rotated across steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--items", type=int, default=0)
    ap.add_argument("--tile-kind", type=int, default=0)
    ap.add_argument("--subset", choices=["all", "prefill", "decode"], default="all",
                    help="time only the sequences with q_len > 1 (prefill) or q_len == 1 (decode)")
    ap.add_argument("--plan-reuse", action="store_true",
                    help="the pool copies are the layers of one model step: plan on the first, run the others "
                         "on that plan (paged_attention_run, or paged_attention_run_prefix with --prefix-pass)")
    ap.add_argument("--fused", action="store_true",
                    help="each step is one paged_attention_write_forward call (write and plan in one launch)")
    ap.add_argument("--prefix-pass", action="store_true",
                    help="prefix workload: attend the shared blocks once for all sequences "
                         "(paged_attention_forward_prefix)")
    ap.add_argument("--layers", type=int, default=1,
                    help="pool layout [num_blocks, layers, block_size, H_kv, D] (layer inside the block), "
                         "attending the last layer through block_stride; 1 = per-layer pool")
    ap.add_argument("--graph", action="store_true",
                    help="replay captured HIP graphs of the step instead of launching each step from the host "
                         "(slower on ROCm 7: graph dispatch adds more than the host launches it saves)")
    ap.add_argument("--no-views", action="store_true",
                    help="skip the decode and prefill views a default run adds beside the headline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)
    if args.fused and (args.prefix_pass or args.plan_reuse or args.graph):
        print("bench.py: --fused times plain steps through paged_attention_write_forward; it does not combine "
              "with --prefix-pass, --plan-reuse or --graph", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_229_amd as pkv
    from workloads import make_config, subset_workload

    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": max(1, args.steps)}), flush=True)
        return
    t_gen = time.perf_counter()
    w = make_config(args.workload, "full")
    if args.subset != "all":
        qlens = np.diff(w.steps[0].query_start_loc)
        keep = np.nonzero(qlens > 1 if args.subset == "prefill" else qlens == 1)[0]
        w = subset_workload(w, keep)
        w.description += f" [{args.subset} sequences only: {len(keep)}]"
    print(f"[bench] generated {w.description} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    if args.prefix_pass and w.shared_prefix_blocks == 0:
        print("bench.py: --prefix-pass needs a workload with shared prefix blocks (prefix)", file=sys.stderr)
        sys.exit(2)
    work = algorithmic_work(w)
    traffic_key = w.name if args.subset == "all" else f"{w.name}:{args.subset}"
    if args.prefix_pass:
        traffic_key += ":prefix_pass"
    kernel_name = kernel_name_for(w, args.tile_kind, args.prefix_pass)
    pkv.set_tuning(args.partition, args.items, args.tile_kind)  # the workspace size depends on it
    t = time_steps(dev, w, args.steps, args.warmup, args.copies, layers=args.layers,
                   prefix_pass=args.prefix_pass, graph=args.graph, reuse=args.plan_reuse, fused=args.fused)
    print(f"[bench] headline timed: {t['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)

    ms_step = t["ms_per_step"]
    k_avg = t["kernel_ms"]
    step_bytes = work["attn_bytes_unique"] + work["write_bytes"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = work["attn_bytes_unique"] / (k_avg * 1e-3) / 1e9
    call_gbs = work["attn_bytes_unique"] / (t["call_ms"] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "subset": args.subset, "description": w.description,
                   "num_seqs": w.num_seqs,
                   "total_q": work["total_q"], "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "pool_copies": t["pool_copies"],
                   "pool_layout": "per_layer" if args.layers == 1 else f"layer_in_block x{args.layers}",
                   "shared_prefix_pass": bool(args.prefix_pass), "plan_reuse": bool(args.plan_reuse),
                   "fused_write": bool(args.fused),
                   "launch": t["launch"]},
        "tokens_per_s": round(work["total_q"] / (ms_step * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "attention_kernel_ms": t["kernel"],
        "attention_call_ms": t["call"],
        "attention_call_frac": round(call_gbs / HBM_PEAK_GBS, 4),
        "attention_tflops": round(work["flops"] / (k_avg * 1e-3) / 1e12, 2),
        "attention_pct_mfma_peak": round(100 * work["flops"] / (k_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
        "attention_logical_gbs": round(work["attn_bytes_logical"] / (k_avg * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(traffic_key),
                     "kernel": kernel_name,
                     "bytes_per_launch": work["attn_bytes_unique"]},
    }
    if args.subset == "prefill":
        # Long query chunks are a dense contraction: price the kernel against the bf16 MFMA peak.
        tflops = work["flops"] / (k_avg * 1e-3) / 1e12
        result["roofline"].update({"bound": "mfma", "achieved": round(tflops, 2),
                                   "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "flops_per_launch": work["flops"]})
        result["attention_call_frac"] = round(work["flops"] / (t["call_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    if work["prefill_flops"]:
        result["prefill_subset_flops"] = work["prefill_flops"]
    default_shape = (args.workload == "spec" and args.subset == "all" and args.layers == 1 and not args.graph
                     and not args.prefix_pass and not args.plan_reuse and not args.fused
                     and not (args.partition or args.items or args.tile_kind))
    if default_shape and not args.no_views:
        torch.cuda.empty_cache()
        result["decode_view"] = hbm_view(dev, "decode", args.steps, args.warmup, args.copies)
        print("[bench] decode view timed", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        result["prefill_view"] = prefill_view(dev, args.steps, args.warmup, args.copies)
        print("[bench] prefill view timed", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        result["plan_reuse_view"] = [plan_reuse_view(dev, name, args.steps, args.warmup, args.copies)
                                     for name in ("spec", "decode")]
        print("[bench] plan-reuse views timed", file=sys.stderr, flush=True)
        result["fused_step_view"] = [fused_step_view(dev, name, args.steps, args.warmup, args.copies)
                                     for name in ("spec", "decode")]
        print("[bench] fused-step views timed", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, work, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
