"""GPU parity: the HIP path (through the C-ABI binding) against the CPU oracle on the same seeded inputs.

KV writes are compared bit for bit; attention within max-abs 2e-2 and mean-abs 2e-3 (bf16 inputs, fp32
accumulation) or max-abs 1e-5 (fp32) of the float64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_229_amd as pkv
from gpu_util import DeviceWorkload, check_close, log, out_f64, pool_bits, to_torch
from workloads import BF16, FP32, build_workload, config_tiny, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_tuning():
    pkv.set_tuning(0, 0, 0)
    yield
    pkv.set_tuning(0, 0, 0)


def _oracle_steps(w, seqs=None):
    kp, vp = w.k_pool, w.v_pool
    outs = []
    for st in w.steps:
        kp, vp, out = oracle.run_step(kp, vp, w.block_tables, st, w.scale, w.dtype, seqs=seqs)
        outs.append(out)
    return kp, vp, outs


@pytest.mark.parametrize("shared_write", ["skip", "rewrite"])
def test_worked_example_fp32(shared_write):
    """Worked example (A on [7,3], B on [7,9], bs 16, fp32): prefill then decode; pools bit exact,
    attention within 1e-5."""
    w = config_tiny(shared_write=shared_write)
    log(f"worked example fp32, shared_write={shared_write}")
    dw = DeviceWorkload(w)
    kp_ref, vp_ref, outs_ref = _oracle_steps(w)
    kp, vp = w.k_pool, w.v_pool
    for i, st in enumerate(w.steps):
        out = dw.run_step(i)
        kp, vp, _ = oracle.run_step(kp, vp, w.block_tables, st, w.scale, w.dtype)
        torch.cuda.synchronize()
        assert np.array_equal(pool_bits(dw.k_pool), kp.view(np.uint32))
        assert np.array_equal(pool_bits(dw.v_pool), vp.view(np.uint32))
        check_close(out_f64(out), outs_ref[i], FP32, f"tiny step {i}")


@pytest.mark.parametrize("name", ["decode", "mixed", "spec", "prefix"])
def test_small_configs_bf16(name):
    w = make_config(name, "small")
    log(f"small {name}: seqs={w.num_seqs} ctx={w.steps[0].context_lens.tolist()}")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    kp, vp, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(dw.k_pool), kp)
    assert np.array_equal(pool_bits(dw.v_pool), vp)
    check_close(out_f64(out), outs[0], BF16, f"small {name}")


@pytest.mark.parametrize("name", ["decode", "spec"])
def test_small_configs_fp32(name):
    w = make_config(name, "small", dtype=FP32)
    log(f"small {name} fp32")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], FP32, f"small {name} fp32")


@pytest.mark.parametrize("partition", [128, 256, 512, 1 << 20])
@pytest.mark.parametrize("name", ["decode", "spec", "mixed"])
def test_forced_partitions(name, partition):
    """Split-context partitions plus the reduce kernel give the oracle's result at any partition size."""
    w = make_config(name, "small")
    log(f"small {name} partition={partition}")
    pkv.set_tuning(partition, 0, 0)
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], BF16, f"{name} P={partition}")


@pytest.mark.parametrize("items", [1, 7, 64, 4096])
@pytest.mark.parametrize("name", ["decode", "mixed", "spec", "prefix"])
def test_item_counts(name, items):
    """Few or many work items (one item per workgroup up to several rounds of the snake assignment, long
    and short partitions) give the oracle's result."""
    w = make_config(name, "small")
    log(f"small {name} target_items={items}")
    pkv.set_tuning(0, items, 0)
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], BF16, f"{name} items={items}")


@pytest.mark.parametrize("kind", [1, 2])
@pytest.mark.parametrize("partition", [0, 256])
@pytest.mark.parametrize("name", ["decode", "mixed", "spec", "prefix"])
def test_tile_kinds(name, partition, kind):
    """Both row-tile shapes (16 or 32 rows per wave), with automatic or short partitions, give the
    oracle's result."""
    w = make_config(name, "small")
    log(f"small {name} tile_kind={kind} partition={partition}")
    pkv.set_tuning(partition, 0, kind)
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], BF16, f"{name} kind={kind} P={partition}")


@pytest.mark.parametrize("kind", [1, 2])
@pytest.mark.parametrize("head_dim,block_size", [(128, 16), (64, 32)])
def test_every_ring_phase(head_dim, block_size, kind):
    """Whole items (one 1024-key partition each) of 1 to 9, 13 and 14 stages of 64 keys: the last stage falls
    on every slot of the four-slot ring, and the long items wrap it several times; exact and ragged ends,
    one or three query tokens per sequence; against the oracle."""
    pkv.set_tuning(1024, 0, kind)
    stages = list(range(1, 10)) + [13, 14]
    ctx = [64 * s for s in stages] + [64 * s - 37 for s in stages]
    q_lens = [1 + 2 * (i % 2) for i in range(len(ctx))]
    w = build_workload(np.random.default_rng(4100 + head_dim + kind), name="ring", dtype=BF16, num_q_heads=8,
                       num_kv_heads=2, head_dim=head_dim, block_size=block_size, q_lens=q_lens, context_lens=ctx)
    log(f"ring phases D={head_dim} bs={block_size} tile_kind={kind}")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], BF16, f"ring phases D{head_dim} kind={kind}")


@pytest.mark.parametrize("dtype,kind", [(BF16, 1), (BF16, 2), (FP32, 0)])  # the float32 path has no row tiles
@pytest.mark.parametrize("head_dim,block_size,hq,hkv", [(64, 8, 8, 2), (64, 32, 4, 4), (128, 64, 16, 1),
                                                         (128, 256, 6, 3)])
def test_geometries(dtype, head_dim, block_size, hq, hkv, kind):
    """head_dim 64/128, block sizes 8..256, MHA/GQA/MQA, ragged lengths including 1 and exact blocks,
    under both bf16 row-tile shapes and on the float32 path."""
    pkv.set_tuning(0, 0, kind)
    rng = np.random.default_rng(head_dim * 1000 + block_size + hq)
    q_lens = [1, 3, 1, 17, 0, 5, 1]
    ctx = [1, 3, block_size, 40 + 3 * block_size, 9, 2 * block_size + 1, 700]
    w = build_workload(rng, name="geo", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim,
                       block_size=block_size, q_lens=q_lens, context_lens=ctx)
    log(f"geometry D={head_dim} bs={block_size} {hq}/{hkv} {dtype}")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], dtype, f"geo D{head_dim} bs{block_size} {hq}/{hkv} {dtype}")


# (dtype, tile kind): both bf16 row-tile shapes and the float32 path (which has no row tiles).
_PATHS = [(BF16, 1), (BF16, 2), (FP32, 0)]


@pytest.mark.parametrize("name", ["spec", "mixed", "decode"])
@pytest.mark.parametrize("dtype,kind", _PATHS)
def test_paging_invariance_and_determinism(name, dtype, kind):
    """Permuted physical blocks vs a contiguous per-sequence layout: bit-identical GPU output; two runs
    of the same call are bit-identical too; and the result matches the oracle.  Under every kernel."""
    pkv.set_tuning(0, 0, kind)
    w = make_config(name, "small", dtype=dtype)
    log(f"paging invariance ({name} small, {dtype}, tile kind {kind})")
    dw = DeviceWorkload(w)
    out1 = dw.run_step(0).clone()
    st = dw.steps[0]
    out2 = pkv.paged_attention_forward(st["q"], dw.k_pool, dw.v_pool, dw.block_tables, st["context_lens"],
                                       st["query_start_loc"], scale=w.scale,
                                       max_q_len=st["max_q_len"])
    # contiguous layout: sequence s occupies consecutive blocks
    L = w.steps[0].context_lens
    nblk = -(-L.astype(np.int64) // w.block_size)
    perm_src = []
    tables = np.full_like(w.block_tables, -1)
    cur = 0
    for s in range(w.num_seqs):
        for j in range(nblk[s]):
            tables[s, j] = cur
            perm_src.append(w.block_tables[s, j])
            cur += 1
    idx = torch.tensor(perm_src, dtype=torch.long, device=dw.k_pool.device)
    kc = dw.k_pool[idx].contiguous()
    vc = dw.v_pool[idx].contiguous()
    out3 = pkv.paged_attention_forward(st["q"], kc, vc, to_torch(tables, None), st["context_lens"],
                                       st["query_start_loc"], scale=w.scale,
                                       max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(out1, out3)
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out1), outs[0], dtype, f"paging {name} {dtype} kind={kind}")


@pytest.mark.parametrize("name", ["decode", "spec", "mixed"])
@pytest.mark.parametrize("dtype,kind", _PATHS)
def test_garbage_invariance(name, dtype, kind):
    """NaN in every pool row no sequence uses (whole unowned blocks and the rows past each context in its
    last block), and -1 past each table's blocks: same output, finite.  Under every kernel."""
    pkv.set_tuning(0, 0, kind)
    w = make_config(name, "small", dtype=dtype)
    log(f"garbage invariance ({name} small, {dtype}, tile kind {kind})")
    dw = DeviceWorkload(w)
    out1 = dw.run_step(0).clone()
    L = w.steps[0].context_lens
    used = np.zeros((w.num_blocks, w.block_size), dtype=bool)
    for s in range(w.num_seqs):
        for p in range(int(L[s])):
            used[w.block_tables[s][p // w.block_size], p % w.block_size] = True
    assert np.all(w.block_tables[w.block_tables < 0] == -1)
    mask = torch.from_numpy(~used).to(dw.k_pool.device)
    kp = dw.k_pool.clone()
    vp = dw.v_pool.clone()
    kp[mask] = float("nan")
    vp[mask] = float("nan")
    st = dw.steps[0]
    out2 = pkv.paged_attention_forward(st["q"], kp, vp, dw.block_tables, st["context_lens"],
                                       st["query_start_loc"], scale=w.scale,
                                       max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    assert torch.isfinite(out2.float()).all()
    assert torch.equal(out1, out2)


def test_shared_prefix_equals_private_copy():
    """Prefix workload: sequence 0 reading the shared blocks equals it reading private copies."""
    w = make_config("prefix", "small")
    log("shared prefix vs private copy")
    dw = DeviceWorkload(w)
    out1 = dw.run_step(0).clone()
    shared = w.shared_prefix_blocks
    used = set(w.block_tables[w.block_tables >= 0].tolist())
    spare = [b for b in range(w.num_blocks) if b not in used][:shared]
    assert len(spare) == shared
    kp, vp = dw.k_pool.clone(), dw.v_pool.clone()
    src = torch.tensor(w.block_tables[0, :shared].tolist(), device=kp.device)
    dst = torch.tensor(spare, device=kp.device)
    kp[dst] = kp[src]
    vp[dst] = vp[src]
    tables = w.block_tables.copy()
    tables[0, :shared] = spare
    st = dw.steps[0]
    out2 = pkv.paged_attention_forward(st["q"], kp, vp, to_torch(tables, None), st["context_lens"],
                                       st["query_start_loc"], scale=w.scale,
                                       max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("workload,layers,layer", [("decode", 3, 1), ("decode", 2, 0), ("mixed", 4, 3),
                                                   ("spec", 2, 1), ("tiny", 3, 2)])
def test_layer_inside_block_pool(workload, layers, layer):
    """The pool layout [num_blocks, layers, block_size, H_kv, D] (layer inside the block, "Paged
    Attention 基础 – 原理与实现进度" §4) addressed through block_stride: its attention output matches the
    oracle (which walks the per-layer pool the layer slice holds), its pool slice holds exactly the oracle's
    pool after each write, the result is bit for bit the per-layer pool's, and the other layers stay
    untouched."""
    w = make_config(workload, "small")
    log(f"layer-inside-block pool {workload} layers={layers} layer={layer}")
    dw = DeviceWorkload(w)
    big_k = torch.zeros((w.num_blocks, layers) + tuple(dw.k_pool.shape[1:]), dtype=dw.k_pool.dtype,
                        device=dw.k_pool.device)
    big_v = torch.zeros_like(big_k)
    big_k[:, layer] = dw.k_pool
    big_v[:, layer] = dw.v_pool
    okp, ovp = w.k_pool, w.v_pool
    for i, st in enumerate(dw.steps):
        out_ref = dw.run_step(i).clone()
        pkv.paged_kv_write(st["k_new"], st["v_new"], st["slot_mapping"], big_k[:, layer], big_v[:, layer])
        out = pkv.paged_attention_forward(st["q"], big_k[:, layer], big_v[:, layer], dw.block_tables,
                                          st["context_lens"], st["query_start_loc"], scale=w.scale,
                                          max_q_len=st["max_q_len"])
        torch.cuda.synchronize()
        okp, ovp, ref = oracle.run_step(okp, ovp, w.block_tables, w.steps[i], w.scale, w.dtype)
        check_close(out_f64(out), ref, w.dtype, f"layer-inside-block {workload} step {i}")
        bits = (lambda a: a.view(np.uint32)) if w.dtype == FP32 else (lambda a: a)
        assert np.array_equal(pool_bits(big_k[:, layer].contiguous()), bits(okp))
        assert np.array_equal(pool_bits(big_v[:, layer].contiguous()), bits(ovp))
        assert torch.equal(out, out_ref)
        assert torch.equal(big_k[:, layer], dw.k_pool) and torch.equal(big_v[:, layer], dw.v_pool)
    for other in range(layers):
        if other != layer:
            assert int((big_k[:, other] != 0).sum()) == 0 and int((big_v[:, other] != 0).sum()) == 0


def test_long_context_chunk_splits_automatically():
    """A 384-token chunk over a long prior context (kv 2 heads, G 4: 1536 rows, six 256-row tiles, up to
    12000 keys) plus two decodes: with default tuning the tall tiles take the wide partition (at least 4096
    keys) and split, so split_reduce merges tall-tile partials; checked against the oracle, and the plan's
    partition words are checked to show the split happened."""
    w = build_workload(np.random.default_rng(31), name="longchunk", dtype=BF16, num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, q_lens=[384, 1, 1],
                       context_lens=[12000, 700, 5000])
    log("long-context chunk, automatic split of tall tiles")
    dw = DeviceWorkload(w)
    st = dw.steps[0]
    ws = torch.zeros(max(256, pkv.workspace_size(w.num_seqs, st["q"].shape[0], w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim, st["q"].dtype, st["max_q_len"])),
                     dtype=torch.uint8, device=st["q"].device)
    pkv.paged_kv_write(st["k_new"], st["v_new"], st["slot_mapping"], dw.k_pool, dw.v_pool)
    out = pkv.paged_attention_forward(st["q"], dw.k_pool, dw.v_pool, dw.block_tables, st["context_lens"],
                                      st["query_start_loc"], scale=w.scale, workspace=ws,
                                      max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    hdr = ws[:64].cpu().numpy().view(np.int32)
    wide_partition = int(hdr[5])
    assert 4096 <= wide_partition < 12000, wide_partition  # the tall tiles were split
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out), outs[0], BF16, "long-context chunk")


def test_single_long_decode_keeps_the_grid_busy():
    """One sequence decoding over 32768 keys (GQA 32/8): with default tuning the context is still split into
    enough partitions for two items per workgroup of the persistent grid (the planner's soft minimum
    partition length gives way), and the merged result matches the oracle."""
    w = build_workload(np.random.default_rng(37), name="onelong", dtype=BF16, num_q_heads=32,
                       num_kv_heads=8, head_dim=128, block_size=16, q_lens=[1], context_lens=[32768])
    log("single long decode, automatic partitions")
    dw = DeviceWorkload(w)
    st = dw.steps[0]
    ws = torch.zeros(max(256, pkv.workspace_size(w.num_seqs, st["q"].shape[0], w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim, st["q"].dtype, st["max_q_len"])),
                     dtype=torch.uint8, device=st["q"].device)
    pkv.paged_kv_write(st["k_new"], st["v_new"], st["slot_mapping"], dw.k_pool, dw.v_pool)
    out = pkv.paged_attention_forward(st["q"], dw.k_pool, dw.v_pool, dw.block_tables, st["context_lens"],
                                      st["query_start_loc"], scale=w.scale, workspace=ws,
                                      max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    hdr = ws[:64].cpu().numpy().view(np.int32)
    items = int(hdr[0]) * w.num_kv_heads
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert items >= 2 * cus, (items, cus)
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out), outs[0], BF16, "single long decode")


@pytest.mark.parametrize("n_seqs,max_q", [(64, 1), (65, 1), (100, 3), (128, 2), (40, 40)])
def test_planner_width(n_seqs, max_q):
    """The planner runs on one wave for at most 64 sequences and row tiles, on four beyond: batches on both
    sides of that bound (65-128 short sequences, and 40 sequences whose queries take about 100 tiles) against
    the oracle."""
    rng = np.random.default_rng(1000 + n_seqs + max_q)
    q_lens = rng.integers(1, max_q + 1, n_seqs)
    ctx = q_lens + rng.integers(0, 400, n_seqs)
    w = build_workload(rng, name="width", dtype=BF16, num_q_heads=16, num_kv_heads=2, head_dim=64,
                       block_size=16, q_lens=q_lens, context_lens=ctx)
    log(f"planner width: {n_seqs} sequences, q_len <= {max_q}")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    torch.cuda.synchronize()
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out), outs[0], BF16, f"{n_seqs} sequences, q_len <= {max_q}")


@pytest.mark.parametrize("block_size,head_dim", [(16, 128), (32, 128), (16, 64)])
def test_late_pieces(block_size, head_dim):
    """Long partitions (a small item target gives P of about 4900 keys) over contexts that end off any stage
    boundary: each split tile's last keys become late pieces (more units than whole partitions of P give),
    which must start on stage boundaries like every other partition; checked against the oracle with
    multi-token queries."""
    ctx = [9001, 12345, 17003, 10477, 15555, 13131]
    w = build_workload(np.random.default_rng(47 + block_size + head_dim), name="late", dtype=BF16, num_q_heads=8,
                       num_kv_heads=2, head_dim=head_dim, block_size=block_size, q_lens=[1, 4, 8, 3, 1, 6],
                       context_lens=ctx)
    log(f"late pieces, block size {block_size}, head dim {head_dim}")
    pkv.set_tuning(0, 32, 0)
    dw = DeviceWorkload(w)
    st = dw.steps[0]
    ws = torch.zeros(max(256, pkv.workspace_size(w.num_seqs, st["q"].shape[0], w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim, st["q"].dtype, st["max_q_len"])),
                     dtype=torch.uint8, device=st["q"].device)
    pkv.paged_kv_write(st["k_new"], st["v_new"], st["slot_mapping"], dw.k_pool, dw.v_pool)
    out = pkv.paged_attention_forward(st["q"], dw.k_pool, dw.v_pool, dw.block_tables, st["context_lens"],
                                      st["query_start_loc"], scale=w.scale, workspace=ws,
                                      max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    hdr = ws[:64].cpu().numpy().view(np.int32)
    units, partition = int(hdr[0]), int(hdr[2])
    whole = sum(-(-int(c) // partition) for c in st["context_lens"].cpu().numpy())
    assert partition >= 4096 and units > whole, (partition, units, whole)
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out), outs[0], BF16, f"late pieces, block size {block_size}, head dim {head_dim}")


def test_empty_and_degenerate():
    """num_seqs == 0 and num_tokens == 0 are no-ops; q_len 0 sequences are skipped."""
    w = build_workload(np.random.default_rng(5), name="deg", dtype=BF16, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, q_lens=[0, 1, 0, 2], context_lens=[5, 1, 33, 2])
    log("degenerate shapes")
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    _, _, outs = _oracle_steps(w)
    torch.cuda.synchronize()
    check_close(out_f64(out), outs[0], BF16, "degenerate")
    d = dw.k_pool.device
    e = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=d)
    pkv.paged_kv_write(e, e, torch.empty(0, dtype=torch.int32, device=d), dw.k_pool, dw.v_pool)
    q0 = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=d)
    pkv.paged_attention_forward(q0, dw.k_pool, dw.v_pool, dw.block_tables[:0],
                                torch.empty(0, dtype=torch.int32, device=d),
                                torch.zeros(1, dtype=torch.int32, device=d))
    torch.cuda.synchronize()


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("kind", [1, 2])
def test_many_sequences(kind, partition):
    """More sequences than the planner keeps in LDS (2048): 3000 short decode and speculative sequences,
    so the planner reads the later ones' metadata from global memory, with automatic and forced partitions
    under both tile kinds."""
    rng = np.random.default_rng(41)
    N = 3000
    q_lens = rng.choice([1, 1, 1, 2, 4, 7], N)
    ctx = q_lens + rng.integers(0, 200, N)
    w = build_workload(rng, name="many", dtype=BF16, num_q_heads=8, num_kv_heads=2, head_dim=64,
                       block_size=16, q_lens=q_lens, context_lens=ctx)
    log(f"{N} sequences, tile kind {kind}, partition {partition}")
    pkv.set_tuning(partition, 0, kind)
    dw = DeviceWorkload(w)
    out = dw.run_step(0)
    torch.cuda.synchronize()
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out), outs[0], BF16, f"{N} sequences kind={kind} P={partition}")


@pytest.mark.parametrize("dtype,kind", _PATHS)
def test_rejected_sequences_give_nan_rows(dtype, kind):
    """Sequences whose metadata the library rejects (more new tokens than cached ones, a negative context,
    a context longer than the table) get NaN output rows; the other sequences' rows are still right."""
    pkv.set_tuning(0, 0, kind)
    w = build_workload(np.random.default_rng(43), name="bad", dtype=dtype, num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, q_lens=[3, 2, 1, 4, 1], context_lens=[40, 30, 60, 20, 9])
    log(f"rejected sequences ({dtype}, tile kind {kind})")
    dw = DeviceWorkload(w)
    st = dw.steps[0]
    pkv.paged_kv_write(st["k_new"], st["v_new"], st["slot_mapping"], dw.k_pool, dw.v_pool)
    ctx = w.steps[0].context_lens.copy()
    ctx[1] = 1                                              # q_len 2 > context 1
    ctx[3] = -5                                             # negative context
    ctx[4] = w.block_tables.shape[1] * w.block_size + 1     # past the table
    out = torch.full_like(st["q"], 7.0)
    pkv.paged_attention_forward(st["q"], dw.k_pool, dw.v_pool, dw.block_tables, to_torch(ctx, None),
                                st["query_start_loc"], scale=w.scale, out=out, max_q_len=st["max_q_len"])
    torch.cuda.synchronize()
    got = out_f64(out)
    qsl = w.steps[0].query_start_loc
    for s in (1, 3, 4):
        assert np.all(np.isnan(got[qsl[s]:qsl[s + 1]])), s
    _, _, ref = oracle.run_step(w.k_pool, w.v_pool, w.block_tables, w.steps[0], w.scale, w.dtype, seqs=[0, 2])
    good = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in (0, 2)])
    check_close(got[good], ref[good], dtype, "valid sequences beside rejected ones")


@pytest.mark.parametrize("hint", [None, 1, 4096])
@pytest.mark.parametrize("name", ["mixed", "decode", "spec"])
def test_q_length_hint_only_changes_speed(name, hint):
    """The q-length hint only picks a kernel build: no hint (each sequence's tile kind chosen on the device),
    a hint too small for the batch (128-row tiles for every sequence, long chunks over several of them), or a
    loose one all give the oracle's result."""
    w = make_config(name, "small")
    log(f"small {name}, q-length hint {hint}")
    dw = DeviceWorkload(w)
    s = dw.steps[0]
    pkv.paged_kv_write(s["k_new"], s["v_new"], s["slot_mapping"], dw.k_pool, dw.v_pool)
    out = pkv.paged_attention_forward(s["q"], dw.k_pool, dw.v_pool, dw.block_tables, s["context_lens"],
                                      s["query_start_loc"], scale=w.scale, max_q_len=hint)
    torch.cuda.synchronize()
    _, _, outs = _oracle_steps(w)
    check_close(out_f64(out), outs[0], BF16, f"{name} hint={hint}")


def test_equal_contexts_one_item_per_workgroup_stay_unsplit():
    """As many single-token MQA sequences as the GPU has CUs (one workgroup each), with contexts within 10% of
    each other: the automatic plan leaves every context unsplit (partition length >= the longest context) and
    the result matches the oracle; the same count with contexts spread over 500-4000 keys is split."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for lo, hi, expect_unsplit in ((1900, 2100, True), (500, 4000, False)):
        n_seqs = cus
        rng = np.random.default_rng(53 + lo)
        ctx = rng.integers(lo, hi, n_seqs)
        w = build_workload(rng, name="even", dtype=BF16, num_q_heads=32, num_kv_heads=1, head_dim=128,
                           block_size=16, q_lens=[1] * n_seqs, context_lens=ctx)
        log(f"{n_seqs} MQA decodes, contexts {lo}-{hi}, on {cus} CUs")
        dw = DeviceWorkload(w)
        st = dw.steps[0]
        ws = torch.zeros(max(256, pkv.workspace_size(w.num_seqs, st["q"].shape[0], w.num_q_heads,
                                                     w.num_kv_heads, w.head_dim, st["q"].dtype, 1)),
                         dtype=torch.uint8, device=st["q"].device)
        pkv.paged_kv_write(st["k_new"], st["v_new"], st["slot_mapping"], dw.k_pool, dw.v_pool)
        out = pkv.paged_attention_forward(st["q"], dw.k_pool, dw.v_pool, dw.block_tables, st["context_lens"],
                                          st["query_start_loc"], scale=w.scale, workspace=ws, max_q_len=1)
        torch.cuda.synchronize()
        partition = int(ws[:64].cpu().numpy().view(np.int32)[2])
        assert (partition >= int(ctx.max())) == expect_unsplit, (n_seqs, partition, int(ctx.max()))
        _, _, outs = _oracle_steps(w)
        check_close(out_f64(out), outs[0], BF16, f"{n_seqs} MQA decodes, contexts {lo}-{hi}")
