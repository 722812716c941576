"""Paged KV-cache write and paged attention for MI355X (gfx950).

Thin Python binding over the C-ABI library ``libpagedkv.so`` (``include/paged_kv.h``).  It only turns
torch tensors into pointers, sizes and the current HIP stream; every step of the computation runs in
the library's kernels.  PyTorch supplies device memory and streams.

    paged_kv_write(k, v, slot_mapping, k_cache, v_cache)
    out = paged_attention_forward(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                                  scale=None)
    paged_attention_forward_noalloc(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                                    out)                       # no workspace: the library's fixed scratch
    mgr = CacheManager(num_blocks, block_size)        # host block allocator, tables, slot mapping
    slots, cow = mgr.append(seq_id, num_tokens)       # cow: (src, dst) block to copy_blocks() first

The two calls follow the problem as the pages state it: new K/V rows go through a slot mapping into
fixed-size physical blocks, and attention reads each sequence's K/V through its block table, with
several new tokens per sequence allowed ("Paged Attention 基础 – 原理与实现进度", §2 and §3.2; ADR 004
"Paged Attention Serving Integration", Decision 4 and Consequences; flash-attention issue 660 "Any plan
for support paged attention?").
"""

from __future__ import annotations

import math

import numpy as np
import torch

from ._native import (  # noqa: F401
    PKV_BF16,
    PKV_ERR_HIP,
    PKV_ERR_INVALID_ARG,
    PKV_ERR_UNSUPPORTED,
    PKV_ERR_WORKSPACE,
    PKV_FP32,
    PKV_OK,
    PagedKVError,
    check,
    lib,
)

__all__ = [
    "paged_kv_write",
    "paged_attention_forward",
    "paged_attention_write_forward",
    "paged_attention_forward_prefix",
    "paged_attention_forward_noalloc",
    "paged_attention_run",
    "paged_attention_run_prefix",
    "workspace_size",
    "prefix_workspace_size",
    "set_tuning",
    "set_profile_events",
    "validate_metadata",
    "PagedKVError",
    "CacheManager",
    "copy_blocks",
]

_DTYPES = {torch.bfloat16: PKV_BF16, torch.float32: PKV_FP32}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")
    return _DTYPES[t.dtype]


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _pool_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """(num_blocks, block_size, num_kv_heads, head_dim, block_stride) of a per-layer pool view."""
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must be 4-D [num_blocks, block_size, H_kv, D] views of one shape")
    nb, bs, hkv, d = k_cache.shape
    st = k_cache.stride()
    if st[3] != 1 or st[2] != d or st[1] != hkv * d:
        raise ValueError("each block of the pool must be a dense [block_size, H_kv, D] array")
    return nb, bs, hkv, d, st[0]


def _same_device(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t in ts:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _int32_vec(t: torch.Tensor, name: str):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")


def _write_args(k, v, slot_mapping, k_cache, v_cache, validate):
    dev = _same_device(k, v, slot_mapping, k_cache, v_cache)
    nb, bs, hkv, d, stride = _pool_geometry(k_cache, v_cache)
    if k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (hkv, d):
        raise ValueError("k and v must be [T, H_kv, D] matching the pool")
    if not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous")
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("k, v and the caches must share one dtype")
    _int32_vec(slot_mapping, "slot_mapping")
    if slot_mapping.numel() != k.shape[0]:
        raise ValueError("slot_mapping must have one entry per token")
    if validate:
        validate_metadata(slot_mapping=slot_mapping, num_blocks=nb, block_size=bs)
    return dev, nb, bs, hkv, d, stride


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, *, validate: bool = False) -> None:
    """Store row t of ``k``/``v`` ``[T, H_kv, D]`` at pool row ``slot_mapping[t]`` (block =
    slot // block_size, offset = slot % block_size) of ``k_cache``/``v_cache``; negative slots are
    skipped.  Asynchronous on the current stream."""
    dev, nb, bs, hkv, d, stride = _write_args(k, v, slot_mapping, k_cache, v_cache, validate)
    check(lib().paged_kv_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k.shape[0],
                               k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, stride, hkv, d,
                               _dtype_code(k), _stream(dev)))


def workspace_size(num_seqs: int, total_q: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   dtype: torch.dtype, max_q_len: int | None = None) -> int:
    n = lib().paged_attention_workspace_size(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                             _DTYPES[dtype], -1 if max_q_len is None else max_q_len)
    err = lib().paged_kv_last_error()
    if err:
        raise PagedKVError(PKV_ERR_INVALID_ARG, err.decode())
    return int(n)


def prefix_workspace_size(num_seqs: int, total_q: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          dtype: torch.dtype) -> int:
    n = lib().paged_attention_prefix_workspace_size(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim,
                                                    _DTYPES[dtype])
    err = lib().paged_kv_last_error()
    if err:
        raise PagedKVError(PKV_ERR_INVALID_ARG, err.decode())
    return int(n)


def _attention_args(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, validate):
    dev = _same_device(q, k_cache, v_cache, block_tables, context_lens, query_start_loc)
    nb, bs, hkv, d, stride = _pool_geometry(k_cache, v_cache)
    if q.dim() != 3 or q.shape[2] != d or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, H_q, D] tensor")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share one dtype")
    total_q, hq, _ = q.shape
    _int32_vec(context_lens, "context_lens")
    _int32_vec(query_start_loc, "query_start_loc")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_contiguous():
        raise TypeError("block_tables must be a contiguous 2-D int32 tensor")
    num_seqs = context_lens.numel()
    if block_tables.shape[0] != num_seqs or query_start_loc.numel() != num_seqs + 1:
        raise ValueError("block_tables, context_lens and query_start_loc disagree on the number of sequences")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous tensor like q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if validate:
        validate_metadata(block_tables=block_tables, context_lens=context_lens,
                          query_start_loc=query_start_loc, num_blocks=nb, block_size=bs,
                          total_q=total_q)
    return dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, float(scale)


# Workspaces the binding owns for callers that pass none: one per (device, stream), grown when a call needs
# more and reused otherwise.  Calls on one stream are ordered, so they can share it; calls on different
# streams get different ones.
_WORKSPACES: dict = {}


def _workspace(workspace, need, dev):
    if workspace is None:
        key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
        ws = _WORKSPACES.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
            _WORKSPACES[key] = ws
        return ws
    if workspace.device != dev or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor on q's device")
    return workspace


def paged_attention_forward(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor,
                            query_start_loc: torch.Tensor, scale: float | None = None,
                            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            max_q_len: int | None = None, validate: bool = False) -> torch.Tensor:
    """Causal paged attention; see ``paged_attention_forward`` in include/paged_kv.h.

    ``q`` ``[total_q, H_q, D]`` packs each sequence's new tokens at ``query_start_loc[s] :
    query_start_loc[s+1]``; ``context_lens[s]`` counts every cached token including them.  ``scale``
    defaults to ``1/sqrt(D)``.  ``workspace`` (uint8, device): when not given, the binding's own workspace for
    this device and stream (allocated once, grown when a call needs more).  ``max_q_len`` (optional, an upper
    bound on q_len) lets decode-like batches run the kernel build with only the 16-row body.  Returns
    ``out`` ``[total_q, H_q, D]`` in q's dtype.  Asynchronous on the current stream."""
    dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, scale = _attention_args(
        q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, validate)
    hint = -1 if max_q_len is None else int(max_q_len)
    workspace = _workspace(workspace, workspace_size(num_seqs, total_q, hq, hkv, d, q.dtype, max_q_len), dev)
    check(lib().paged_attention_forward(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), num_seqs, total_q,
        hq, hkv, d, bs, nb, stride, scale, _dtype_code(q), hint, workspace.data_ptr(),
        workspace.numel(), _stream(dev)))
    return out


def paged_attention_write_forward(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                  q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  query_start_loc: torch.Tensor, scale: float | None = None,
                                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                  max_q_len: int | None = None, validate: bool = False) -> torch.Tensor:
    """``paged_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache)`` then ``paged_attention_forward(q,
    k_cache, v_cache, ...)``: the same pools and output, one launch fewer (the work plan is made in the
    write's launch); see ``paged_attention_write_forward`` in include/paged_kv.h."""
    _write_args(k_new, v_new, slot_mapping, k_cache, v_cache, validate)
    dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, scale = _attention_args(
        q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, validate)
    hint = -1 if max_q_len is None else int(max_q_len)
    workspace = _workspace(workspace, workspace_size(num_seqs, total_q, hq, hkv, d, q.dtype, max_q_len), dev)
    check(lib().paged_attention_write_forward(
        k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(), k_new.shape[0], out.data_ptr(),
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), query_start_loc.data_ptr(), num_seqs, total_q, hq, hkv, d, bs, nb, stride,
        scale, _dtype_code(q), hint, workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return out


def paged_attention_run(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                        scale: float | None = None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, max_q_len: int | None = None) -> torch.Tensor:
    """``paged_attention_forward`` on the work plan the last attention call with this ``workspace`` made (the
    binding's own workspace for this device and stream when none is given), without planning again: for the
    layers after the first of a model step, whose metadata is the same; see ``paged_attention_run`` in
    include/paged_kv.h.  A workspace holding no plan for this call's shape gives an all-NaN output."""
    dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, scale = _attention_args(
        q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, False)
    hint = -1 if max_q_len is None else int(max_q_len)
    need = workspace_size(num_seqs, total_q, hq, hkv, d, q.dtype, max_q_len)
    if workspace is None:
        workspace = _WORKSPACES.get((dev.index, torch.cuda.current_stream(dev).cuda_stream))
        if need > 0 and (workspace is None or workspace.numel() < need):
            raise ValueError("no plan to run: call paged_attention_forward with this metadata first")
    workspace = _workspace(workspace, need, dev) if workspace is not None else None
    check(lib().paged_attention_run(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), num_seqs, total_q,
        hq, hkv, d, bs, nb, stride, scale, _dtype_code(q), hint,
        workspace.data_ptr() if workspace is not None else None, workspace.numel() if workspace is not None else 0,
        _stream(dev)))
    return out


def paged_attention_forward_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                    block_tables: torch.Tensor, context_lens: torch.Tensor,
                                    query_start_loc: torch.Tensor, out: torch.Tensor, scale: float | None = None,
                                    max_q_len: int | None = None, validate: bool = False) -> torch.Tensor:
    """``paged_attention_forward`` into the caller's ``out`` with no workspace and no device allocation in
    the library (its fixed per-GPU scratch instead; calls on one GPU must not overlap); see
    ``paged_attention_forward_noalloc`` in include/paged_kv.h."""
    dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, scale = _attention_args(
        q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, validate)
    hint = -1 if max_q_len is None else int(max_q_len)
    check(lib().paged_attention_forward_noalloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), num_seqs, total_q,
        hq, hkv, d, bs, nb, stride, scale, _dtype_code(q), hint, _stream(dev)))
    return out


def paged_attention_forward_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                                   query_start_loc: torch.Tensor, prefix_begin: int, prefix_end: int,
                                   prefix_tokens: int, scale: float | None = None,
                                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                   validate: bool = False) -> torch.Tensor:
    """``paged_attention_forward`` for a batch whose sequences ``prefix_begin .. prefix_end - 1`` share the
    blocks of their first ``prefix_tokens`` tokens: the shared keys are attended once for all of them.
    Same result; see ``paged_attention_forward_prefix`` in include/paged_kv.h.  ``validate`` also checks
    on the host that the range's block tables agree over the prefix."""
    dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, scale = _attention_args(
        q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, validate)
    if validate and prefix_tokens > 0 and prefix_end > prefix_begin:
        nblk = -(-int(prefix_tokens) // bs)
        rows = block_tables[prefix_begin:prefix_end, :nblk].cpu()
        if not bool((rows == rows[0:1]).all()):
            raise ValueError("the prefix range's block tables differ over the prefix")
    workspace = _workspace(workspace, prefix_workspace_size(num_seqs, total_q, hq, hkv, d, q.dtype), dev)
    check(lib().paged_attention_forward_prefix(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), num_seqs, total_q,
        hq, hkv, d, bs, nb, stride, scale, _dtype_code(q), int(prefix_begin), int(prefix_end),
        int(prefix_tokens), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return out


def paged_attention_run_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_tables: torch.Tensor, context_lens: torch.Tensor,
                               query_start_loc: torch.Tensor, prefix_begin: int, prefix_end: int,
                               prefix_tokens: int, scale: float | None = None, out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``paged_attention_forward_prefix`` on the work plan the last call with this ``workspace`` made (the
    binding's own workspace for this device and stream when none is given), without planning again: for the
    layers after the first of a model step; see ``paged_attention_run_prefix`` in include/paged_kv.h.  A
    workspace holding no plan for this call's shape and prefix range gives an all-NaN output."""
    dev, nb, bs, hkv, d, stride, total_q, hq, num_seqs, out, scale = _attention_args(
        q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, out, False)
    need = prefix_workspace_size(num_seqs, total_q, hq, hkv, d, q.dtype)
    if workspace is None:
        workspace = _WORKSPACES.get((dev.index, torch.cuda.current_stream(dev).cuda_stream))
        if need > 0 and (workspace is None or workspace.numel() < need):
            raise ValueError("no plan to run: call paged_attention_forward_prefix with this metadata first")
    workspace = _workspace(workspace, need, dev) if workspace is not None else None
    check(lib().paged_attention_run_prefix(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), query_start_loc.data_ptr(), num_seqs, total_q,
        hq, hkv, d, bs, nb, stride, scale, _dtype_code(q), int(prefix_begin), int(prefix_end), int(prefix_tokens),
        workspace.data_ptr() if workspace is not None else None, workspace.numel() if workspace is not None else 0,
        _stream(dev)))
    return out


def set_tuning(partition_keys: int = 0, target_items: int = 0, tile_kind: int = 0) -> None:
    """Work division knobs (0 = automatic); see paged_attention_set_tuning in include/paged_kv.h."""
    check(lib().paged_attention_set_tuning(partition_keys, target_items, tile_kind))


def set_profile_events(start_event: int | None, stop_event: int | None) -> None:
    """Raw hipEvent_t handles recorded around the main attention kernel (None, None to stop)."""
    check(lib().paged_attention_set_profile_events(start_event, stop_event))


def validate_metadata(*, block_tables=None, context_lens=None, query_start_loc=None, slot_mapping=None,
                      num_blocks: int, block_size: int, total_q: int | None = None) -> None:
    """Debug check of metadata contents on the host (copies them off the device).  Raises ValueError on
    anything the library treats as outside its supported inputs."""
    if slot_mapping is not None:
        sm = slot_mapping.cpu().numpy().astype(np.int64)
        live = sm[sm >= 0]
        if np.any(live >= num_blocks * block_size):
            raise ValueError("slot outside the pool")
        if np.unique(live).size != live.size:
            raise ValueError("a slot is repeated within one write")
    if context_lens is not None:
        L = context_lens.cpu().numpy().astype(np.int64)
        qsl = query_start_loc.cpu().numpy().astype(np.int64)
        bt = block_tables.cpu().numpy()
        if qsl[0] != 0 or np.any(np.diff(qsl) < 0) or (total_q is not None and qsl[-1] != total_q):
            raise ValueError("query_start_loc must start at 0, not decrease, and end at total_q")
        n = np.diff(qsl)
        if np.any(n > L):
            raise ValueError("a sequence has more new tokens than cached tokens")
        nblk = -(-L // block_size)
        if np.any(nblk > bt.shape[1]):
            raise ValueError("a context is longer than max_blocks_per_seq * block_size")
        for s in range(len(L)):
            row = bt[s, :nblk[s]]
            if np.any(row < 0) or np.any(row >= num_blocks):
                raise ValueError(f"sequence {s} names a block outside the pool")


from .cache_manager import CacheManager, copy_blocks  # noqa: E402  (uses the helpers above)
