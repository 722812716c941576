"""Python view of the library's host cache manager (``pkv_cm_*`` in include/paged_kv.h) and of its device
block copy.  Argument marshalling only: allocation, tables, slot mapping and reference counting run in
the C++ manager, the block copy in the HIP kernel.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._native import PKV_ERR_INVALID_ARG, PagedKVError, check, lib


class CacheManager:
    """Blocks of ``block_size`` tokens, ``num_blocks`` of them, shared by reference counting.

    ``append`` is the per-step update (fresh or growing sequence): it returns the slots to pass to
    ``paged_kv_write`` and, when the last block was shared and partly filled, the (src, dst) block pair to
    copy first (``copy_blocks``).  ``build_tables`` gives the block tables and context lengths of a batch.
    """

    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        self._h = lib().pkv_cm_create(self.num_blocks, self.block_size)
        if not self._h:
            raise PagedKVError(PKV_ERR_INVALID_ARG, lib().paged_kv_last_error().decode(errors="replace"))

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().pkv_cm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def num_free(self) -> int:
        return int(lib().pkv_cm_num_free(self._h))

    def seq_len(self, seq_id: int) -> int:
        return int(lib().pkv_cm_seq_len(self._h, int(seq_id)))

    def append(self, seq_id: int, num_tokens: int):
        slots = np.empty(max(0, int(num_tokens)), dtype=np.int32)
        cow = (ctypes.c_int32 * 2)()
        check(lib().pkv_cm_append(self._h, int(seq_id), int(num_tokens),
                                  slots.ctypes.data if slots.size else None, ctypes.addressof(cow)))
        return slots, (None if cow[0] < 0 else (int(cow[0]), int(cow[1])))

    def free(self, seq_id: int) -> None:
        check(lib().pkv_cm_free(self._h, int(seq_id)))

    def fork(self, parent: int, child: int) -> None:
        check(lib().pkv_cm_fork(self._h, int(parent), int(child)))

    def add_prefix(self, key: int, seq_id: int, num_tokens: int) -> None:
        check(lib().pkv_cm_add_prefix(self._h, int(key), int(seq_id), int(num_tokens)))

    def attach_prefix(self, key: int, seq_id: int) -> int:
        got = ctypes.c_int32(0)
        check(lib().pkv_cm_attach_prefix(self._h, int(key), int(seq_id), ctypes.addressof(got)))
        return int(got.value)

    def drop_prefix(self, key: int) -> None:
        check(lib().pkv_cm_drop_prefix(self._h, int(key)))

    def build_tables(self, seq_ids, max_blocks_per_seq: int):
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        tables = np.empty((ids.size, int(max_blocks_per_seq)), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        check(lib().pkv_cm_build_tables(self._h, ids.ctypes.data if ids.size else None, int(ids.size),
                                        int(max_blocks_per_seq), tables.ctypes.data if ids.size else None,
                                        lens.ctypes.data if ids.size else None))
        return tables, lens


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs) -> None:
    """Block ``dst`` of both caches takes block ``src``'s contents, for each (src, dst) in ``pairs`` (on
    the current stream).  ``pairs``: a sequence of pairs or an int32 tensor [n, 2]."""
    from . import _dtype_code, _pool_geometry, _same_device, _stream

    dev = _same_device(k_cache, v_cache)
    nb, bs, hkv, d, stride = _pool_geometry(k_cache, v_cache)
    if v_cache.dtype != k_cache.dtype:
        raise TypeError("the caches must share one dtype")
    p = torch.as_tensor(pairs, dtype=torch.int32).reshape(-1, 2)
    if p.shape[0] == 0:
        return
    p = p.to(dev)
    src = p[:, 0].contiguous()
    dst = p[:, 1].contiguous()
    check(lib().paged_kv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, stride, hkv, d,
                                     _dtype_code(k_cache), src.data_ptr(), dst.data_ptr(), int(p.shape[0]),
                                     _stream(dev)))


__all__ = ["CacheManager", "copy_blocks"]
