"""Python binding of the library's host block manager (C ABI: the kv_bm_* calls of
include/pagedkv.h) and of the device copy-on-write copy.  Argument marshalling only:
the bookkeeping runs in the library's C++ code, the copies in its HIP kernel.
"""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import KV_ERR_OUT_OF_BLOCKS, PagedKVError, check, lib

__all__ = ["BlockManager", "OutOfBlocks", "copy_blocks", "swap_blocks"]


class OutOfBlocks(PagedKVError):
    """The free list cannot cover the appends; the manager did not change."""


def _check(status: int, what: str) -> None:
    if status == KV_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocks(status, what)
    check(status, what)


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


class BlockManager:
    """Free list, reference counts and per-request block tables (integer request ids)."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        h = ctypes.c_void_p()
        check(lib().kv_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)), "kv_bm_create")
        self.handle = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().kv_bm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, rid: int) -> None:
        check(lib().kv_bm_add_request(self.handle, int(rid)), "kv_bm_add_request")

    def fork(self, parent: int, child: int) -> None:
        check(lib().kv_bm_fork(self.handle, int(parent), int(child)), "kv_bm_fork")

    def free(self, rid: int) -> None:
        check(lib().kv_bm_free_request(self.handle, int(rid)), "kv_bm_free_request")

    def append_batch(self, rids, counts=None):
        """Slots for counts[i] tokens of rids[i] (one each if counts is None), and the
        copy-on-write copies.  Returns (slots int64 [sum counts], copies int32 [k, 3])."""
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        n = r.shape[0]
        c = None if counts is None else np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
        total = n if c is None else int(np.maximum(c, 0).sum())
        slots = np.empty(max(total, 1), dtype=np.int64)
        copies = np.empty((max(n, 1), 3), dtype=np.int32)
        nc = ctypes.c_int32()
        _check(lib().kv_bm_append(self.handle, _p(r) if n else None,
                                  _p(c) if c is not None else None, n, _p(slots), total,
                                  _p(copies), n, ctypes.byref(nc)), "kv_bm_append")
        return slots[:total], copies[:nc.value]

    def length(self, rid: int) -> int:
        v = ctypes.c_int32()
        check(lib().kv_bm_get_length(self.handle, int(rid), ctypes.byref(v)), "kv_bm_get_length")
        return v.value

    def table(self, rid: int):
        n = self.length(rid)
        buf = np.empty(max(1, -(-n // self.block_size)), dtype=np.int32)
        got = ctypes.c_int32()
        check(lib().kv_bm_get_table(self.handle, int(rid), _p(buf), buf.shape[0], ctypes.byref(got)),
              "kv_bm_get_table")
        return buf[:got.value].tolist()

    def export(self, rids, max_blocks: int):
        """(tables int32 [n, max_blocks] padded with -1, lengths int32 [n])."""
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        n = r.shape[0]
        tables = np.empty((max(n, 1), int(max_blocks)), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        check(lib().kv_bm_export(self.handle, _p(r), n, int(max_blocks), _p(tables), _p(lens)),
              "kv_bm_export")
        return tables[:n], lens[:n]

    def num_free(self) -> int:
        return int(lib().kv_bm_num_free(self.handle))

    def ref_count(self, block: int) -> int:
        v = ctypes.c_int32()
        check(lib().kv_bm_ref_count(self.handle, int(block), ctypes.byref(v)), "kv_bm_ref_count")
        return v.value

    def move_to(self, dst: "BlockManager", rids):
        """Swap: move requests to manager ``dst`` (device to host, or back).  Returns the
        copies as int32 (src block, dst block) pairs [k, 2] for ``swap_blocks``."""
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        n = r.shape[0]
        cap = sum(len(self.table(int(x))) for x in r) if n else 0
        pairs = np.empty((max(cap, 1), 2), dtype=np.int32)
        got = ctypes.c_int32()
        _check(lib().kv_bm_move(self.handle, dst.handle, _p(r) if n else None, n, _p(pairs), cap,
                                ctypes.byref(got)), "kv_bm_move")
        return pairs[:got.value]

    def free_list(self):
        buf = np.empty(self.num_blocks, dtype=np.int32)
        got = ctypes.c_int32()
        check(lib().kv_bm_free_list(self.handle, _p(buf), self.num_blocks, ctypes.byref(got)),
              "kv_bm_free_list")
        return buf[:got.value].tolist()


def copy_blocks(pool, copies, stream=None) -> None:
    """Device copy-on-write copies for every layer: copies is an int32 device tensor
    [k, 3] of (src, dst, rows) on the pool's device."""
    import torch
    from . import _need, _stream
    _need(copies, "copies", torch.int32, (None, 3), device=pool.device)
    n = int(copies.shape[0])
    check(lib().kv_copy_blocks(pool.handle, copies.data_ptr() if n else None, n, _stream(stream)),
          "kv_copy_blocks")


def swap_blocks(src_pool, dst_pool, pairs, stream=None) -> None:
    """Swap copies: every layer's K and V of block pairs[i, 0] of ``src_pool`` go to block
    pairs[i, 1] of ``dst_pool`` (one of them a host pool).  ``pairs`` is an int32 tensor
    [k, 2] on the GPU, or in pinned host memory."""
    import torch
    from . import _need, _stream
    if not isinstance(pairs, torch.Tensor):
        raise ValueError(f"pairs: expected a torch.Tensor, got {type(pairs).__name__}")
    if pairs.device.type == "cpu":
        if not pairs.is_pinned():
            raise ValueError("pairs: a host tensor must be in pinned memory")
        _need(pairs, "pairs", torch.int32, (None, 2), device=pairs.device)
    else:
        _need(pairs, "pairs", torch.int32, (None, 2))
    n = int(pairs.shape[0])
    check(lib().kv_swap_blocks(src_pool.handle, dst_pool.handle, pairs.data_ptr() if n else None,
                               n, _stream(stream)), "kv_swap_blocks")
