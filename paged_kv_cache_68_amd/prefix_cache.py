"""Python binding of the library's host prefix cache (C ABI: the kv_pc_* calls of
include/pagedkv.h).  Argument marshalling only: the bookkeeping runs in the library."""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import check, lib
from .block_manager import _check

__all__ = ["PrefixCache", "hash_block"]


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def hash_block(prev: int, tokens, first: bool = False, salt: int = 0) -> int:
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    return int(lib().kv_pc_hash_block(prev, _p(t) if t.size else None, int(t.size), int(first), salt))


class PrefixCache:
    """Block pool with automatic prefix caching (integer request ids)."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        h = ctypes.c_void_p()
        check(lib().kv_pc_create(int(num_blocks), int(block_size), ctypes.byref(h)), "kv_pc_create")
        self.handle = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().kv_pc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, rid: int, prompt, salt: int = 0) -> int:
        p = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))
        found = ctypes.c_int32()
        check(lib().kv_pc_add_request(self.handle, int(rid), _p(p) if p.size else None, int(p.size),
                                      int(salt), ctypes.byref(found)), "kv_pc_add_request")
        return found.value

    def append(self, rid: int, tokens):
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        slots = np.empty(max(1, t.size), dtype=np.int64)
        _check(lib().kv_pc_append(self.handle, int(rid), _p(t) if t.size else None, int(t.size),
                                  _p(slots), int(t.size)), "kv_pc_append")
        return slots[:t.size]

    def append_step(self, rids, tokens):
        """One decode step: token tokens[i] for the distinct requests rids[i]; their slots.
        All or nothing."""
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        if r.shape != t.shape or r.ndim != 1:
            raise ValueError("rids and tokens must be 1-D of the same length")
        slots = np.empty(max(1, r.size), dtype=np.int64)
        _check(lib().kv_pc_append_step(self.handle, _p(r) if r.size else None,
                                       _p(t) if t.size else None, int(r.size), _p(slots)),
               "kv_pc_append_step")
        return slots[:r.size]

    def free_request(self, rid: int) -> None:
        check(lib().kv_pc_free_request(self.handle, int(rid)), "kv_pc_free_request")

    def length(self, rid: int) -> int:
        v = ctypes.c_int32()
        check(lib().kv_pc_get_length(self.handle, int(rid), ctypes.byref(v)), "kv_pc_get_length")
        return v.value

    def table(self, rid: int):
        buf = np.empty(max(1, -(-self.length(rid) // self.block_size)), dtype=np.int32)
        n = ctypes.c_int32()
        check(lib().kv_pc_get_table(self.handle, int(rid), _p(buf), buf.size, ctypes.byref(n)),
              "kv_pc_get_table")
        return buf[:n.value].tolist()

    def export(self, rids, max_blocks: int):
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        tables = np.empty((max(1, r.size), int(max_blocks)), dtype=np.int32)
        lens = np.empty(max(1, r.size), dtype=np.int32)
        check(lib().kv_pc_export(self.handle, _p(r), int(r.size), int(max_blocks), _p(tables), _p(lens)),
              "kv_pc_export")
        return tables[:r.size], lens[:r.size]

    def num_free(self) -> int:
        return int(lib().kv_pc_num_free(self.handle))

    def num_cached(self) -> int:
        return int(lib().kv_pc_num_cached(self.handle))

    def free_queue(self):
        buf = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32()
        check(lib().kv_pc_free_queue(self.handle, _p(buf), self.num_blocks, ctypes.byref(n)),
              "kv_pc_free_queue")
        return buf[:n.value].tolist()

    def block_info(self, block: int):
        """(reference count, cached, hash or None)."""
        ref, cached, h = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint64()
        check(lib().kv_pc_block_info(self.handle, int(block), ctypes.byref(ref), ctypes.byref(cached),
                                     ctypes.byref(h)), "kv_pc_block_info")
        return ref.value, bool(cached.value), (h.value if cached.value else None)
