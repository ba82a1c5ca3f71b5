"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Thin Python binding over ``libpagedkv.so`` (C ABI: include/pagedkv.h).  PyTorch is
used only for device memory, pointers and streams; every step of the decode path
(cache write, block-table gather, q.K^T, online softmax, P.V, partition reduce) runs
in the library's HIP kernels.  Names and argument order follow the C ABI.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional

from ._lib import (  # noqa: F401
    KV_DTYPE_BF16, KV_DTYPE_F16, KV_DTYPE_FP8_E4M3, KV_ERR_HIP, KV_ERR_INVALID_ARG, KV_ERR_OUT_OF_MEMORY,
    KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE, KV_OK, KVPoolDesc, PagedKVError, check, lib,
    status_string,
)

__all__ = [
    "KVPool", "kv_pool_bytes", "kv_bytes_per_token", "reshape_and_cache",
    "paged_attention_workspace_bytes", "paged_attention_decode", "paged_attention_partitions",
    "paged_attention_reduce", "kv_pool_gather", "make_desc", "PagedKVError",
    "BlockManager", "OutOfBlocks", "copy_blocks", "paged_attention_prefill", "PrefixCache",
    "hash_block", "swap_blocks", "paged_attention_decode_append", "paged_attention_partitions_append",
    "paged_attention_prefill_split", "prefill_workspace_bytes", "alloc_prefill_workspace",
]

BLOCK_SIZE = 16
DEFAULT_PARTITION = 512


def _torch():
    import torch
    return torch


def _dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    torch = _torch()
    if dtype in ("f16", "float16", torch.float16):
        return KV_DTYPE_F16
    if dtype in ("bf16", "bfloat16", torch.bfloat16):
        return KV_DTYPE_BF16
    if dtype in ("fp8", "fp8_e4m3", "float8_e4m3fn", torch.float8_e4m3fn):
        return KV_DTYPE_FP8_E4M3
    raise ValueError(f"unsupported dtype {dtype}")


def _torch_dtype(code: int):
    """torch dtype of a pool's stored elements (E4M3 codes are viewed as uint8)."""
    torch = _torch()
    return {KV_DTYPE_F16: torch.float16, KV_DTYPE_BF16: torch.bfloat16,
            KV_DTYPE_FP8_E4M3: torch.uint8}[code]


def make_desc(num_layers, num_blocks, num_kv_heads, head_dim, dtype, block_size=BLOCK_SIZE,
              io_dtype=None):
    """Pool descriptor.  ``dtype`` is the storage of K and V (f16, bf16 or fp8);
    ``io_dtype`` the 16-bit type of queries, outputs and new keys / values (default:
    ``dtype`` for a 16-bit pool, bf16 for an FP8 pool)."""
    code = _dtype_code(dtype)
    io = _dtype_code(io_dtype) if io_dtype is not None else (
        KV_DTYPE_BF16 if code == KV_DTYPE_FP8_E4M3 else code)
    return KVPoolDesc(int(num_layers), int(num_blocks), int(block_size), int(num_kv_heads),
                      int(head_dim), code, io)


def kv_pool_bytes(desc: KVPoolDesc) -> int:
    return int(lib().kv_pool_bytes(ctypes.byref(desc)))


def kv_bytes_per_token(desc: KVPoolDesc) -> int:
    return int(lib().kv_bytes_per_token(ctypes.byref(desc)))


def _stream(stream) -> int:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class KVPool:
    """A paged K/V pool: ``num_layers`` layers of K and V caches, each
    [num_blocks][16][num_kv_heads][head_dim].  The memory is a torch tensor owned by
    this object (or caller memory passed as ``base``); the library handle borrows it.
    """

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, dtype,
                 block_size=BLOCK_SIZE, device=None, base=None, io_dtype=None, host=False):
        torch = _torch()
        self.host = bool(host)
        self.desc = make_desc(num_layers, num_blocks, num_kv_heads, head_dim, dtype, block_size,
                              io_dtype)
        nbytes = kv_pool_bytes(self.desc)
        if nbytes == 0:
            # let the library name the problem
            h = ctypes.c_void_p()
            check(lib().kv_pool_create(ctypes.byref(self.desc), None, 0, ctypes.byref(h)),
                  "kv_pool_create")
            raise PagedKVError(KV_ERR_INVALID_ARG, "kv_pool_create")
        self.dtype = _torch_dtype(self.desc.dtype)            # stored K / V elements
        self.io_dtype = _torch_dtype(self.desc.io_dtype)      # queries, outputs, new K / V
        h = ctypes.c_void_p()
        if self.host:
            # pinned host memory for swapped-out blocks: the library's own allocation
            # (or the caller's pinned CPU tensor); ``memory`` is a CPU view of it, valid
            # while the pool lives
            ptr, size = (None, 0) if base is None else (base.data_ptr(),
                                                        base.numel() * base.element_size())
            check(lib().kv_host_pool_create(ctypes.byref(self.desc), ptr, size, ctypes.byref(h)),
                  "kv_host_pool_create")
            self.handle = h
            if base is None:
                k0 = ctypes.c_void_p()
                check(lib().kv_pool_layer_ptrs(h, 0, ctypes.byref(k0), None), "kv_pool_layer_ptrs")
                base = torch.frombuffer((ctypes.c_uint8 * nbytes).from_address(k0.value),
                                        dtype=torch.uint8)
            self.memory = base
            return
        if base is None:
            dev = torch.device(device if device is not None else "cuda")
            base = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.memory = base
        check(lib().kv_pool_create(ctypes.byref(self.desc), base.data_ptr(),
                                   base.numel() * base.element_size(), ctypes.byref(h)),
              "kv_pool_create")
        self.handle = h

    @property
    def num_layers(self):
        return self.desc.num_layers

    @property
    def num_blocks(self):
        return self.desc.num_blocks

    @property
    def num_kv_heads(self):
        return self.desc.num_kv_heads

    @property
    def head_dim(self):
        return self.desc.head_dim

    def _cache(self, layer: int, which: int):
        per = self.desc.num_blocks * self.desc.block_size * self.desc.num_kv_heads * self.desc.head_dim
        flat = self.memory.view(self.dtype)
        start = (2 * layer + which) * per
        return flat[start:start + per].view(self.desc.num_blocks, self.desc.block_size,
                                            self.desc.num_kv_heads, self.desc.head_dim)

    def k_cache(self, layer: int = 0):
        return self._cache(layer, 0)

    def v_cache(self, layer: int = 0):
        return self._cache(layer, 1)

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            if self.host:
                self.memory = None          # a view of memory the library frees next
            check(lib().kv_pool_destroy(self.handle), "kv_pool_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def reshape_and_cache(pool: KVPool, layer: int, key, value, slot_mapping, stream=None) -> None:
    """Write key[i], value[i] ([T, Hkv, D]) into slot slot_mapping[i] (int64) of ``layer``."""
    n = int(slot_mapping.shape[0])
    check(lib().reshape_and_cache(pool.handle, int(layer), _ptr(key), _ptr(value),
                                  _ptr(slot_mapping), n, _stream(stream)),
          "reshape_and_cache")


def paged_attention_workspace_bytes(batch, num_q_heads, head_dim, max_blocks_per_seq,
                                    block_size=BLOCK_SIZE, partition_size=0) -> int:
    return int(lib().paged_attention_workspace_bytes(int(batch), int(num_q_heads), int(head_dim),
                                                     int(max_blocks_per_seq), int(block_size),
                                                     int(partition_size)))


def alloc_workspace(pool: KVPool, batch, num_q_heads, max_blocks_per_seq, partition_size=0,
                    device=None):
    torch = _torch()
    n = paged_attention_workspace_bytes(batch, num_q_heads, pool.head_dim, max_blocks_per_seq,
                                        pool.desc.block_size, partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device or pool.memory.device)


def _decode_call(fn_name, pool, layer, out, query, block_tables, context_lens, scale,
                 partition_size, workspace, stream):
    batch, hq, d = (int(x) for x in query.shape)
    max_blocks = int(block_tables.shape[1]) if block_tables.dim() == 2 else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = getattr(lib(), fn_name)
    check(fn(pool.handle, int(layer), _ptr(out), _ptr(query), _ptr(block_tables), max_blocks,
             _ptr(context_lens), batch, hq, float(scale), int(partition_size), _ptr(workspace),
             ws_bytes, _stream(stream)),
          fn_name)


def paged_attention_decode(pool: KVPool, layer: int, out, query, block_tables, context_lens,
                           scale=None, partition_size=0, workspace=None, stream=None):
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the sequence's paged K/V."""
    if workspace is None:
        workspace = alloc_workspace(pool, query.shape[0], query.shape[1], block_tables.shape[1],
                                    partition_size)
    _decode_call("paged_attention_decode", pool, layer, out, query, block_tables, context_lens,
                 scale, partition_size, workspace, stream)
    return out


def _append_call(fn_name, pool, layer, out, query, new_key, new_value, block_tables,
                 context_lens, scale, partition_size, workspace, stream):
    batch, hq, d = (int(x) for x in query.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None and fn_name == "paged_attention_decode_append":
        workspace = alloc_workspace(pool, batch, hq, block_tables.shape[1], partition_size)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(getattr(lib(), fn_name)(pool.handle, int(layer), _ptr(out), _ptr(query), _ptr(new_key),
                                  _ptr(new_value), _ptr(block_tables), int(block_tables.shape[1]),
                                  _ptr(context_lens), batch, hq, float(scale), int(partition_size),
                                  _ptr(workspace), ws_bytes, _stream(stream)),
          fn_name)


def paged_attention_decode_append(pool: KVPool, layer: int, out, query, new_key, new_value,
                                  block_tables, context_lens, scale=None, partition_size=0,
                                  workspace=None, stream=None):
    """Write new_key[b] / new_value[b] ([B, Hkv, D]) at position context_lens[b] - 1 of
    each sequence (slot through its table), then decode: reshape_and_cache + decode in
    fewer launches."""
    _append_call("paged_attention_decode_append", pool, layer, out, query, new_key, new_value,
                 block_tables, context_lens, scale, partition_size, workspace, stream)
    return out


def paged_attention_partitions_append(pool, layer, out, query, new_key, new_value, block_tables,
                                      context_lens, scale=None, partition_size=0, workspace=None,
                                      stream=None):
    _append_call("paged_attention_partitions_append", pool, layer, out, query, new_key, new_value,
                 block_tables, context_lens, scale, partition_size, workspace, stream)


def paged_attention_partitions(pool, layer, out, query, block_tables, context_lens, scale=None,
                               partition_size=0, workspace=None, stream=None):
    _decode_call("paged_attention_partitions", pool, layer, out, query, block_tables,
                 context_lens, scale, partition_size, workspace, stream)


def paged_attention_reduce(pool, layer, out, query, block_tables, context_lens, scale=None,
                           partition_size=0, workspace=None, stream=None):
    _decode_call("paged_attention_reduce", pool, layer, out, query, block_tables, context_lens,
                 scale, partition_size, workspace, stream)


def paged_attention_prefill(pool: KVPool, layer: int, out, query, query_start, max_query_len,
                            block_tables, context_lens, scale=None, stream=None) -> None:
    """Causal attention of each sequence's chunk of new tokens (rows
    [query_start[b], query_start[b+1]) of ``query``) over its paged K/V."""
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    batch = int(context_lens.shape[0])
    check(lib().paged_attention_prefill(pool.handle, int(layer), _ptr(out), _ptr(query),
                                        _ptr(query_start), int(max_query_len), _ptr(block_tables),
                                        int(block_tables.shape[1]), _ptr(context_lens), batch,
                                        int(query.shape[1]), float(scale), _stream(stream)),
          "paged_attention_prefill")


def prefill_workspace_bytes(pool: KVPool, batch, num_q_heads, num_tokens, max_query_len,
                            max_blocks_per_seq) -> int:
    """Workspace bytes paged_attention_prefill_split needs for these shapes (0: none)."""
    return int(lib().paged_attention_prefill_workspace_bytes(pool.handle, int(batch), int(num_q_heads),
                                                            int(num_tokens), int(max_query_len),
                                                            int(max_blocks_per_seq)))


def alloc_prefill_workspace(pool: KVPool, batch, num_q_heads, num_tokens, max_query_len,
                            max_blocks_per_seq, device=None):
    n = prefill_workspace_bytes(pool, batch, num_q_heads, num_tokens, max_query_len, max_blocks_per_seq)
    if n == 0:
        return None
    torch = _torch()
    return torch.empty(n, dtype=torch.uint8, device=device or pool.memory.device)


def paged_attention_prefill_split(pool: KVPool, layer: int, out, query, query_start, max_query_len,
                                  block_tables, context_lens, scale=None, workspace=None,
                                  stream=None) -> None:
    """paged_attention_prefill with each row tile's keys split over several work-groups
    when the launch is too small to fill the GPU (partial results in ``workspace``)."""
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    batch = int(context_lens.shape[0])
    num_tokens = int(query.shape[0])
    nbytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    check(lib().paged_attention_prefill_split(pool.handle, int(layer), _ptr(out), _ptr(query),
                                              _ptr(query_start), int(max_query_len), num_tokens,
                                              _ptr(block_tables), int(block_tables.shape[1]),
                                              _ptr(context_lens), batch, int(query.shape[1]),
                                              float(scale), _ptr(workspace) if workspace is not None else None,
                                              nbytes, _stream(stream)),
          "paged_attention_prefill_split")


def kv_pool_gather(pool: KVPool, layer: int, block_tables, context_lens, k_out, v_out,
                   stream=None) -> None:
    batch = int(context_lens.shape[0])
    check(lib().kv_pool_gather(pool.handle, int(layer), _ptr(block_tables),
                               int(block_tables.shape[1]), _ptr(context_lens), batch, _ptr(k_out),
                               _ptr(v_out), _stream(stream)),
          "kv_pool_gather")


from .block_manager import BlockManager, OutOfBlocks, copy_blocks, swap_blocks  # noqa: E402
from .prefix_cache import PrefixCache, hash_block  # noqa: E402
