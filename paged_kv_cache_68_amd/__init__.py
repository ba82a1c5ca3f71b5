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
    "DecodeStep", "paged_attention_decode_noalloc", "paged_attention_decode_shared_prefix",
    "shared_prefix_workspace_bytes", "alloc_shared_prefix_workspace", "shared_prefix_blocks",
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


# ---------------------------------------------------------------- argument checks
# The C ABI sees only addresses and counts, not buffer sizes, so a tensor of the wrong
# type, shape or device would make the kernels read or write outside it.  Every entry
# point below checks its tensors here first and raises ValueError on a mismatch, before
# anything reaches the library.

def _need(t, name, dtype=None, shape=None, ndim=None, device=None):
    """Check that ``t`` is a dense tensor on ``device`` (a torch.device; None: any CUDA
    device) with the given dtype and shape (None entries of ``shape`` match any size)."""
    try:                      # fast path: everything as asked
        if ((dtype is None or t.dtype == dtype) and t.is_contiguous() and
                (t.is_cuda if device is None else
                 (t.is_cuda and t.get_device() == device.index) if device.type == "cuda" else
                 t.device == device)):
            if shape is not None:
                got = t.shape
                if len(got) == len(shape) and all(w is None or g == w for g, w in zip(got, shape)):
                    return t
            elif ndim is None or t.dim() == ndim:
                return t
    except AttributeError:
        pass
    _explain(t, name, dtype, shape, ndim, device)
    return t


def _explain(t, name, dtype, shape, ndim, device):
    """Raise ValueError naming what is wrong with ``t``."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if device is None:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
    elif t.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}, got one on {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != w for g, w in zip(t.shape, shape)):
            want = tuple("*" if w is None else w for w in shape)
            raise ValueError(f"{name}: expected shape {want}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    raise ValueError(f"{name}: not accepted")


def _need_bytes(t, name, device):
    """A raw device buffer (workspace): any dtype, contiguous, on ``device``."""
    if t is None:
        return None
    return _need(t, name, device=device)


def _decode_args_ok(pool, out, query, block_tables, context_lens, new_key, new_value, workspace):
    """The common case in one expression: every tensor as _check_decode_args wants it."""
    torch = _torch()
    dt, i32 = pool.io_dtype, torch.int32
    di = pool.device_index
    b, hq, d = query.shape
    ok = (query.dtype == dt and out.dtype == dt and d == pool.head_dim and hq > 0 and
          hq % pool.num_kv_heads == 0 and out.shape == query.shape and
          block_tables.dtype == i32 and context_lens.dtype == i32 and block_tables.dim() == 2 and
          block_tables.shape[0] == b and context_lens.dim() == 1 and context_lens.shape[0] == b and
          query.get_device() == di and out.get_device() == di and block_tables.get_device() == di and
          context_lens.get_device() == di and query.is_contiguous() and out.is_contiguous() and
          block_tables.is_contiguous() and context_lens.is_contiguous())
    if ok and (new_key is not None or new_value is not None):
        row = (b, pool.num_kv_heads, d)
        ok = (new_key.dtype == dt and new_value.dtype == dt and new_key.shape == row and
              new_value.shape == row and new_key.get_device() == di and
              new_value.get_device() == di and new_key.is_contiguous() and new_value.is_contiguous())
    if ok and workspace is not None:
        ok = workspace.get_device() == di and workspace.is_contiguous()
    return ok


def _check_decode_args(pool, out, query, block_tables, context_lens, new_key=None, new_value=None,
                       workspace=None):
    """Shapes of a decode call: query / out [B, Hq, D] in the pool's io dtype with D the
    pool's head size and Hq a multiple of its KV heads; tables int32 [B, max_blocks];
    lengths int32 [B]; new keys / values [B, Hkv, D]; all on the pool's device."""
    try:
        fast = _decode_args_ok(pool, out, query, block_tables, context_lens, new_key, new_value,
                               workspace)
    except (AttributeError, TypeError, ValueError):
        fast = False
    if fast:
        return int(query.shape[0]), int(query.shape[1]), int(block_tables.shape[1])
    dev = pool.device
    _need(query, "query", pool.io_dtype, ndim=3, device=dev)
    batch, hq, d = (int(x) for x in query.shape)
    if d != pool.head_dim:
        raise ValueError(f"query: head size {d} differs from the pool's {pool.head_dim}")
    if hq < 1 or hq % pool.num_kv_heads:
        raise ValueError(f"query: {hq} heads is not a multiple of the pool's {pool.num_kv_heads} KV heads")
    _need(out, "out", pool.io_dtype, (batch, hq, d), device=dev)
    _need(block_tables, "block_tables", _torch().int32, (batch, None), device=dev)
    _need(context_lens, "context_lens", _torch().int32, (batch,), device=dev)
    if new_key is not None or new_value is not None:
        _need(new_key, "new_key", pool.io_dtype, (batch, pool.num_kv_heads, d), device=dev)
        _need(new_value, "new_value", pool.io_dtype, (batch, pool.num_kv_heads, d), device=dev)
    _need_bytes(workspace, "workspace", dev)
    return batch, hq, int(block_tables.shape[1])


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

    @property
    def block_size(self):
        return self.desc.block_size

    @property
    def device_index(self):
        """Index of the pool's GPU, as torch's get_device() gives it."""
        return self.device.index

    @property
    def device(self):
        """The GPU the pool lives on; the attention and cache-write calls need their
        tensors there.  A host pool (swap target) has none and refuses those calls."""
        if self.host:
            raise ValueError("this pool is in host memory: only swap_blocks accepts it")
        return self.memory.device

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
    """Write key[i], value[i] ([T, Hkv, D], the pool's io dtype) into slot
    slot_mapping[i] (int64 [T]) of ``layer``."""
    torch = _torch()
    dev = pool.device
    _need(slot_mapping, "slot_mapping", torch.int64, ndim=1, device=dev)
    n = int(slot_mapping.shape[0])
    row = (n, pool.num_kv_heads, pool.head_dim)
    _need(key, "key", pool.io_dtype, row, device=dev)
    _need(value, "value", pool.io_dtype, row, device=dev)
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


def _nbytes(t) -> int:
    return 0 if t is None else int(t.numel() * t.element_size())


def _decode_call(fn_name, pool, layer, out, query, block_tables, context_lens, scale,
                 partition_size, workspace, stream):
    batch, hq, max_blocks = _check_decode_args(pool, out, query, block_tables, context_lens,
                                               workspace=workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    fn = getattr(lib(), fn_name)
    check(fn(pool.handle, int(layer), _ptr(out), _ptr(query), _ptr(block_tables), max_blocks,
             _ptr(context_lens), batch, hq, float(scale), int(partition_size), _ptr(workspace),
             _nbytes(workspace), _stream(stream)),
          fn_name)


def paged_attention_decode(pool: KVPool, layer: int, out, query, block_tables, context_lens,
                           scale=None, partition_size=0, workspace=None, stream=None):
    """out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the sequence's paged K/V."""
    if workspace is None:
        _check_decode_args(pool, out, query, block_tables, context_lens)
        workspace = alloc_workspace(pool, query.shape[0], query.shape[1], block_tables.shape[1],
                                    partition_size)
    _decode_call("paged_attention_decode", pool, layer, out, query, block_tables, context_lens,
                 scale, partition_size, workspace, stream)
    return out


def _append_call(fn_name, pool, layer, out, query, new_key, new_value, block_tables,
                 context_lens, scale, partition_size, workspace, stream):
    if new_key is None or new_value is None:
        raise ValueError(f"{fn_name}: new_key and new_value are required")
    batch, hq, max_blocks = _check_decode_args(pool, out, query, block_tables, context_lens,
                                               new_key, new_value, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    if workspace is None and fn_name == "paged_attention_decode_append":
        workspace = alloc_workspace(pool, batch, hq, max_blocks, partition_size)
    check(getattr(lib(), fn_name)(pool.handle, int(layer), _ptr(out), _ptr(query), _ptr(new_key),
                                  _ptr(new_value), _ptr(block_tables), max_blocks,
                                  _ptr(context_lens), batch, hq, float(scale), int(partition_size),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream)),
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


SCRATCH_BYTES = 64 << 20      # PAGEDKV_SCRATCH_BYTES


def paged_attention_decode_noalloc(pool: KVPool, layer: int, out, query, block_tables, context_lens,
                                   scale=None, partition_size=0, stream=None):
    """paged_attention_decode with no workspace argument and no allocation: partial
    results go to the library's per-GPU scratch array (SCRATCH_BYTES).  Shapes that
    need more are refused (KV_ERR_WORKSPACE); calls that overlap on one GPU race."""
    batch, hq, max_blocks = _check_decode_args(pool, out, query, block_tables, context_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    check(lib().paged_attention_decode_noalloc(pool.handle, int(layer), _ptr(out), _ptr(query),
                                               _ptr(block_tables), max_blocks, _ptr(context_lens),
                                               batch, hq, float(scale), int(partition_size),
                                               _stream(stream)),
          "paged_attention_decode_noalloc")
    return out


def shared_prefix_blocks(tables, lengths, block_size=BLOCK_SIZE, appending=False) -> int:
    """The largest prefix_blocks paged_attention_decode_shared_prefix accepts for these
    host tables ([B, max_blocks] int32) and lengths ([B] int32): numpy arrays or CPU
    tensors, as BlockManager.export / PrefixCache.export return them.  ``appending``: the
    step also writes each sequence's token at position L - 1, which must fall after the
    prefix."""
    import numpy as np
    t = np.ascontiguousarray(np.asarray(tables), dtype=np.int32)
    n = np.ascontiguousarray(np.asarray(lengths), dtype=np.int32)
    if t.ndim != 2 or n.ndim != 1 or n.shape[0] != t.shape[0]:
        raise ValueError(f"shared_prefix_blocks: tables {t.shape} and lengths {n.shape} do not match")
    r = int(lib().kv_shared_prefix_blocks(t.ctypes.data, n.ctypes.data, int(t.shape[0]),
                                          int(t.shape[1]), int(block_size), int(bool(appending))))
    if r < 0:
        raise ValueError("shared_prefix_blocks: invalid arguments")
    return r


def decode_order(lengths):
    """A batch order for a decode step (kv_decode_order): the indices of the host
    ``lengths`` ([B] int32, numpy or CPU tensor) by length, longest first, ties in batch
    order.  Build the step's batch in this order (queries, tables, lengths, outputs alike)."""
    import numpy as np
    n = np.ascontiguousarray(np.asarray(lengths), dtype=np.int32)
    if n.ndim != 1:
        raise ValueError(f"decode_order: lengths must be one-dimensional, not {n.shape}")
    order = np.empty(n.shape[0], dtype=np.int32)
    if int(lib().kv_decode_order(n.ctypes.data, int(n.shape[0]), order.ctypes.data)) != 0:
        raise ValueError("decode_order: invalid arguments")
    return order


def shared_prefix_workspace_bytes(pool: KVPool, batch, num_q_heads, max_blocks_per_seq,
                                  prefix_blocks, partition_size=0) -> int:
    """Workspace bytes of paged_attention_decode_shared_prefix for this shape on the
    current device."""
    n = int(lib().paged_attention_shared_prefix_workspace_bytes(
        pool.handle, int(batch), int(num_q_heads), int(max_blocks_per_seq), int(prefix_blocks),
        int(partition_size)))
    if n == (1 << 64) - 1:
        raise ValueError("shared_prefix_workspace_bytes: invalid arguments")
    return n


def alloc_shared_prefix_workspace(pool: KVPool, batch, num_q_heads, max_blocks_per_seq,
                                  prefix_blocks, partition_size=0):
    torch = _torch()
    n = shared_prefix_workspace_bytes(pool, batch, num_q_heads, max_blocks_per_seq, prefix_blocks,
                                      partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=pool.device)


def _shared_prefix_args(pool, layer, out, query, block_tables, context_lens, prefix_blocks,
                        new_key, new_value, scale, partition_size, workspace):
    """The checked argument list of paged_attention_decode_shared_prefix (no stream)."""
    if (new_key is None) != (new_value is None):
        raise ValueError("paged_attention_decode_shared_prefix: give both new_key and new_value, or neither")
    batch, hq, max_blocks = _check_decode_args(pool, out, query, block_tables, context_lens,
                                               new_key, new_value, workspace)
    prefix_blocks = int(prefix_blocks)
    if not 0 <= prefix_blocks <= max_blocks:
        raise ValueError(f"prefix_blocks: {prefix_blocks} is outside [0, {max_blocks}]")
    if workspace is None:
        workspace = alloc_shared_prefix_workspace(pool, batch, hq, max_blocks, prefix_blocks,
                                                  partition_size)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    vp = ctypes.c_void_p
    args = [pool.handle, ctypes.c_int32(int(layer)), vp(_ptr(out)), vp(_ptr(query)),
            vp(_ptr(new_key)), vp(_ptr(new_value)), vp(_ptr(block_tables)),
            ctypes.c_int32(max_blocks), vp(_ptr(context_lens)), ctypes.c_int32(batch),
            ctypes.c_int32(hq), ctypes.c_float(float(scale)), ctypes.c_int32(prefix_blocks),
            ctypes.c_int32(int(partition_size)), vp(_ptr(workspace)),
            ctypes.c_size_t(_nbytes(workspace))]
    return args, workspace


def paged_attention_decode_shared_prefix(pool: KVPool, layer: int, out, query, block_tables,
                                         context_lens, prefix_blocks, new_key=None, new_value=None,
                                         scale=None, partition_size=0, workspace=None, stream=None):
    """paged_attention_decode(_append) for a batch whose table rows all begin with the
    same ``prefix_blocks`` entries (row 0's): the shared keys are read once for the batch.
    With ``new_key`` / ``new_value`` the new tokens are written first, as in
    paged_attention_decode_append; they must fall after the prefix."""
    args, _ = _shared_prefix_args(pool, layer, out, query, block_tables, context_lens,
                                  prefix_blocks, new_key, new_value, scale, partition_size,
                                  workspace)
    check(lib().paged_attention_decode_shared_prefix(*args, _stream(stream)),
          "paged_attention_decode_shared_prefix")
    return out


class DecodeStep:
    """One decode step prepared once for buffers a serving loop reuses: the tensors are
    checked when the step is built, and each call is then a single call into the library
    with the arguments already converted.  ``step()`` runs the whole step
    (paged_attention_decode_append when new keys / values are given, else
    paged_attention_decode); ``step.partitions()`` and ``step.reduce()`` run its two
    phases (paged_attention_partitions[_append], paged_attention_reduce) for callers that
    time or schedule them separately.

    The step keeps the tensors' addresses, so the tensors must stay alive and keep their
    storage (update their contents in place between calls).  Lengths and tables are read
    on the device at each call, so they may change, within the shapes given here.
    ``stream`` (a torch stream or a raw handle) fixes the stream; without it each call
    uses torch's current stream.

    ``prefix_blocks`` > 0: the rows of ``block_tables`` share their first prefix_blocks
    entries, and each call is paged_attention_decode_shared_prefix (a single phase:
    ``partitions()`` / ``reduce()`` are not available)."""

    def __init__(self, pool: KVPool, layer: int, out, query, block_tables, context_lens,
                 new_key=None, new_value=None, scale=None, partition_size=0, workspace=None,
                 stream=None, prefix_blocks=0):
        if (new_key is None) != (new_value is None):
            raise ValueError("DecodeStep: give both new_key and new_value, or neither")
        self._stream = None if stream is None else ctypes.c_void_p(_stream(stream))
        self.out = out
        if int(prefix_blocks) > 0:
            args, workspace = _shared_prefix_args(pool, layer, out, query, block_tables,
                                                  context_lens, prefix_blocks, new_key, new_value,
                                                  scale, partition_size, workspace)
            self._keep = (pool, out, query, block_tables, context_lens, new_key, new_value, workspace)
            self._whole = ("paged_attention_decode_shared_prefix",
                           lib().paged_attention_decode_shared_prefix, args)
            self._first = self._second = None
            return
        batch, hq, max_blocks = _check_decode_args(pool, out, query, block_tables, context_lens,
                                                   new_key, new_value, workspace)
        if workspace is None:
            workspace = alloc_workspace(pool, batch, hq, max_blocks, partition_size)
        if scale is None:
            scale = 1.0 / math.sqrt(pool.head_dim)
        # keep every buffer alive as long as the step
        self._keep = (pool, out, query, block_tables, context_lens, new_key, new_value, workspace)
        vp = ctypes.c_void_p
        head = [pool.handle, ctypes.c_int32(int(layer)), vp(_ptr(out)), vp(_ptr(query))]
        tail = [vp(_ptr(block_tables)), ctypes.c_int32(max_blocks), vp(_ptr(context_lens)),
                ctypes.c_int32(batch), ctypes.c_int32(hq), ctypes.c_float(float(scale)),
                ctypes.c_int32(int(partition_size)), vp(_ptr(workspace)),
                ctypes.c_size_t(_nbytes(workspace))]
        L = lib()
        if new_key is not None:
            rows = [vp(_ptr(new_key)), vp(_ptr(new_value))]
            self._whole = ("paged_attention_decode_append", L.paged_attention_decode_append, head + rows + tail)
            self._first = ("paged_attention_partitions_append", L.paged_attention_partitions_append,
                           head + rows + tail)
        else:
            self._whole = ("paged_attention_decode", L.paged_attention_decode, head + tail)
            self._first = ("paged_attention_partitions", L.paged_attention_partitions, head + tail)
        self._second = ("paged_attention_reduce", L.paged_attention_reduce, head + tail)

    def _run(self, call, stream):
        if call is None:
            raise ValueError("DecodeStep: a shared-prefix step runs as one call")
        name, fn, args = call
        st = fn(*args, self._stream if stream is None and self._stream is not None else _stream(stream))
        if st:
            check(st, name)

    def __call__(self, stream=None):
        self._run(self._whole, stream)
        return self.out

    def partitions(self, stream=None):
        self._run(self._first, stream)

    def reduce(self, stream=None):
        self._run(self._second, stream)


def _check_prefill_args(pool, out, query, query_start, block_tables, context_lens):
    torch = _torch()
    dev = pool.device
    _need(query, "query", pool.io_dtype, ndim=3, device=dev)
    tokens, hq, d = (int(x) for x in query.shape)
    if d != pool.head_dim:
        raise ValueError(f"query: head size {d} differs from the pool's {pool.head_dim}")
    if hq < 1 or hq % pool.num_kv_heads:
        raise ValueError(f"query: {hq} heads is not a multiple of the pool's {pool.num_kv_heads} KV heads")
    _need(out, "out", pool.io_dtype, (tokens, hq, d), device=dev)
    _need(context_lens, "context_lens", torch.int32, ndim=1, device=dev)
    batch = int(context_lens.shape[0])
    _need(query_start, "query_start", torch.int32, (batch + 1,), device=dev)
    _need(block_tables, "block_tables", torch.int32, (batch, None), device=dev)
    return batch, tokens, hq


def paged_attention_prefill(pool: KVPool, layer: int, out, query, query_start, max_query_len,
                            block_tables, context_lens, scale=None, stream=None) -> None:
    """Causal attention of each sequence's chunk of new tokens (rows
    [query_start[b], query_start[b+1]) of ``query``) over its paged K/V.  ``query_start``
    must end at no more than the rows of ``query`` (it is read on the device)."""
    batch, _, hq = _check_prefill_args(pool, out, query, query_start, block_tables, context_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    check(lib().paged_attention_prefill(pool.handle, int(layer), _ptr(out), _ptr(query),
                                        _ptr(query_start), int(max_query_len), _ptr(block_tables),
                                        int(block_tables.shape[1]), _ptr(context_lens), batch,
                                        hq, float(scale), _stream(stream)),
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
    batch, num_tokens, hq = _check_prefill_args(pool, out, query, query_start, block_tables,
                                                context_lens)
    _need_bytes(workspace, "workspace", pool.device)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.head_dim)
    check(lib().paged_attention_prefill_split(pool.handle, int(layer), _ptr(out), _ptr(query),
                                              _ptr(query_start), int(max_query_len), num_tokens,
                                              _ptr(block_tables), int(block_tables.shape[1]),
                                              _ptr(context_lens), batch, hq,
                                              float(scale), _ptr(workspace), _nbytes(workspace),
                                              _stream(stream)),
          "paged_attention_prefill_split")


def kv_pool_gather(pool: KVPool, layer: int, block_tables, context_lens, k_out, v_out,
                   stream=None) -> None:
    """Test hook: k_out / v_out [B, max_blocks * block_size, Hkv, D] in the pool's storage
    type receive each sequence's rows through its table (zeros past its length)."""
    torch = _torch()
    dev = pool.device
    _need(context_lens, "context_lens", torch.int32, ndim=1, device=dev)
    batch = int(context_lens.shape[0])
    _need(block_tables, "block_tables", torch.int32, (batch, None), device=dev)
    rows = (batch, int(block_tables.shape[1]) * pool.block_size, pool.num_kv_heads, pool.head_dim)
    _need(k_out, "k_out", pool.dtype, rows, device=dev)
    _need(v_out, "v_out", pool.dtype, rows, device=dev)
    check(lib().kv_pool_gather(pool.handle, int(layer), _ptr(block_tables),
                               int(block_tables.shape[1]), _ptr(context_lens), batch, _ptr(k_out),
                               _ptr(v_out), _stream(stream)),
          "kv_pool_gather")


from .block_manager import BlockManager, OutOfBlocks, copy_blocks, swap_blocks  # noqa: E402
from .prefix_cache import PrefixCache, hash_block  # noqa: E402
