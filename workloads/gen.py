"""Seeded construction of one decode step's inputs.

A decode step (as in "Why AI servers waste memory, and how paging fixes it",
"The real implementation": write the new token into its slot, then read through the
table) is described here by:

* ``lengths[b]``      context length of sequence b *including* the new token;
* ``block_tables``    int32 [B, max_blocks]; entry j is the physical block holding
                      logical block j; entries past ceil(L/16) are -1;
* ``slot_mapping``    int64 [B]; physical slot (block * block_size + offset) that
                      receives the new token, i.e. position L-1 of the sequence;
* ``query``           [B, Hq, d]; ``new_key`` / ``new_value`` [B, Hkv, d];
* ``k_pool``/``v_pool`` [num_blocks, block_size, Hkv, d] holding positions < L-1.

16-bit values are kept as uint16 bit patterns on the host so that fp16 and bf16 can
be handled the same way and compared bit for bit.  Values are i.i.d. N(0, 1) drawn in
fp32 and rounded to the storage type with round-to-nearest-even.  FP8 (E4M3) pools hold
uint8 codes, drawn the same way and rounded by torch's float8_e4m3fn conversion.

Slots nobody may read (unused blocks, positions >= L-1 of a last block) can be
poisoned with NaN, so a reader that touches them shows up as NaN in its output.
"""

from __future__ import annotations

import math
from collections import deque
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .configs import DecodeConfig

# lognormal spread: mean 260 / median 180 of the length mix described in
# "PagedAttention: Treating KV Memory Like Virtual Memory" (tail-waste simulation)
LOGNORMAL_SIGMA = math.sqrt(2.0 * math.log(260.0 / 180.0))
SHARED_PREFIX_TOKENS = 4096 + 7   # 256 full blocks + a 7-token partial block
SHARED_FORKS = 64


def bits_dtype_name(dtype: str) -> str:
    return {"f16": "float16", "bf16": "bfloat16"}[dtype]


def nan_bits(dtype: str) -> int:
    return {"f16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}[dtype]


def _np_storage(dtype: str):
    return np.uint8 if dtype == "fp8" else np.uint16


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array -> uint16 bit patterns of fp16 / bf16, round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # finite inputs only (normal samples): no overflow in uint32
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return r.astype(np.uint16)
    raise ValueError(dtype)


@dataclass
class DecodeCase:
    cfg: DecodeConfig
    lengths: np.ndarray
    block_tables: np.ndarray
    slot_mapping: np.ndarray
    query: np.ndarray
    new_key: np.ndarray
    new_value: np.ndarray
    k_pool: object            # np.uint16 array (host) or torch tensor (device)
    v_pool: object
    where: str                # "host" or "device"
    used_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    shared_blocks: Optional[np.ndarray] = None
    refcounts: Optional[np.ndarray] = None
    cow_copies: list = field(default_factory=list)

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])


def draw_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.lengths == "fixed_1_16_17_40":
        lens = np.array([1, 16, 17, 40], dtype=np.int64)
    elif cfg.lengths == "lognormal_200":
        raw = rng.lognormal(mean=math.log(200.0), sigma=LOGNORMAL_SIGMA, size=cfg.batch)
        lens = np.clip(np.rint(raw), 1, 2048).astype(np.int64)
    elif cfg.lengths == "const_8192":
        lens = np.full(cfg.batch, 8192, dtype=np.int64)
    elif cfg.lengths == "uniform_4096":
        lens = rng.integers(1, 4096, size=cfg.batch, endpoint=True).astype(np.int64)
    elif cfg.lengths.startswith("uniform_"):          # "uniform_<N>": U[1, N]
        lens = rng.integers(1, int(cfg.lengths.split("_")[1]), size=cfg.batch,
                            endpoint=True).astype(np.int64)
    else:
        raise ValueError(cfg.lengths)
    assert lens.shape == (cfg.batch,)
    return lens.astype(np.int32)


def _blocks_for(n_tokens: int, bs: int) -> int:
    return -(-int(n_tokens) // bs)


def _scattered_tables(cfg, lens, rng):
    """Each sequence takes ceil(L/bs) blocks, in order, from a seeded permutation."""
    bs = cfg.block_size
    need = np.array([_blocks_for(L, bs) for L in lens], dtype=np.int64)
    if need.sum() > cfg.num_blocks:
        raise ValueError("pool too small for the drawn lengths")
    perm = rng.permutation(cfg.num_blocks)
    width = int(need.max())
    tables = np.full((cfg.batch, width), -1, dtype=np.int32)
    pos = 0
    for b in range(cfg.batch):
        tables[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    return tables, perm[:pos].astype(np.int64)


def _slots_of_new_tokens(lens, tables, bs):
    pos = lens.astype(np.int64) - 1
    return (tables[np.arange(len(lens)), pos // bs].astype(np.int64) * bs + pos % bs)


def _stale_mask(cfg, lens, tables):
    """Positions >= L-1 inside each sequence's last block (before the write)."""
    out = []
    bs = cfg.block_size
    for b, L in enumerate(lens):
        last = int(tables[b, (int(L) - 1) // bs])
        for o in range((int(L) - 1) % bs, bs):
            out.append((last, o))
    return out


def _host_values(shape, rng, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "fp8":
        import torch  # E4M3 rounding of the drawn values (input data only)
        return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return round_to_bits(x, dtype)


def _make_scattered_host(cfg, rng, lens, poison):
    bs, H, d = cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    tables, used = _scattered_tables(cfg, lens, rng)
    fill = nan_bits(cfg.kv) if poison else 0
    pools = []
    for _ in range(2):   # K then V
        pool = np.full((cfg.num_blocks, bs, H, d), fill, dtype=_np_storage(cfg.kv))
        pool[used] = _host_values((len(used), bs, H, d), rng, cfg.kv)
        pools.append(pool)
    return tables, used, pools


def fork_shape(cfg: DecodeConfig):
    """(prefix tokens, forks, largest private suffix) of a forked-batch config:
    "shared_prefix" is 64 forks of 4,103 tokens with U[1, 512] more each;
    "fork_<P>_<S>" is cfg.batch forks of P tokens with U[1, S] more each."""
    if cfg.lengths == "shared_prefix":
        return SHARED_PREFIX_TOKENS, SHARED_FORKS, 512
    _, p, s = cfg.lengths.split("_")
    return int(p), cfg.batch, int(s)


def is_fork(cfg: DecodeConfig) -> bool:
    return cfg.lengths == "shared_prefix" or cfg.lengths.startswith("fork_")


def _make_shared_prefix_host(cfg, rng, poison):
    """Fork 64 ways from a 4,103-token prefix (or as fork_shape says), copy-on-write the
    shared partial block.

    Follows the append rule of "Why AI servers waste memory, and how paging fixes
    it" ("Sharing a prefix with copy-on-write"): a fork copies the table and raises
    every named block's count; a write into a shared block that still has room first
    copies the whole block into a new one; a full shared block is never written.
    """
    bs, H, d = cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    nb = cfg.num_blocks
    fill = nan_bits(cfg.kv) if poison else 0
    kp = np.full((nb, bs, H, d), fill, dtype=_np_storage(cfg.kv))
    vp = np.full((nb, bs, H, d), fill, dtype=_np_storage(cfg.kv))
    free = deque(int(x) for x in rng.permutation(nb))
    ref = np.zeros(nb, dtype=np.int64)

    n_tokens, forks, suffix_max = fork_shape(cfg)
    n_prefix_blocks = _blocks_for(n_tokens, bs)
    prefix = [free.popleft() for _ in range(n_prefix_blocks)]
    ref[prefix] = 1
    # prefix tokens (the parent's prompt)
    for j, blk in enumerate(prefix):
        n_valid = min(bs, n_tokens - j * bs)
        kp[blk, :n_valid] = _host_values((n_valid, H, d), rng, cfg.kv)
        vp[blk, :n_valid] = _host_values((n_valid, H, d), rng, cfg.kv)
    # fork: every child copies the parent's table; counts rise by forks-1
    tables = [list(prefix) for _ in range(forks)]
    ref[prefix] += forks - 1
    suffix = rng.integers(1, suffix_max, size=forks, endpoint=True)
    lens = n_tokens + suffix
    copies = []
    for b in range(forks):
        n = n_tokens
        last = tables[b][-1]
        if n % bs != 0 and ref[last] > 1:        # shared block with room -> private copy
            new = free.popleft()
            kp[new] = kp[last]
            vp[new] = vp[last]
            ref[last] -= 1
            ref[new] = 1
            tables[b][-1] = new
            copies.append((last, new))
        # private suffix: positions n .. L-2 are history, L-1 is the new token
        L = int(lens[b])
        for t in range(n, L):
            j, o = divmod(t, bs)
            if j == len(tables[b]):
                blk = free.popleft()
                ref[blk] = 1
                tables[b].append(blk)
            if t < L - 1:
                blk = tables[b][j]
                kp[blk, o] = _host_values((H, d), rng, cfg.kv)
                vp[blk, o] = _host_values((H, d), rng, cfg.kv)
    width = max(len(t) for t in tables)
    tab = np.full((forks, width), -1, dtype=np.int32)
    for b, t in enumerate(tables):
        tab[b, :len(t)] = t
    used = np.array(sorted({x for t in tables for x in t}), dtype=np.int64)
    return (lens.astype(np.int32), tab, used, [kp, vp], np.array(prefix[:n_tokens // bs], dtype=np.int64),
            ref, copies)


def make_case(cfg: DecodeConfig, where: str = "host", poison: bool = True,
              device=None, batch: Optional[int] = None) -> DecodeCase:
    """Build one decode step of ``cfg``.

    ``where="host"``: pools are numpy uint16 bit arrays.  ``where="device"``: pools
    are torch tensors on ``device`` filled by a torch generator seeded with the
    config index (used where a host copy of the pool would be too large).
    ``batch`` truncates the batch (same seed, first sequences only) for quick tests.
    """
    rng = np.random.default_rng(cfg.index)
    bs, H, d, Hq = cfg.block_size, cfg.num_kv_heads, cfg.head_dim, cfg.num_q_heads
    shared = ref = None
    copies = []
    if is_fork(cfg):
        if where != "host":
            raise ValueError("the shared-prefix case is built on the host")
        lens, tables, used, pools, shared, ref, copies = _make_shared_prefix_host(cfg, rng, poison)
    else:
        lens = draw_lengths(cfg, rng)
        if where == "host":
            tables, used, pools = _make_scattered_host(cfg, rng, lens, poison)
        else:
            tables, used = _scattered_tables(cfg, lens, rng)
            pools = None
    query = _host_values((cfg.batch, Hq, d), rng, cfg.dtype)
    new_k = _host_values((cfg.batch, H, d), rng, cfg.dtype)
    new_v = _host_values((cfg.batch, H, d), rng, cfg.dtype)
    slots = _slots_of_new_tokens(lens, tables, bs)

    if where == "host":
        kp, vp = pools
        if poison:
            for blk, o in _stale_mask(cfg, lens, tables):
                kp[blk, o] = nan_bits(cfg.kv)
                vp[blk, o] = nan_bits(cfg.kv)
    else:
        kp, vp = _device_pools(cfg, lens, tables, used, poison, device)

    case = DecodeCase(cfg=cfg, lengths=lens, block_tables=tables, slot_mapping=slots,
                      query=query, new_key=new_k, new_value=new_v, k_pool=kp, v_pool=vp,
                      where=where, used_blocks=used, shared_blocks=shared, refcounts=ref,
                      cow_copies=copies)
    if batch is not None and batch < cfg.batch:
        case = truncate(case, batch)
    return case


def truncate(case: DecodeCase, batch: int) -> DecodeCase:
    lens = case.lengths[:batch]
    width = max(1, _blocks_for(int(lens.max()), case.cfg.block_size))
    return DecodeCase(cfg=case.cfg, lengths=lens.copy(),
                      block_tables=case.block_tables[:batch, :width].copy(),
                      slot_mapping=case.slot_mapping[:batch].copy(),
                      query=case.query[:batch].copy(), new_key=case.new_key[:batch].copy(),
                      new_value=case.new_value[:batch].copy(), k_pool=case.k_pool,
                      v_pool=case.v_pool, where=case.where, used_blocks=case.used_blocks,
                      shared_blocks=case.shared_blocks, refcounts=case.refcounts,
                      cow_copies=case.cow_copies)


def _device_pools(cfg, lens, tables, used, poison, device):
    import torch  # device inputs only

    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[cfg.kv]
    bs, H, d = cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    dev = torch.device(device if device is not None else "cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.index)
    pools = []
    chunk = max(1, (1 << 27) // (bs * H * d))   # ~128M elements per draw
    # K and V share one allocation (K first) so a one-layer pool can adopt it as is
    both = torch.empty((2, cfg.num_blocks, bs, H, d), dtype=tdt, device=dev)
    for which in range(2):
        pool = both[which]
        for s in range(0, cfg.num_blocks, chunk):
            e = min(cfg.num_blocks, s + chunk)
            pool[s:e] = torch.randn((e - s, bs, H, d), generator=gen, device=dev,
                                    dtype=torch.float32).to(tdt)
        pools.append(pool)
    if poison:
        mask = torch.ones(cfg.num_blocks, dtype=torch.bool, device=dev)
        mask[torch.as_tensor(used, device=dev)] = False
        idx = torch.nonzero(mask).flatten()
        stale = _stale_mask(cfg, lens, tables)
        sb = torch.as_tensor([s[0] for s in stale], device=dev, dtype=torch.long)
        so = torch.as_tensor([s[1] for s in stale], device=dev, dtype=torch.long)
        for pool in pools:
            # NaN bit patterns written through an integer view of the storage
            ints = pool.view(torch.uint8) if cfg.kv == "fp8" else pool.view(torch.int16)
            nan = nan_bits(cfg.kv)              # < 0x8000: fits the int16 view as is
            if idx.numel():
                ints.index_fill_(0, idx, nan)
            ints[sb, so] = nan
    return pools[0], pools[1]
