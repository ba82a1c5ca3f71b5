"""Oracle-side helpers of the GPU tests: the oracle's answer for a case, for chosen
sequences, and the error measure."""

from __future__ import annotations

import numpy as np

import oracle
from workloads import DecodeCase

from .device_case import DeviceCase, TORCH_DT, to_dev, to_host_bits  # noqa: F401

TOL = {"f16": 2e-3, "bf16": 8e-3}


def oracle_after_write(case: DecodeCase):
    """Host oracle for a host case: scatter the new tokens, then decode every sequence."""
    cfg = case.cfg
    kp = case.k_pool.copy()
    vp = case.v_pool.copy()
    key, value = case.new_key, case.new_value
    if cfg.kv == "fp8":               # the cache write of an FP8 pool rounds to E4M3
        key, value = oracle.quantize_fp8(key, cfg.dtype), oracle.quantize_fp8(value, cfg.dtype)
    oracle.scatter(kp, vp, key, value, case.slot_mapping, cfg.block_size)
    ref = oracle.paged_decode(case.query, kp, vp, case.block_tables, case.lengths, cfg.scale,
                              cfg.block_size, cfg.kv, q_dtype=cfg.dtype)
    return ref, kp, vp


def oracle_for_seqs(dc: DeviceCase, seqs):
    """Oracle outputs for the listed sequences, from the bytes the GPU holds (after the write)."""
    cfg = dc.cfg
    out = []
    for b in seqs:
        kb, vb, table = dc.blocks_of(b)
        out.append(oracle.paged_decode_seq(dc.case.query[b], kb, vb, table,
                                           int(dc.case.lengths[b]), cfg.scale, cfg.block_size,
                                           cfg.kv, q_dtype=cfg.dtype))
    return np.stack(out)


SIG = {"bf16": 8, "f16": 11}      # significand bits of each io type


def flat_bar(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per element: the max-abs bar TOL, except where rounding the exact value to the io
    type by itself costs more (half an ulp of |ref|: bf16 at |o| >= 4, fp16 at |o| >= 8),
    there that half ulp plus an eighth of the bar."""
    _, e = np.frexp(np.abs(ref))
    half_ulp = np.ldexp(1.0, e - 1 - SIG[dtype])
    return np.where(half_ulp < TOL[dtype], TOL[dtype], half_ulp + TOL[dtype] / 8)


def max_abs_err(gpu_bits: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    got = oracle.to_f64(gpu_bits, dtype)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)))


def relabelled(dc: DeviceCase, seed: int):
    """A copy of the pool with block p moved to pi(p), and the matching tables."""
    import torch

    import paged_kv_cache_68_amd as pk
    cfg = dc.cfg
    nb = cfg.num_blocks
    pi = torch.randperm(nb, generator=torch.Generator().manual_seed(seed)).cuda()
    inv = torch.argsort(pi)
    pool2 = pk.KVPool(1, nb, cfg.num_kv_heads, cfg.head_dim, cfg.kv, block_size=cfg.block_size,
                      io_dtype=cfg.dtype)
    for which in ("k_cache", "v_cache"):
        torch.index_select(getattr(dc.pool, which)(0), 0, inv, out=getattr(pool2, which)(0))
    t = dc.tables
    tables2 = torch.where(t >= 0, pi[t.clamp(min=0).long()].to(torch.int32), t).contiguous()
    return pool2, tables2, pi
