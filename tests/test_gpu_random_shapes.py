"""Seeded random shapes through the decode step (cache write folded in) and the
shared-prefix step, each against the CPU oracle to the flat bar per element, with the
pool's bytes after the write equal to the oracle's scatter.

Each case draws, from its own seed: KV heads and the GQA group (1-16), head size (64,
128), the query type (fp16, bf16) and storage (16-bit or FP8), the block size (8-64),
the partition size (a power of two from the block size to 2,048 tokens), the batch and
U[1, N] lengths (N from 1 to 3,000), and a layer of a 1-3 layer pool (the other
layers NaN), so that plan boundaries (one partition or several,
split, item and group plans, the matrix-core and VALU kernels) fall where they may.  The
fork cases draw a prefix of 1-1,500 tokens and private suffixes of U[1, 1-1,200] tokens
(fused or with the reduce, as the table width decides)."""

import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import paged_kv_cache_68_amd as pk  # noqa: E402
from workloads import make_case  # noqa: E402
from workloads.configs import DecodeConfig  # noqa: E402

from .gpu_helpers import DeviceCase, flat_bar, oracle_after_write, to_host_bits  # noqa: E402


# PAGEDKV_TEST_RANDOM_CASES=n widens both sweeps (default 24 decode and 12 fork cases)
_N = int(os.environ.get("PAGEDKV_TEST_RANDOM_CASES", "0"))


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _draw(seed, fork):
    rng = np.random.default_rng(90_000 + seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([g for g in (1, 2, 3, 4, 5, 6, 7, 8, 12, 16) if g * hkv <= 64]))
    d = int(rng.choice([64, 128]))
    io = str(rng.choice(["f16", "bf16"]))
    kv = "fp8" if rng.random() < 0.3 else ""
    bs = int(rng.choice([8, 16, 32, 64]))
    part = int(rng.choice([p for p in (8, 16, 32, 64, 128, 256, 512, 1024, 2048) if p >= bs]))
    batch = int(rng.integers(1, 13))
    if fork:
        prefix = int(rng.integers(1, 1501))
        smax = int(rng.integers(1, 1201))
        lengths = f"fork_{prefix}_{smax}"
        nb = batch * (-(-(prefix + smax) // bs) + 2) + 64
    else:
        nmax = int(rng.choice([1, 15, 100, 700, 3000]))
        lengths = f"uniform_{nmax}"
        nb = batch * (-(-nmax // bs)) + 16
    layers = int(rng.integers(1, 4))
    layer = int(rng.integers(0, layers))
    return layers, layer, DecodeConfig(index=5000 + seed + (500 if fork else 0), name=f"rand{seed}_{lengths}",
                        num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=d, dtype=io,
                        block_size=bs, num_blocks=nb, batch=batch, lengths=lengths,
                        partition_size=part, description="random shape", kv_dtype=kv)


def _check(out_bits, ref, cfg, what):
    got = oracle.to_f64(out_bits, cfg.dtype)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    _say(f"{what}: max abs err {err.max():.3e}")
    assert np.all(err <= flat_bar(ref, cfg.dtype)), what


def _desc(cfg, layers, layer):
    return (f"{cfg.name}: {cfg.num_q_heads}/{cfg.num_kv_heads} x {cfg.head_dim} {cfg.dtype}"
            f"{'/fp8' if cfg.kv_dtype else ''} B{cfg.block_size} P{cfg.partition_size} batch {cfg.batch}"
            f" layer {layer} of {layers}")


@pytest.mark.parametrize("seed", range(_N or 24))
def test_random_decode_shapes(seed):
    layers, layer, cfg = _draw(seed, fork=False)
    _say(_desc(cfg, layers, layer))
    case = make_case(cfg)
    dc = DeviceCase(case, num_layers=layers, layer=layer)
    out = to_host_bits(dc.step_append())
    ref, kp, vp = oracle_after_write(case)
    _check(out, ref, cfg, cfg.name)
    assert np.array_equal(to_host_bits(dc.pool.k_cache(layer)), kp)
    assert np.array_equal(to_host_bits(dc.pool.v_cache(layer)), vp)


@pytest.mark.parametrize("seed", range(_N or 12))
def test_random_fork_shapes(seed):
    layers, layer, cfg = _draw(seed, fork=True)
    _say(_desc(cfg, layers, layer))
    case = make_case(cfg)
    P = len(case.shared_blocks)
    # (a single sequence shares any number of its own blocks: the generator's prefix is one;
    # a prefix shorter than one block shares none, and the call is then the plain step)
    assert 0 <= P <= pk.shared_prefix_blocks(case.block_tables, case.lengths, cfg.block_size,
                                            appending=True)
    dc = DeviceCase(case, num_layers=layers, layer=layer)
    n = pk.shared_prefix_workspace_bytes(dc.pool, cfg.batch, cfg.num_q_heads,
                                         dc.tables.shape[1], P, cfg.partition_size)
    ws = torch.full((max(n, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dc.query)
    pk.paged_attention_decode_shared_prefix(dc.pool, layer, out, dc.query, dc.tables, dc.lens, P,
                                            new_key=dc.new_key, new_value=dc.new_value,
                                            scale=cfg.scale, partition_size=cfg.partition_size,
                                            workspace=ws)
    ref, kp, vp = oracle_after_write(case)
    _check(to_host_bits(out), ref, cfg, f"{cfg.name} prefix {P} blocks")
    assert np.array_equal(to_host_bits(dc.pool.k_cache(layer)), kp)
    assert np.array_equal(to_host_bits(dc.pool.v_cache(layer)), vp)
