"""Bit-identity under a relabelling of physical blocks, on the launch plans that produce
the measured numbers.

A block's physical place carries no meaning: relabel every block by a permutation pi
(block p's contents move to block pi(p), every table entry t becomes pi(t)) and the
attention output must be the same bits ("Why AI servers waste memory, and how paging
fixes it", "The idea: a block table": position p is found through table[p // B] alone).
Each case runs the decode step bench.py times (the partition kernel with the cache write
folded in, then the reduce) and plain decode, on the original pool and on a relabelled
copy made on the device, at the workload's full size, so that the plan each workload
takes is the one checked: the streamed 4-head group plan with chunk partials and the
reduce kernel (64 x 8,192 tokens), the single-head group plan (512 MHA sequences), the
split plan (the 256-sequence serving batch), paired 8-token tiles, FP8 widening, the
cache-served plan of the shared-prefix batch, and the item plan and VALU kernel forced
by their switches.  The step also runs twice on the same pool: the same bits again.

Also here: full-size oracle checks (sampled sequences) of the two variant workloads
whose rates are reported, FP8 keys / values on the 512-sequence MHA batch and 8-token
blocks on the 64 x 8,192 batch, in the launch configuration bench.py uses.
"""

import dataclasses

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import paged_kv_cache_68_amd as pk  # noqa: E402
from workloads import config_by_name, make_case  # noqa: E402

from .gpu_helpers import (  # noqa: E402
    TOL, DeviceCase, max_abs_err, oracle_for_seqs, relabelled as _relabelled, to_host_bits,
)


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def bench_variant(idx, block_size=None, kv=None):
    """The workload as bench.py builds it for --config / --block-size / --kv-dtype."""
    cfg = config_by_name(idx)
    if block_size and block_size != cfg.block_size:
        cfg = dataclasses.replace(cfg, block_size=block_size,
                                  num_blocks=cfg.num_blocks * cfg.block_size // block_size,
                                  name=f"{cfg.name}_b{block_size}")
    if kv:
        cfg = dataclasses.replace(cfg, kv_dtype=kv, name=f"{cfg.name}_{kv}kv")
    return cfg


def _device_case(cfg):
    where = "device" if cfg.index in (3, 5) else "host"
    return DeviceCase(make_case(cfg, where=where, poison=where == "host"))


def _step(pool, dc, tables, out):
    """The launches bench.py times: partitions with the cache write folded in, then reduce."""
    cfg = dc.cfg
    pk.paged_attention_partitions_append(pool, 0, out, dc.query, dc.new_key, dc.new_value, tables,
                                         dc.lens, cfg.scale, cfg.partition_size, dc.workspace)
    pk.paged_attention_reduce(pool, 0, out, dc.query, tables, dc.lens, cfg.scale,
                              cfg.partition_size, dc.workspace)
    return to_host_bits(out)


def _decode(pool, dc, tables, out):
    cfg = dc.cfg
    pk.paged_attention_decode(pool, 0, out, dc.query, tables, dc.lens, cfg.scale,
                              cfg.partition_size, dc.workspace)
    return to_host_bits(out)


CASES = [
    ("c3", 3, None, None, {}),
    ("c3_no_stream_hint", 3, None, None, {"PAGEDKV_STREAM": "0"}),
    ("c3_b8_paired", 3, 8, None, {}),
    ("c3_fp8", 3, None, "fp8", {}),
    ("c5_g1", 5, None, None, {}),
    ("c5_g1_batch_order", 5, None, None, {"PAGEDKV_ORDER": "0"}),
    ("c5_fp8", 5, None, "fp8", {}),
    ("c2_split", 2, None, None, {}),
    ("c4_shared_prefix", 4, None, None, {}),
    ("c2_item", 2, None, None, {"PAGEDKV_SPLIT": "0", "PAGEDKV_GROUP": "0"}),
    ("c2_valu", 2, None, None, {"PAGEDKV_KERNEL": "valu"}),
    ("c3_valu", 3, None, None, {"PAGEDKV_KERNEL": "valu"}),
]


@pytest.mark.parametrize("name,idx,bs,kv,env", CASES, ids=[c[0] for c in CASES])
def test_relabelled_blocks_give_identical_bits(monkeypatch, name, idx, bs, kv, env):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    cfg = bench_variant(idx, bs, kv)
    _say(f"relabel {name}: {cfg.name} {env}")
    dc = _device_case(cfg)
    pool2, tables2, pi = _relabelled(dc, seed=1000 + idx)
    out = torch.empty_like(dc.query)
    first = _step(dc.pool, dc, dc.tables, out)
    again = _step(dc.pool, dc, dc.tables, out)
    moved = _step(pool2, dc, tables2, out)
    assert np.all(np.isfinite(oracle.to_f64(first, cfg.dtype)))
    assert np.array_equal(first, again), "step not deterministic"
    assert np.array_equal(first, moved), "relabelled blocks changed the output"
    # the new tokens landed in the same logical slots of both pools
    B = cfg.block_size
    L = dc.lens.long()
    j = ((L - 1) // B).clamp(min=0)
    o = ((L - 1) % B).clamp(min=0)
    blk = dc.tables.long().gather(1, j[:, None])[:, 0]
    for which in ("k_cache", "v_cache"):
        a = getattr(dc.pool, which)(0)[blk, o]
        b = getattr(pool2, which)(0)[pi[blk], o]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    # plain decode (no write) on both pools
    d1 = _decode(dc.pool, dc, dc.tables, out)
    d2 = _decode(pool2, dc, tables2, out)
    assert np.array_equal(d1, d2)
    assert np.array_equal(d1, first)
    del pool2, dc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("idx,bs,kv", [(5, None, "fp8"), (3, 8, None)], ids=["c5_fp8", "c3_b8"])
def test_reported_variants_full_size_against_the_oracle(idx, bs, kv):
    cfg = bench_variant(idx, bs, kv)
    dc = _device_case(cfg)
    lens = dc.case.lengths
    order = np.argsort(lens, kind="stable")
    if cfg.batch <= 64:                         # the 64 x 8,192 batch: every sequence
        seqs = list(range(cfg.batch))
    else:                                       # shortest, longest and every 8th by length
        seqs = sorted({int(order[0]), int(order[-1]), *[int(x) for x in order[::8]]})
    _say(f"full size {cfg.name}: oracle on sequences {seqs}")
    out = _step(dc.pool, dc, dc.tables, torch.empty_like(dc.query))
    ref = oracle_for_seqs(dc, seqs)
    err = max_abs_err(out[seqs], ref, cfg.dtype)
    _say(f"{cfg.name}: max abs err {err:.3e}")
    assert err <= TOL[cfg.dtype]
    del dc
    torch.cuda.empty_cache()
