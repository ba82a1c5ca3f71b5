"""FP8 (E4M3) keys and values ("PagedAttention and Virtual Memory Management", section
1: b = 1).  The cache write rounds 16-bit keys / values to E4M3 bit-exactly like the
oracle (ties to even, saturation at 448, NaN kept); the gather and the block copy move
the codes bit-exactly; decode reads the codes exactly and matches the oracle within the
tolerance of the query's type, on every launch plan and block size."""

import dataclasses
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import paged_kv_cache_68_amd as pk  # noqa: E402
from workloads import config_by_name, make_case, round_to_bits  # noqa: E402

from .gpu_helpers import (  # noqa: E402
    TOL, DeviceCase, max_abs_err, oracle_after_write, oracle_for_seqs, to_dev, to_host_bits,
)


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _fp8(cfg):
    return dataclasses.replace(cfg, kv_dtype="fp8", name=f"{cfg.name}_fp8kv")


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_cache_write_rounds_like_the_oracle(io):
    """Special values and a dense sweep of ordinary ones through reshape_and_cache."""
    H, d, T = 2, 64, 64
    special = [0.0, -0.0, 1.0, 1.0625, 1.1875, -1.0625, 447.9, 448.0, 460.0, 464.0, 470.0,
               1000.0, -1000.0, math.inf, -math.inf, math.nan, 2.0 ** -9, 2.0 ** -10,
               1.5 * 2.0 ** -10, 2.0 ** -6, 0.3, -0.3, 240.0, 256.0, 1e-6, 65504.0]
    rng = np.random.default_rng(70)
    vals = np.concatenate([np.array(special, dtype=np.float32),
                           (rng.standard_normal(T * H * d - len(special)) *
                            np.exp2(rng.integers(-12, 10, T * H * d - len(special)))).astype(np.float32)])
    if io == "f16":
        bits = vals.astype(np.float16).view(np.uint16)
    else:
        bits = round_to_bits(np.nan_to_num(vals, nan=0.0, posinf=3e38, neginf=-3e38), "bf16")
        bits[np.isnan(vals)] = 0x7FC0
        bits[vals == math.inf] = 0x7F80
        bits[vals == -math.inf] = 0xFF80
    key = bits.reshape(T, H, d)
    value = key[::-1].copy()
    pool = pk.KVPool(1, 8, H, d, "fp8", io_dtype=io)
    pool.k_cache(0).zero_()
    pool.v_cache(0).zero_()
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    pk.reshape_and_cache(pool, 0, to_dev(key, io), to_dev(value, io), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kp = np.zeros((8, 16, H, d), np.uint8)
    vp = np.zeros((8, 16, H, d), np.uint8)
    oracle.scatter(kp, vp, oracle.quantize_fp8(key, io), oracle.quantize_fp8(value, io), slots, 16)
    assert np.array_equal(to_host_bits(pool.k_cache(0)), kp)
    assert np.array_equal(to_host_bits(pool.v_cache(0)), vp)


@pytest.mark.parametrize("cfg_idx", [1, 2, 4])
def test_configs_with_fp8_pools(cfg_idx):
    cfg = _fp8(config_by_name(cfg_idx))
    _say(cfg.name)
    case = make_case(cfg)
    dc = DeviceCase(case)
    out = to_host_bits(dc.step())
    torch.cuda.synchronize()
    ref, kp, vp = oracle_after_write(case)
    assert np.array_equal(to_host_bits(dc.pool.k_cache(0)), kp)
    assert np.array_equal(to_host_bits(dc.pool.v_cache(0)), vp)
    assert max_abs_err(out, ref, cfg.dtype) <= TOL[cfg.dtype]
    # the gather hook returns the stored codes
    W = dc.tables.shape[1]
    kg = torch.empty((cfg.batch, W * cfg.block_size, cfg.num_kv_heads, cfg.head_dim),
                     dtype=torch.uint8, device="cuda")
    vg = torch.empty_like(kg)
    pk.kv_pool_gather(dc.pool, 0, dc.tables, dc.lens, kg, vg)
    torch.cuda.synchronize()
    kgh = to_host_bits(kg)
    for b in range(min(cfg.batch, 16)):
        L = int(case.lengths[b])
        assert np.array_equal(kgh[b, :L], oracle.gather(kp, case.block_tables[b], L, cfg.block_size))


def test_llama3_8b_fp8_full_size_sampled():
    cfg = _fp8(config_by_name(3))
    _say(cfg.name)
    case = make_case(cfg, where="device", poison=True)
    dc = DeviceCase(case)
    out = to_host_bits(dc.step())
    torch.cuda.synchronize()
    seqs = list(range(cfg.batch))               # every sequence of the 64 x 8,192 batch
    ref = oracle_for_seqs(dc, seqs)
    err = max_abs_err(out[seqs], ref, cfg.dtype)
    _say(f"{cfg.name}: max abs err {err:.3e} over {len(seqs)} sequences")
    assert err <= TOL[cfg.dtype]


def _random_codes(rng, shape):
    """E4M3 codes of magnitude 2**-3 .. 2**1 (exponent fields 4..8) with random signs."""
    mag = rng.integers(0x20, 0x41, shape, dtype=np.uint8)
    return mag | (rng.integers(0, 2, shape, dtype=np.uint8) << 7)


PLANS = [
    {"PAGEDKV_SPLIT": "1"},
    {"PAGEDKV_SPLIT": "0"},
    {"PAGEDKV_SPLIT": "0", "PAGEDKV_GROUP": "0", "PAGEDKV_PARTS_PER_WAVE": "3"},
    {"PAGEDKV_SPLIT": "0", "PAGEDKV_GROUP_HEADS": "2", "PAGEDKV_GROUP_SLOTS": "2", "PAGEDKV_GROUP_PPW": "1"},
    {"PAGEDKV_SPLIT": "0", "PAGEDKV_STREAM": "1"},
]


@pytest.mark.parametrize("plan", range(len(PLANS)))
@pytest.mark.parametrize("B", [8, 16, 32])
@pytest.mark.parametrize("hq,hkv,d,io", [(32, 8, 128, "bf16"), (14, 2, 64, "f16"), (8, 8, 128, "f16"),
                                         (32, 2, 128, "bf16")])
def test_decode_plans_and_block_sizes(plan, B, hq, hkv, d, io, monkeypatch):
    for k, v in PLANS[plan].items():
        monkeypatch.setenv(k, v)
    _say(f"fp8 plan {PLANS[plan]} B={B} hq={hq} hkv={hkv} d={d} io={io}")
    rng = np.random.default_rng(80 + B)
    lens = np.array([1, B - 1, B, B + 1, 511, 512, 513, 2000, 0, 3000, 17], dtype=np.int32)
    need = int(sum(-(-int(L) // B) for L in lens))
    nb = need + 8
    perm = rng.permutation(nb)
    W = -(-int(lens.max()) // B)
    tables = np.full((len(lens), W), -1, dtype=np.int32)
    pos = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // B)
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    kp = _random_codes(rng, (nb, B, hkv, d))
    vp = _random_codes(rng, (nb, B, hkv, d))
    q = round_to_bits(rng.standard_normal((len(lens), hq, d), dtype=np.float32), io)
    pool = pk.KVPool(1, nb, hkv, d, "fp8", block_size=B, io_dtype=io)
    pool.k_cache(0).copy_(to_dev(kp, "fp8"))
    pool.v_cache(0).copy_(to_dev(vp, "fp8"))
    qd = to_dev(q, io)
    out = torch.empty_like(qd)
    scale = 1.0 / math.sqrt(d)
    pk.paged_attention_decode(pool, 0, out, qd, torch.from_numpy(tables).cuda(),
                              torch.from_numpy(lens).cuda(), scale=scale)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, scale, B, "fp8", q_dtype=io)
    assert max_abs_err(got, ref, io) <= TOL[io]
    assert not got[8].any()


def test_copy_blocks_on_fp8_pool():
    nb, hkv, d = 48, 8, 128
    rng = np.random.default_rng(90)
    pool = pk.KVPool(2, nb, hkv, d, "fp8")
    host = []
    for layer in range(2):
        for which in (pool.k_cache, pool.v_cache):
            codes = rng.integers(0, 256, (nb, 16, hkv, d), dtype=np.uint8)
            which(layer).copy_(to_dev(codes, "fp8"))
            host.append(codes)
    perm = rng.permutation(nb)
    copies = np.stack([perm[:12], perm[12:24], rng.integers(0, 17, 12)], axis=1).astype(np.int32)
    pk.copy_blocks(pool, torch.from_numpy(copies).cuda())
    torch.cuda.synchronize()
    got = [to_host_bits(f(l)) for l in range(2) for f in (pool.k_cache, pool.v_cache)]
    for g, h in zip(got, host):
        want = h.copy()
        oracle.copy_blocks(want, copies.tolist())
        assert np.array_equal(g, want)
