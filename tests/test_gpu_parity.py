"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Cache write and block-table gather: bit-exact.  Attention: max-abs error against the
unrounded fp64 oracle within 2e-3 (fp16) / 8e-3 (bf16); bit-identical under a
relabelling of physical blocks and from run to run.
"""

import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import paged_kv_cache_68_amd as pk  # noqa: E402
from workloads import config_by_name, make_case, nan_bits, round_to_bits  # noqa: E402
from workloads.configs import DecodeConfig  # noqa: E402

from .gpu_helpers import (  # noqa: E402
    TOL, DeviceCase, flat_bar, max_abs_err, oracle_after_write, oracle_for_seqs, to_dev, to_host_bits,
)


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


# ------------------------------------------------------------------ cache write / gather

@pytest.mark.parametrize("cfg_idx", [1, 2])
def test_reshape_and_cache_bit_exact(cfg_idx):
    cfg = config_by_name(cfg_idx)
    case = make_case(cfg)
    _say(f"reshape_and_cache {cfg.name}")
    dc = DeviceCase(case)
    dc.write()
    torch.cuda.synchronize()
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    oracle.scatter(kp, vp, case.new_key, case.new_value, case.slot_mapping, cfg.block_size)
    assert np.array_equal(to_host_bits(dc.pool.k_cache(0)), kp)
    assert np.array_equal(to_host_bits(dc.pool.v_cache(0)), vp)


def test_reshape_and_cache_mha_shape_with_padding():
    """Llama-2-70B head shape (64 x 128 fp16 rows); 512 distinct random slots and
    negative (padding) slots that must write nothing."""
    rng = np.random.default_rng(55)
    nb, H, d, T = 2048, 64, 128, 512
    _say("reshape_and_cache 64x128 rows")
    pool = pk.KVPool(1, nb, H, d, "f16")
    kp = rng.integers(0, 1 << 16, size=(nb, 16, H, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(nb, 16, H, d), dtype=np.uint16)
    pool.k_cache(0).copy_(to_dev(kp, "f16"))
    pool.v_cache(0).copy_(to_dev(vp, "f16"))
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int64)
    slots[::37] = -1
    key = rng.integers(0, 1 << 16, size=(T, H, d), dtype=np.uint16)
    val = rng.integers(0, 1 << 16, size=(T, H, d), dtype=np.uint16)
    pk.reshape_and_cache(pool, 0, to_dev(key, "f16"), to_dev(val, "f16"),
                         torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    keep = slots >= 0
    oracle.scatter(kp, vp, key[keep], val[keep], slots[keep], 16)
    assert np.array_equal(to_host_bits(pool.k_cache(0)), kp)
    assert np.array_equal(to_host_bits(pool.v_cache(0)), vp)


@pytest.mark.parametrize("cfg_idx", [1, 2, 4])
def test_gather_bit_exact(cfg_idx):
    cfg = config_by_name(cfg_idx)
    case = make_case(cfg, batch=min(cfg.batch, 48))
    _say(f"kv_pool_gather {cfg.name}")
    dc = DeviceCase(case)
    B, W = case.block_tables.shape
    ko = torch.empty((B, W * 16, cfg.num_kv_heads, cfg.head_dim), dtype=dc.query.dtype, device="cuda")
    vo = torch.empty_like(ko)
    pk.kv_pool_gather(dc.pool, 0, dc.tables, dc.lens, ko, vo)
    torch.cuda.synchronize()
    kh, vh = to_host_bits(ko), to_host_bits(vo)
    for b in range(B):
        L = int(case.lengths[b])
        assert np.array_equal(kh[b, :L], oracle.gather(case.k_pool, case.block_tables[b], L, 16))
        assert np.array_equal(vh[b, :L], oracle.gather(case.v_pool, case.block_tables[b], L, 16))
        assert not kh[b, L:].any() and not vh[b, L:].any()


# ------------------------------------------------------------------ decode parity, whole configs

@pytest.mark.parametrize("cfg_idx", [1, 2, 4])
def test_decode_step_matches_oracle(cfg_idx):
    cfg = config_by_name(cfg_idx)
    case = make_case(cfg)
    _say(f"decode step {cfg.name}")
    dc = DeviceCase(case)
    out = to_host_bits(dc.step())
    ref, _, _ = oracle_after_write(case)
    err = max_abs_err(out, ref, cfg.dtype)
    _say(f"{cfg.name}: max abs err {err:.3e}")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("cfg_idx", [3, 5])
def test_decode_step_full_size_sampled(cfg_idx):
    """Full-size configs built on the device; the oracle checks every sequence (the 64 x
    8,192 batch and the 512-sequence one)."""
    cfg = config_by_name(cfg_idx)
    case = make_case(cfg, where="device")
    seqs = list(range(cfg.batch))
    _say(f"decode step {cfg.name} (checked {len(seqs)} sequences)")
    dc = DeviceCase(case)
    out = to_host_bits(dc.step())
    assert np.all(np.isfinite(oracle.to_f64(out, cfg.dtype)))
    ref = oracle_for_seqs(dc, seqs)
    got = oracle.to_f64(out[seqs], cfg.dtype)
    err = max_abs_err(out[seqs], ref, cfg.dtype)
    _say(f"{cfg.name}: max abs err {err:.3e}")
    assert err <= TOL[cfg.dtype]
    assert np.all(np.abs(got - ref) <= flat_bar(ref, cfg.dtype))
    # the phases called separately produce the same bits
    out2 = torch.empty_like(dc.out)
    pk.paged_attention_partitions(dc.pool, 0, out2, dc.query, dc.tables, dc.lens, cfg.scale,
                                  cfg.partition_size, dc.workspace)
    pk.paged_attention_reduce(dc.pool, 0, out2, dc.query, dc.tables, dc.lens, cfg.scale,
                              cfg.partition_size, dc.workspace)
    assert np.array_equal(to_host_bits(out2), out)


# ------------------------------------------------------------------ shapes and partitions

def _small_cfg(hq, hkv, d, dtype, lens_name="fixed_1_16_17_40", nb=256, batch=4, part=512):
    return DecodeConfig(index=900 + hq * 3 + hkv + d, name=f"sweep_{hq}_{hkv}_{d}_{dtype}",
                        num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, block_size=16,
                        num_blocks=nb, batch=batch, lengths=lens_name, partition_size=part,
                        description="sweep")


@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_group_and_head_dim_sweep(g, d, dtype):
    cfg = _small_cfg(2 * g, 2, d, dtype)
    case = make_case(cfg)
    dc = DeviceCase(case)
    out = to_host_bits(dc.step())
    ref, _, _ = oracle_after_write(case)
    assert max_abs_err(out, ref, dtype) <= TOL[dtype]


def _custom_case(lens, hq=8, hkv=2, d=128, dtype="bf16", nb=None, seed=0):
    """Scattered case with the given lengths (host-built)."""
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum(-(-int(L) // 16) for L in lens))
    nb = nb or max(16, need + 8)
    cfg = DecodeConfig(index=1000 + seed, name="custom", num_q_heads=hq, num_kv_heads=hkv,
                       head_dim=d, dtype=dtype, block_size=16, num_blocks=nb, batch=len(lens),
                       lengths="fixed_1_16_17_40", partition_size=512, description="custom")
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    W = max(1, max(-(-int(L) // 16) for L in lens))
    tables = np.full((len(lens), W), -1, dtype=np.int32)
    pos = 0
    for b, L in enumerate(lens):
        n = -(-int(L) // 16)
        tables[b, :n] = perm[pos:pos + n]
        pos += n
    kp = np.full((nb, 16, hkv, d), nan_bits(dtype), dtype=np.uint16)
    vp = np.full((nb, 16, hkv, d), nan_bits(dtype), dtype=np.uint16)
    for b, L in enumerate(lens):
        for t in range(int(L)):
            blk = tables[b, t // 16]
            kp[blk, t % 16] = round_to_bits(rng.standard_normal((hkv, d), dtype=np.float32), dtype)
            vp[blk, t % 16] = round_to_bits(rng.standard_normal((hkv, d), dtype=np.float32), dtype)
    q = round_to_bits(rng.standard_normal((len(lens), hq, d), dtype=np.float32), dtype)
    return cfg, lens, tables, kp, vp, q


def _run_custom(cfg, lens, tables, kp, vp, q, part=512, scale=None):
    pool = pk.KVPool(1, cfg.num_blocks, cfg.num_kv_heads, cfg.head_dim, cfg.dtype)
    pool.k_cache(0).copy_(to_dev(kp, cfg.dtype))
    pool.v_cache(0).copy_(to_dev(vp, cfg.dtype))
    qd = to_dev(q, cfg.dtype)
    out = torch.empty_like(qd)
    td = torch.from_numpy(tables).cuda()
    ld = torch.from_numpy(lens).cuda()
    pk.paged_attention_decode(pool, 0, out, qd, td, ld, scale=cfg.scale if scale is None else scale,
                              partition_size=part)
    return to_host_bits(out)


@pytest.mark.parametrize("scale", [-0.3, 0.0])
@pytest.mark.parametrize("hq,env", [(8, {}), (8, {"PAGEDKV_SPLIT": "0", "PAGEDKV_GROUP": "0"}),
                                    (2, {"PAGEDKV_KERNEL": "valu"}), (2, {"PAGEDKV_KERNEL": "mfma"})])
def test_negative_and_zero_scale(monkeypatch, scale, hq, env):
    """The scale multiplies q.k whatever its sign: a negative one favours the lowest
    scores, zero gives every position the same weight (the mean of the values)."""
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    lens = [1, 17, 600, 1500]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=hq, seed=31)
    out = _run_custom(cfg, lens, tables, kp, vp, q, scale=scale)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, scale, 16, cfg.dtype)
    assert np.all(np.abs(oracle.to_f64(out, cfg.dtype) - ref) <= flat_bar(ref, cfg.dtype))


@pytest.mark.parametrize("part", [16, 64, 512, 4096])
def test_partition_boundaries(part):
    lens = [1, 15, 16, 17, 511, 512, 513, 1024, 1025, 2000]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, seed=part)
    out = _run_custom(cfg, lens, tables, kp, vp, q, part)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, cfg.dtype)
    assert max_abs_err(out, ref, cfg.dtype) <= TOL[cfg.dtype]


def test_length_one_is_exact_value():
    cfg, lens, tables, kp, vp, q = _custom_case([1, 1, 17], hq=8, hkv=2, d=64, dtype="f16", seed=3)
    out = _run_custom(cfg, lens, tables, kp, vp, q)
    for b in (0, 1):
        v = vp[tables[b, 0], 0]            # [Hkv, d]
        for h in range(8):
            assert np.array_equal(out[b, h], v[h // 4])


def test_zero_length_gives_zeros_and_others_unaffected():
    cfg, lens, tables, kp, vp, q = _custom_case([5, 0, 40], seed=4)
    out = _run_custom(cfg, lens, tables, kp, vp, q)
    assert not out[1].any()
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, cfg.dtype)
    assert max_abs_err(out, ref, cfg.dtype) <= TOL[cfg.dtype]


def test_zero_query_and_constant_values():
    cfg, lens, tables, kp, vp, q = _custom_case([33, 700], hq=4, hkv=4, d=128, dtype="f16", seed=5)
    q[0] = 0                          # -> mean of V
    c = np.float16(0.8125).view(np.uint16)
    for t in range(700):              # sequence 1: constant V -> that constant
        vp[tables[1, t // 16], t % 16] = c
    out = oracle.to_f64(_run_custom(cfg, lens, tables, kp, vp, q), "f16")
    vf = oracle.to_f64(oracle.gather(vp, tables[0], 33, 16), "f16")
    assert np.max(np.abs(out[0] - vf.mean(axis=0))) <= TOL["f16"]
    assert np.max(np.abs(out[1] - 0.8125)) <= 2 ** -11


def test_block_permutation_bit_identical_and_deterministic():
    cfg, lens, tables, kp, vp, q = _custom_case([3000, 777, 16, 1], hq=32, hkv=8, d=128,
                                               dtype="bf16", nb=400, seed=6)
    out = _run_custom(cfg, lens, tables, kp, vp, q)
    again = _run_custom(cfg, lens, tables, kp, vp, q)
    assert np.array_equal(out, again)
    pi = np.random.default_rng(7).permutation(cfg.num_blocks)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    out2 = _run_custom(cfg, lens, t2, kp2, vp2, q)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("hq,hkv,d,dtype", [(32, 8, 128, "bf16"), (14, 2, 64, "f16"), (8, 8, 128, "bf16")])
def test_short_contexts_meet_the_flat_bar(hq, hkv, d, dtype):
    """Contexts of 2 to 33 tokens average few values, so rounding the softmax weights for
    the value product would show there first: every element within the flat bar."""
    lens = list(range(2, 34)) * 2
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=40 + d)
    out = _run_custom(cfg, lens, tables, kp, vp, q)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, dtype)
    err = np.abs(oracle.to_f64(out, dtype) - ref)
    _say(f"short contexts {dtype} G={hq // hkv}: max abs err {err.max():.3e}")
    assert np.all(err <= flat_bar(ref, dtype))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4)])
def test_valu_kernel_with_whole_sequences_per_wave(monkeypatch, hq, hkv):
    """The VALU kernel's item plan with every partition of a sequence on one wave (no
    partial results, no reduce): the oracle's answer, sequences of 0 to 3,000 tokens."""
    monkeypatch.setenv("PAGEDKV_KERNEL", "valu")
    monkeypatch.setenv("PAGEDKV_SPLIT", "0")
    monkeypatch.setenv("PAGEDKV_PARTS_PER_WAVE", "16")
    lens = [3000, 777, 16, 1, 0, 513, 2048, 1500]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=hq, hkv=hkv, d=128, dtype="f16", seed=70 + hq)
    out = _run_custom(cfg, lens, tables, kp, vp, q)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, "f16")
    err = np.abs(oracle.to_f64(out, "f16") - ref)
    _say(f"VALU whole-sequence waves G={hq // hkv}: max abs err {err.max():.3e}")
    assert np.all(err <= flat_bar(ref, "f16"))


def test_table_padding_is_never_read():
    cfg, lens, tables, kp, vp, q = _custom_case([20, 100, 3], seed=8)
    base = _run_custom(cfg, lens, tables, kp, vp, q)
    t2 = tables.copy()
    t2[t2 < 0] = 1 << 30            # garbage past each sequence's blocks
    assert np.array_equal(_run_custom(cfg, lens, t2, kp, vp, q), base)


def test_scale_is_applied():
    cfg, lens, tables, kp, vp, q = _custom_case([300], hq=2, hkv=2, d=64, dtype="f16", seed=9)
    pool = pk.KVPool(1, cfg.num_blocks, 2, 64, "f16")
    pool.k_cache(0).copy_(to_dev(kp, "f16"))
    pool.v_cache(0).copy_(to_dev(vp, "f16"))
    qd = to_dev(q, "f16")
    out = torch.empty_like(qd)
    for scale in (0.0, 0.05, 0.3):
        pk.paged_attention_decode(pool, 0, out, qd, torch.from_numpy(tables).cuda(),
                                  torch.from_numpy(lens).cuda(), scale=scale)
        ref = oracle.paged_decode(q, kp, vp, tables, lens, scale, 16, "f16")
        assert max_abs_err(to_host_bits(out), ref, "f16") <= TOL["f16"]


# ------------------------------------------------------------------ every launch shape

@pytest.mark.parametrize("split,per", [("1", None), ("0", "1"), ("0", "2"), ("0", "3"), ("0", "8")])
@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("hq,hkv,d,dtype", [(8, 2, 128, "bf16"), (4, 4, 128, "f16"), (14, 2, 64, "f16")])
def test_launch_shapes_match_oracle(split, per, kernel, hq, hkv, d, dtype, monkeypatch):
    """Four waves per partition, or one wave walking 1/2/3/8 partitions in one stream;
    matrix-core and VALU kernels: all must match the oracle (and each other's bits
    within a kernel, since the summation order depends only on logical positions)."""
    monkeypatch.setenv("PAGEDKV_SPLIT", split)
    if per is not None:
        monkeypatch.setenv("PAGEDKV_PARTS_PER_WAVE", per)
    if kernel != "auto":
        monkeypatch.setenv("PAGEDKV_KERNEL", kernel)
    lens = [1, 15, 16, 17, 511, 512, 513, 1024, 1025, 2000, 0, 3000]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=11)
    out = _run_custom(cfg, lens, tables, kp, vp, q, 512)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, dtype)
    assert max_abs_err(out, ref, dtype) <= TOL[dtype]
    assert not out[10].any()                       # the empty sequence


@pytest.mark.parametrize("heads,slots,ppw", [(1, 1, 1), (1, 4, 2), (2, 4, 4), (2, 2, 1), (4, 2, 3),
                                             (1, 8, 8), (2, 1, 8), (8, 1, 2)])
@pytest.mark.parametrize("hq,hkv,d,dtype", [(32, 8, 128, "bf16"), (16, 8, 64, "f16"),
                                           (8, 8, 128, "f16")])
def test_group_plan_shapes_match_oracle(heads, slots, ppw, hq, hkv, d, dtype, monkeypatch):
    """Work-groups of `heads` KV heads x `slots` waves, each wave walking `ppw`
    partitions: one chunk per sequence or several (then the reduce kernel combines the
    chunks' partials); short sequences leave waves without blocks."""
    monkeypatch.setenv("PAGEDKV_SPLIT", "0")
    monkeypatch.setenv("PAGEDKV_GROUP_HEADS", str(heads))
    monkeypatch.setenv("PAGEDKV_GROUP_SLOTS", str(slots))
    monkeypatch.setenv("PAGEDKV_GROUP_PPW", str(ppw))
    lens = [1, 15, 16, 17, 511, 512, 513, 1024, 1025, 2000, 0, 4500]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=12)
    out = _run_custom(cfg, lens, tables, kp, vp, q, 512)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, dtype)
    assert max_abs_err(out, ref, dtype) <= TOL[dtype]
    assert not out[10].any()
    # the same plan gives the same bits every time
    assert np.array_equal(_run_custom(cfg, lens, tables, kp, vp, q, 512), out)


def test_group_plan_off_matches_oracle(monkeypatch):
    """PAGEDKV_GROUP=0: one wave per item with partials for every partition."""
    monkeypatch.setenv("PAGEDKV_SPLIT", "0")
    monkeypatch.setenv("PAGEDKV_GROUP", "0")
    lens = [1, 17, 513, 2000, 0, 4500]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=32, hkv=8, d=128, dtype="bf16", seed=13)
    out = _run_custom(cfg, lens, tables, kp, vp, q, 512)
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, "bf16")
    assert max_abs_err(out, ref, "bf16") <= TOL["bf16"]


@pytest.mark.parametrize("group", ["1", "0"])
def test_streaming_loads_give_identical_bits(group, monkeypatch):
    """The non-temporal load hint is a cache policy only: results are bit-identical with
    and without it, in the group plan and in the one-wave-per-item plan."""
    monkeypatch.setenv("PAGEDKV_SPLIT", "0")
    monkeypatch.setenv("PAGEDKV_GROUP", group)
    lens = [1, 17, 513, 2000, 0, 4500, 33]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=32, hkv=8, d=128, dtype="bf16", seed=14)
    outs = []
    for stream in ("0", "1"):
        monkeypatch.setenv("PAGEDKV_STREAM", stream)
        outs.append(_run_custom(cfg, lens, tables, kp, vp, q, 512))
    assert np.array_equal(outs[0], outs[1])
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, "bf16")
    assert max_abs_err(outs[1], ref, "bf16") <= TOL["bf16"]


@pytest.mark.parametrize("hq,hkv,d,dtype,heads,slots,ppw", [
    (32, 8, 128, "bf16", 1, 4, 3), (32, 8, 128, "bf16", 2, 2, 5), (8, 8, 128, "f16", 2, 2, 5)])
def test_longest_first_order_gives_identical_bits(hq, hkv, d, dtype, heads, slots, ppw, monkeypatch):
    """Group plans with one chunk per sequence may take the sequences longest first (a
    one-work-group kernel writes the order into the workspace, PAGEDKV_ORDER=1 forces
    it): the same bits as in batch order, and the oracle's values."""
    monkeypatch.setenv("PAGEDKV_SPLIT", "0")
    monkeypatch.setenv("PAGEDKV_GROUP_HEADS", str(heads))
    monkeypatch.setenv("PAGEDKV_GROUP_SLOTS", str(slots))
    monkeypatch.setenv("PAGEDKV_GROUP_PPW", str(ppw))
    lens = [1, 15, 16, 17, 511, 512, 513, 1024, 1025, 2000, 0, 4500, 33, 4500, 7]
    cfg, lens, tables, kp, vp, q = _custom_case(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=15)
    outs = {}
    for order in ("0", "1"):
        monkeypatch.setenv("PAGEDKV_ORDER", order)
        outs[order] = _run_custom(cfg, lens, tables, kp, vp, q, 512)
    assert np.array_equal(outs["0"], outs["1"])
    ref = oracle.paged_decode(q, kp, vp, tables, lens, cfg.scale, 16, dtype)
    assert max_abs_err(outs["1"], ref, dtype) <= TOL[dtype]
    assert not outs["1"][10].any()


@pytest.mark.parametrize("kv", ["", "fp8"])
def test_longest_first_order_on_a_ragged_batch(kv, monkeypatch):
    """300 sequences of U[1, 1,500] tokens, MHA heads (the group plan with whole
    sequences per work-group), the cache write folded in: longest first (forced) and
    batch order give the same bits, the pool the oracle's bytes, the output the oracle's
    values to the flat bar."""
    cfg = DecodeConfig(index=7100, name="ragged_mha_b300", num_q_heads=8, num_kv_heads=8,
                       head_dim=128, dtype="f16", block_size=16, num_blocks=300 * 94 + 16,
                       batch=300, lengths="uniform_1500", partition_size=512,
                       description="ragged MHA batch", kv_dtype=kv)
    case = make_case(cfg)
    outs = {}
    for order in ("0", "1"):
        monkeypatch.setenv("PAGEDKV_ORDER", order)
        dc = DeviceCase(case)
        outs[order] = to_host_bits(dc.step_append())
    assert np.array_equal(outs["0"], outs["1"])
    ref, kp, vp = oracle_after_write(case)
    got = oracle.to_f64(outs["1"], cfg.dtype)
    _say(f"ragged batch{' fp8' if kv else ''}: max abs err {np.abs(got - ref).max():.3e}")
    assert np.all(np.abs(got - ref) <= flat_bar(ref, cfg.dtype))
    assert np.array_equal(to_host_bits(dc.pool.k_cache(0)), kp)
    assert np.array_equal(to_host_bits(dc.pool.v_cache(0)), vp)


# ------------------------------------------------------------------ long contexts

@pytest.mark.parametrize("plan", [{}, {"PAGEDKV_GROUP": "0"}, {"PAGEDKV_SPLIT": "1"}])
def test_long_context_128k(plan, monkeypatch):
    """A 131,072-token sequence (256 partitions of 512, more than the in-kernel merge
    takes, so the reduce combines many chunks) beside 70,001-, 4,095- and 1-token ones;
    Llama-3-8B heads, bf16, on each launch plan; the folded cache write gives the same
    bits as the separate one."""
    for k, v in plan.items():
        monkeypatch.setenv(k, v)
    _say(f"long context 128k plan={plan}")
    hq, hkv, d, B = 32, 8, 128, 16
    lens = np.array([131072, 70001, 4095, 1], dtype=np.int32)
    nblk = [-(-int(L) // B) for L in lens]
    nb = sum(nblk) + 8
    rng = np.random.default_rng(1280)
    perm = rng.permutation(nb)
    W = max(nblk)
    tables = np.full((len(lens), W), -1, dtype=np.int32)
    pos = 0
    for b, m in enumerate(nblk):
        tables[b, :m] = perm[pos:pos + m]
        pos += m
    pool = pk.KVPool(1, nb, hkv, d, "bf16")
    gen = torch.Generator(device="cuda").manual_seed(1280)
    for cache in (pool.k_cache(0), pool.v_cache(0)):
        cache.copy_(torch.randn(cache.shape, generator=gen, device="cuda").to(torch.bfloat16))
    q = torch.randn(len(lens), hq, d, generator=gen, device="cuda").to(torch.bfloat16)
    t_d, l_d = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    scale = 1.0 / math.sqrt(d)
    out = pk.paged_attention_decode(pool, 0, torch.empty_like(q), q, t_d, l_d, scale=scale)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    q_bits = to_host_bits(q)
    for b in range(len(lens)):
        ids = torch.from_numpy(tables[b, :nblk[b]].astype(np.int64)).cuda()
        kb = to_host_bits(pool.k_cache(0).index_select(0, ids))
        vb = to_host_bits(pool.v_cache(0).index_select(0, ids))
        ref = oracle.paged_decode_seq(q_bits[b], kb, vb, np.arange(nblk[b]), int(lens[b]), scale, B, "bf16")
        err = max_abs_err(got[b:b + 1], ref[None], "bf16")
        _say(f"  seq {b} (L={lens[b]}): max abs err {err:.3e}")
        assert err <= TOL["bf16"]
    # the new token of each sequence written by the partition kernel: same bits as the
    # separate write followed by the decode above (the rows written are the same)
    nk = torch.randn(len(lens), hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    nv = torch.randn(len(lens), hkv, d, generator=gen, device="cuda").to(torch.bfloat16)
    slots = torch.from_numpy(np.array([tables[b, (L - 1) // B] * B + (L - 1) % B
                                       for b, L in enumerate(lens)], dtype=np.int64)).cuda()
    pk.reshape_and_cache(pool, 0, nk, nv, slots)
    ref_out = pk.paged_attention_decode(pool, 0, torch.empty_like(q), q, t_d, l_d, scale=scale)
    out2 = pk.paged_attention_decode_append(pool, 0, torch.empty_like(q), q, nk, nv, t_d, l_d, scale=scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(out2), to_host_bits(ref_out))
