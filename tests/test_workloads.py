"""The seeded input generators: determinism, shapes, and the structure each config asks for."""

import numpy as np
import pytest

from workloads import CONFIGS, config_by_name, make_case, nan_bits
from workloads.gen import LOGNORMAL_SIGMA, SHARED_PREFIX_TOKENS, draw_lengths


def test_five_configs():
    assert [c.index for c in CONFIGS] == [1, 2, 3, 4, 5]
    c3 = config_by_name("c3")
    assert (c3.num_q_heads, c3.num_kv_heads, c3.head_dim, c3.dtype, c3.batch) == (32, 8, 128, "bf16", 64)
    assert config_by_name(5).group == 1 and config_by_name(1).group == 7


def test_c1_structure_and_determinism():
    cfg = config_by_name(1)
    a = make_case(cfg)
    b = make_case(cfg)
    assert list(a.lengths) == [1, 16, 17, 40]
    assert a.block_tables.shape == (4, 3)
    assert [int((t >= 0).sum()) for t in a.block_tables] == [1, 1, 2, 3]
    for x, y in ((a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.query, b.query),
                 (a.block_tables, b.block_tables), (a.slot_mapping, b.slot_mapping)):
        assert np.array_equal(x, y)
    # the new token's slot is position L-1
    for i, L in enumerate(a.lengths):
        blk = a.block_tables[i, (L - 1) // 16]
        assert a.slot_mapping[i] == blk * 16 + (L - 1) % 16
        # before the write the slot holds poison
        assert np.all(a.k_pool[blk, (L - 1) % 16] == nan_bits("f16"))
    # blocks are distinct across sequences
    used = a.block_tables[a.block_tables >= 0]
    assert len(np.unique(used)) == len(used)


def test_c2_lengths_lognormal():
    cfg = config_by_name(2)
    lens = draw_lengths(cfg, np.random.default_rng(cfg.index))
    assert lens.min() >= 1 and lens.max() <= 2048
    assert 150 <= np.median(lens) <= 260
    assert abs(LOGNORMAL_SIGMA - 0.8577) < 1e-3


def test_c4_shared_prefix_copy_on_write():
    cfg = config_by_name(4)
    c = make_case(cfg)
    t = c.block_tables
    # all 64 tables share the same 256 full blocks
    assert np.all(t[:, :256] == t[0, :256])
    assert len(np.unique(t[:, :256])) == 256
    # 63 copies of the shared partial block, the last sequence writes in place
    assert len(c.cow_copies) == 63
    src = {s for s, _ in c.cow_copies}
    assert len(src) == 1
    partial = src.pop()
    assert t[63, 256] == partial
    assert len(set(t[:, 256].tolist())) == 64
    assert np.all(c.lengths > SHARED_PREFIX_TOKENS) and np.all(c.lengths <= SHARED_PREFIX_TOKENS + 512)
    # reference counts: shared full blocks 64, everything else 1
    assert np.all(c.refcounts[t[0, :256]] == 64)
    private = np.unique(t[:, 256:][t[:, 256:] >= 0])
    assert np.all(c.refcounts[private] == 1)
    # each copy keeps the 7 prefix tokens of the source block
    for s, dst in c.cow_copies:
        assert np.array_equal(c.k_pool[dst, :7], c.k_pool[s, :7])


def test_truncate_keeps_prefix_sequences():
    cfg = config_by_name(2)
    full = make_case(cfg)
    small = make_case(cfg, batch=8)
    assert np.array_equal(small.lengths, full.lengths[:8])
    assert np.array_equal(small.query, full.query[:8])
    w = small.block_tables.shape[1]
    assert np.array_equal(small.block_tables, full.block_tables[:8, :w])


@pytest.mark.parametrize("idx", [3, 5])
def test_large_configs_metadata(idx):
    cfg = config_by_name(idx)
    lens = draw_lengths(cfg, np.random.default_rng(cfg.index))
    need = sum(-(-int(L) // 16) for L in lens)
    assert need <= cfg.num_blocks
    if idx == 3:
        assert np.all(lens == 8192)
    else:
        assert lens.min() >= 1 and lens.max() <= 4096


def test_fork_batches():
    """fork_<P>_<S>: cfg.batch forks of a P-token prefix, U[1, S] private tokens each; the
    full blocks of the prefix are shared, the partial one copied on write."""
    import dataclasses

    from workloads import fork_shape
    assert fork_shape(config_by_name(4)) == (SHARED_PREFIX_TOKENS, 64, 512)
    cfg = dataclasses.replace(config_by_name(4), index=77, batch=8, num_blocks=200,
                              lengths="fork_100_40")
    c = make_case(cfg)
    assert fork_shape(cfg) == (100, 8, 40)
    t = c.block_tables
    assert np.all(t[:, :6] == t[0, :6]) and list(c.shared_blocks) == list(t[0, :6])
    assert len(c.cow_copies) == 7 and len(set(t[:, 6].tolist())) == 8
    assert np.all(c.lengths > 100) and np.all(c.lengths <= 140)
    private = t[:, 6:][t[:, 6:] >= 0]
    assert len(private) == len(set(private.tolist()))
