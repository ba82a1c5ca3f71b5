"""Pins of the oracle's multi-token (prefill) attention: one query token equals the
decode definition; every row equals an independent library routine with an explicit
causal mask; pure-Python brute force on tiny inputs; the FLOP count in closed form."""

import numpy as np
import pytest

import oracle
from workloads import round_to_bits

torch = pytest.importorskip("torch")


def _paged(rng, L, hkv, d, B, nb, dtype="f16"):
    perm = rng.permutation(nb)
    table = perm[:-(-L // B)]
    kp = round_to_bits(rng.standard_normal((nb, B, hkv, d), dtype=np.float32), dtype)
    vp = round_to_bits(rng.standard_normal((nb, B, hkv, d), dtype=np.float32), dtype)
    return table, kp, vp


def test_single_query_is_decode():
    rng = np.random.default_rng(0)
    table, kp, vp = _paged(rng, 37, 2, 8, 16, 8)
    q = round_to_bits(rng.standard_normal((1, 4, 8), dtype=np.float32), "f16")
    a = oracle.paged_prefill_seq(q, kp, vp, table, 37, 0.3, 16, "f16")
    b = oracle.paged_decode_seq(q[0], kp, vp, table, 37, 0.3, 16, "f16")
    assert np.array_equal(a[0], b)


@pytest.mark.parametrize("L,n", [(40, 40), (40, 7), (100, 33), (16, 16)])
def test_rows_equal_library_attention_with_causal_mask(L, n):
    rng = np.random.default_rng(L * 100 + n)
    hq, hkv, d, B = 6, 2, 16, 8
    table, kp, vp = _paged(rng, L, hkv, d, B, 20)
    q = round_to_bits(rng.standard_normal((n, hq, d), dtype=np.float32), "f16")
    got = oracle.paged_prefill_seq(q, kp, vp, table, L, 0.25, B, "f16")
    # independent: SDPA in float64 over the gathered sequence, boolean mask key <= position
    kc = torch.from_numpy(oracle.to_f64(oracle.gather(kp, table, L, B), "f16"))
    vc = torch.from_numpy(oracle.to_f64(oracle.gather(vp, table, L, B), "f16"))
    qf = torch.from_numpy(oracle.to_f64(q, "f16"))
    g = hq // hkv
    pos = torch.arange(L - n, L).view(n, 1)
    mask = torch.arange(L).view(1, L) <= pos                          # [n, L]
    for h in range(hq):
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[:, h].unsqueeze(0), kc[:, h // g].unsqueeze(0), vc[:, h // g].unsqueeze(0),
            attn_mask=mask.unsqueeze(0), scale=0.25)[0]
        assert np.allclose(got[:, h], ref.numpy(), rtol=0, atol=1e-12)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    L, n, hq, hkv, d, B = 9, 4, 2, 1, 3, 4
    table, kp, vp = _paged(rng, L, hkv, d, B, 5)
    q = round_to_bits(rng.standard_normal((n, hq, d), dtype=np.float32), "f16")
    got = oracle.paged_prefill_seq(q, kp, vp, table, L, 0.5, B, "f16")
    kc = oracle.to_f64(oracle.gather(kp, table, L, B), "f16").tolist()
    vc = oracle.to_f64(oracle.gather(vp, table, L, B), "f16").tolist()
    qf = oracle.to_f64(q, "f16").tolist()
    for i in range(n):
        p = L - n + i
        want = oracle.brute_force_seq(qf[i], kc[:p + 1], vc[:p + 1], 0.5)
        assert np.allclose(got[i], np.array(want), rtol=0, atol=1e-12)


def test_first_position_returns_its_own_value():
    rng = np.random.default_rng(4)
    L = 5
    table, kp, vp = _paged(rng, L, 1, 8, 4, 4)
    q = round_to_bits(rng.standard_normal((L, 3, 8), dtype=np.float32), "f16")
    got = oracle.paged_prefill_seq(q, kp, vp, table, L, 0.5, 4, "f16")
    v0 = oracle.to_f64(vp[table[0], 0, 0], "f16")
    for h in range(3):
        assert np.array_equal(got[0, h], v0)          # position 0 sees only itself


def test_more_queries_than_positions_gives_zeros():
    rng = np.random.default_rng(5)
    table, kp, vp = _paged(rng, 3, 1, 4, 4, 2)
    q = round_to_bits(rng.standard_normal((5, 1, 4), dtype=np.float32), "f16")
    got = oracle.paged_prefill_seq(q, kp, vp, table, 3, 0.5, 4, "f16")
    assert not got[:2].any() and got[2:].any()


def test_batch_layout_and_flops():
    rng = np.random.default_rng(6)
    table0, kp, vp = _paged(rng, 20, 2, 8, 16, 8)
    tables = np.stack([table0, table0])
    q = round_to_bits(rng.standard_normal((7, 4, 8), dtype=np.float32), "f16")
    qs = [0, 3, 7]
    out = oracle.paged_prefill(q, qs, kp, vp, tables, [20, 18], 0.3, 16, "f16")
    assert np.array_equal(out[0:3], oracle.paged_prefill_seq(q[0:3], kp, vp, table0, 20, 0.3, 16, "f16"))
    assert np.array_equal(out[3:7], oracle.paged_prefill_seq(q[3:7], kp, vp, table0, 18, 0.3, 16, "f16"))
    # FLOPs: positions 17..19 and 14..17 -> (18+19+20) + (15+16+17+18) key positions
    assert oracle.prefill_flops([3, 4], [20, 18], 4, 8) == 4 * (57 + 66) * 4 * 8
    # a whole prompt of n tokens: n (n + 1) / 2 key positions per query head
    assert oracle.prefill_flops([2407], [2407], 14, 64) == 4 * (2407 * 2408 // 2) * 14 * 64
