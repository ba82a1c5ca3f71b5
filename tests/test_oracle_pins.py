"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: values the pages
print (tests/golden), brute force on tiny inputs, closed forms, invariants, and an
independent library routine (torch's scaled-dot-product attention in float64).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ page-printed values

def test_indexing_examples_from_pages():
    g = _load("indexing_examples.json")
    for ex in g["examples"]:
        table = ex["table"]
        if isinstance(table, dict):      # only the entry the page names is known
            full = [-1] * (max(int(k) for k in table) + 1)
            for k, v in table.items():
                full[int(k)] = v
            table = full
        j, o, p = oracle.locate(ex["t"], ex["block_size"], table)
        assert (j, o, p) == (ex["logical_block"], ex["offset"], ex["physical_block"]), ex["cite"]


def test_block_counts_from_pages():
    g = _load("indexing_examples.json")
    for ex in g["block_counts"]:
        n, bs = ex["tokens"], ex["block_size"]
        table = list(range(1000, 1000 + 10_000))
        # the last token sits in the last block, at the fill level the page prints
        j, o, _ = oracle.locate(n - 1, bs, table)
        assert j + 1 == ex["blocks"], ex["cite"]
        assert o + 1 == ex["last_block_fill"], ex["cite"]


def test_address_example_from_page():
    a = _load("indexing_examples.json")["address"]
    table = [-1, -1, 93]
    addr = oracle.physical_address(a["t"], a["block_size"], table, a["block_bytes"], a["token_bytes"])
    assert addr == a["physical_block"] * a["block_bytes"] + a["offset"] * a["token_bytes"]


@pytest.mark.parametrize("h", [1, 5, 7])
def test_address_head_term_matches_the_pools_own_element_addresses(h):
    """Addr_K(t) with a non-zero head ("PagedAttention and Virtual Memory Management",
    section 4): for the Llama-3-8B layer layout [blocks][16][8 KV heads][128] in bf16
    the oracle's address of (t, h) must be the address numpy itself gives element
    [table[t // 16], t % 16, h, 0] of such an array, and the bytes there must be the
    value planted at that element."""
    nb, B, hkv, d = 96, 16, 8, 128
    pool = np.zeros((nb, B, hkv, d), dtype=np.uint16)
    table = [40, 3, 93, 17]
    base = pool.__array_interface__["data"][0]
    for t in (0, 15, 16, 38, 63):
        blk, o = table[t // B], t % B
        pool[blk, o, h, 0] = 1000 + t
        addr = oracle.physical_address(t, B, table, B * hkv * d * 2, hkv * d * 2, head=h,
                                       stride_head=d * 2, base=base)
        assert addr == pool[blk, o, h, :].__array_interface__["data"][0]
        assert addr - base == np.ravel_multi_index((blk, o, h, 0), pool.shape) * 2
        flat = pool.reshape(-1).view(np.uint8)
        assert int(flat[addr - base]) | (int(flat[addr - base + 1]) << 8) == 1000 + t


def test_footprints_from_pages():
    g = _load("footprints.json")
    for ex in g["bytes_per_token"]:
        got = oracle.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"], ex["elem_bytes"])
        assert got == ex["bytes"], ex["cite"]
    for ex in g["request_bytes"]:
        got = oracle.kv_bytes_per_token(ex["layers"], ex["kv_heads"], ex["head_dim"],
                                        ex["elem_bytes"]) * ex["tokens"]
        assert got == ex["bytes"], ex["cite"]
    for ex in g["block_bytes"]:
        got = oracle.block_bytes(ex["kv_heads"], ex["head_dim"], ex["elem_bytes"],
                                 ex["block_size"], ex["layers"])
        assert got == ex["bytes"], ex["cite"]


def test_per_tile_cost_from_page():
    t = _load("footprints.json")["per_tile"]
    assert t["positions"] * t["table_entry_bytes"] == t["table_bytes"]
    # K and V of one KV head for one tile = one block's worth of that head
    kv = oracle.block_bytes(1, t["head_dim"], t["elem_bytes"], t["positions"])
    assert kv == t["kv_bytes"]
    assert 2 * t["q_heads_per_kv"] * t["positions"] * t["head_dim"] == t["multiply_adds"]


def test_table_reads_from_page():
    t = _load("footprints.json")["table_reads"]
    assert t["tokens"] * t["layers"] * t["kv_heads"] == t["reads"]


def test_pool_bytes_closed_form_matches_allocation():
    # 12 KiB / token for the Qwen shape and 128 KiB / token for Llama-3-8B
    nb, bs = 58064, 16
    assert oracle.kv_pool_bytes(24, 2, 64, 2, nb, bs) == 12288 * nb * bs
    assert oracle.kv_pool_bytes(32, 8, 128, 2, 40960, 16) == 131072 * 40960 * 16


# ------------------------------------------------------------------ storage types

def test_to_f64_exact():
    x = np.array([0.0, 1.0, -2.5, 65504.0, 2.0 ** -24], dtype=np.float16)
    assert np.array_equal(oracle.to_f64(x.view(np.uint16), "f16"), x.astype(np.float64))
    # bf16: 1.0 = 0x3F80, -2.0 = 0xC000, 1 + 2^-7 = 0x3F81
    b = np.array([0x3F80, 0xC000, 0x3F81, 0x0000], dtype=np.uint16)
    assert list(oracle.to_f64(b, "bf16")) == [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0]


# ------------------------------------------------------------------ tiny-case builders

def _tiny_case(rng, L, hq, hkv, d, bs, nb=64, dtype="f16"):
    """Contiguous K/V first, then scattered into a pool through a random table."""
    from workloads import round_to_bits
    k = round_to_bits(rng.standard_normal((L, hkv, d), dtype=np.float32), dtype)
    v = round_to_bits(rng.standard_normal((L, hkv, d), dtype=np.float32), dtype)
    q = round_to_bits(rng.standard_normal((hq, d), dtype=np.float32), dtype)
    n_blocks = -(-L // bs)
    table = rng.permutation(nb)[:max(n_blocks, 1)]
    kp = np.full((nb, bs, hkv, d), 0x7E00, dtype=np.uint16)   # NaN everywhere else
    vp = np.full((nb, bs, hkv, d), 0x7E00, dtype=np.uint16)
    for t in range(L):
        kp[table[t // bs], t % bs] = k[t]
        vp[table[t // bs], t % bs] = v[t]
    return q, k, v, kp, vp, table


def _nested(a):
    return a.tolist()


@pytest.mark.parametrize("seed", range(6))
def test_oracle_equals_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    hkv = [1, 2, 2, 1, 3, 2][seed]
    g = [1, 2, 3, 4, 2, 7][seed]
    d = [4, 8, 4, 8, 4, 8][seed]
    bs = [1, 4, 16, 16, 4, 16][seed]
    L = [1, 13, 17, 40, 9, 33][seed]
    hq = hkv * g
    q, k, v, kp, vp, table = _tiny_case(rng, L, hq, hkv, d, bs)
    scale = 1.0 / math.sqrt(d)
    got = oracle.paged_decode_seq(q, kp, vp, table, L, scale, bs, "f16")
    ref = np.array(oracle.brute_force_seq(_nested(oracle.to_f64(q, "f16")),
                                          _nested(oracle.to_f64(k, "f16")),
                                          _nested(oracle.to_f64(v, "f16")), scale))
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_online_and_partitioned_forms_equal_two_pass(seed):
    rng = np.random.default_rng(200 + seed)
    hkv, g, d, bs = 2, [1, 4, 7, 2][seed], 8, 16
    L = [1, 100, 1000, 513][seed]
    q, k, v, kp, vp, table = _tiny_case(rng, L, hkv * g, hkv, d, bs, nb=128)
    scale = 1.0 / math.sqrt(d)
    two_pass = oracle.paged_decode_seq(q, kp, vp, table, L, scale, bs, "f16")
    qf, kf, vf = (oracle.to_f64(x, "f16") for x in (q, kp, vp))
    online = oracle.online_decode_seq(qf, kf, vf, table, L, scale, bs)
    for part in (16, 64, 512):
        parted = oracle.partitioned_decode_seq(qf, kf, vf, table, L, scale, bs, part)
        assert np.max(np.abs(parted - two_pass)) <= 1e-12
    assert np.max(np.abs(online - two_pass)) <= 1e-12


def test_attention_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    hkv, g, d, L = 2, 4, 16, 37
    q = rng.standard_normal((hkv * g, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    scale = 1.0 / math.sqrt(d)
    got = oracle.attention_contiguous(q, k, v, scale)
    tq = torch.from_numpy(q)[:, None, :]                                  # [Hq, 1, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)  # [Hq, L, d]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[:, 0, :]
    assert np.max(np.abs(got - ref.numpy())) <= 1e-12


# ------------------------------------------------------------------ invariants / closed forms

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    for scale in (1.0, 30.0, 300.0):
        s = rng.standard_normal((16, 257)) * scale
        w = oracle.softmax_weights(s)
        assert np.all(np.abs(w.sum(axis=-1) - 1.0) <= 1e-12)
        assert np.all(w >= 0)


def test_length_one_returns_that_tokens_value():
    rng = np.random.default_rng(4)
    hkv, g, d = 2, 7, 64
    q, k, v, kp, vp, table = _tiny_case(rng, 1, hkv * g, hkv, d, 16)
    out = oracle.paged_decode_seq(q, kp, vp, table, 1, 0.125, 16, "f16")
    vf = oracle.to_f64(v, "f16")
    for h in range(hkv * g):
        assert np.array_equal(out[h], vf[0, h // g])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(5)
    hkv, g, d, L = 2, 2, 8, 29
    q, k, v, kp, vp, table = _tiny_case(rng, L, hkv * g, hkv, d, 4)
    q[:] = 0
    out = oracle.paged_decode_seq(q, kp, vp, table, L, 0.35, 4, "f16")
    vf = oracle.to_f64(v, "f16")
    for h in range(hkv * g):
        assert np.max(np.abs(out[h] - vf[:, h // g].mean(axis=0))) <= 1e-14


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(6)
    hkv, g, d, L = 1, 3, 8, 21
    q, k, v, kp, vp, table = _tiny_case(rng, L, hkv * g, hkv, d, 16)
    c = np.float16(-1.75).view(np.uint16)
    for t in range(L):
        vp[table[t // 16], t % 16] = c
    out = oracle.paged_decode_seq(q, kp, vp, table, L, 0.35, 16, "f16")
    assert np.max(np.abs(out + 1.75)) <= 1e-14


def test_two_token_closed_form_fixes_scale_and_sign():
    # L = 2, V = [1, 0]: o = exp(a) / (exp(a) + exp(b)) with a, b = scale * q.k
    q = np.array([[0.5, -1.0, 2.0, 0.25]])
    k = np.array([[[1.0, 0.0, 0.5, 2.0]], [[-1.0, 1.0, 0.0, 0.5]]])
    v = np.array([[[1.0, 1.0, 1.0, 1.0]], [[0.0, 0.0, 0.0, 0.0]]])
    scale = 0.5
    a, b = scale * (q[0] @ k[0, 0]), scale * (q[0] @ k[1, 0])
    expect = 1.0 / (1.0 + math.exp(b - a))
    out = oracle.attention_contiguous(q, k, v, scale)
    assert abs(out[0, 0] - expect) <= 1e-15


def test_gqa_groups_are_contiguous():
    # KV head 0 holds V = -3, KV head 1 holds V = 5; q heads 0,1 -> -3 and 2,3 -> 5
    L, d = 5, 4
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, d))
    k = rng.standard_normal((L, 2, d))
    v = np.empty((L, 2, d))
    v[:, 0] = -3.0
    v[:, 1] = 5.0
    out = oracle.attention_contiguous(q, k, v, 0.5)
    assert np.allclose(out[:2], -3.0, atol=1e-14) and np.allclose(out[2:], 5.0, atol=1e-14)


def test_block_permutation_leaves_output_unchanged():
    rng = np.random.default_rng(9)
    hkv, g, d, L, bs, nb = 2, 4, 8, 75, 16, 32
    q, k, v, kp, vp, table = _tiny_case(rng, L, hkv * g, hkv, d, bs, nb=nb)
    out = oracle.paged_decode_seq(q, kp, vp, table, L, 0.3, bs, "f16")
    pi = rng.permutation(nb)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    out2 = oracle.paged_decode_seq(q, kp2, vp2, pi[table], L, 0.3, bs, "f16")
    assert np.array_equal(out, out2)


def test_empty_sequence_is_zero():
    q = np.zeros((4, 8), dtype=np.uint16)
    kp = np.zeros((2, 16, 2, 8), dtype=np.uint16)
    out = oracle.paged_decode_seq(q, kp, kp, [0], 0, 0.3, 16, "f16")
    assert np.array_equal(out, np.zeros((4, 8)))


# ------------------------------------------------------------------ paged == contiguous

class _BumpPool:
    """Blocks handed out in increasing id order, one table per request, a fresh block
    whenever a request's length is a multiple of the block size; every slot starts as
    a NaN bit pattern so a read of a slot nobody wrote would show."""

    def __init__(self, nb, bs, hkv, d):
        self.bs, self.next_block = bs, 0
        self.k = np.full((nb, bs, hkv, d), 0x7E00, np.uint16)
        self.v = np.full((nb, bs, hkv, d), 0x7E00, np.uint16)
        self.tables, self.lens = {}, {}

    def write(self, rid, kbits, vbits):
        n = self.lens.setdefault(rid, 0)
        table = self.tables.setdefault(rid, [])
        if n % self.bs == 0:
            table.append(self.next_block)
            self.next_block += 1
        self.k[table[-1], n % self.bs] = kbits
        self.v[table[-1], n % self.bs] = vbits
        self.lens[rid] = n + 1


@pytest.mark.parametrize("bs", [1, 2, 8, 16])
def test_reading_through_table_equals_one_array(bs):
    """Requests grown in a shuffled order, so their blocks interleave in the pool
    ("Why AI servers waste memory", "Proof it works": reading through the table gives
    what one flat array per request gives), for three requests of 19, 6 and 11 tokens
    at block sizes 1, 2, 8 and 16."""
    from workloads import round_to_bits
    rng = np.random.default_rng(900 + bs)
    hkv, d = 2, 4
    targets = {"r0": 19, "r1": 6, "r2": 11}
    schedule = [rid for rid, n in targets.items() for _ in range(n)]
    rng.shuffle(schedule)
    pool = _BumpPool(64, bs, hkv, d)
    flat = {rid: ([], []) for rid in targets}
    for rid in schedule:
        kb = round_to_bits(rng.standard_normal((hkv, d), dtype=np.float32), "f16")
        vb = round_to_bits(rng.standard_normal((hkv, d), dtype=np.float32), "f16")
        pool.write(rid, kb, vb)
        flat[rid][0].append(kb)
        flat[rid][1].append(vb)
    if bs <= 2:       # the requests' blocks are not contiguous runs
        assert any(t != list(range(t[0], t[0] + len(t))) for t in pool.tables.values())
    q = round_to_bits(rng.standard_normal((hkv * 2, d), dtype=np.float32), "f16")
    for rid, (ks, vs) in flat.items():
        kc = oracle.to_f64(np.stack(ks), "f16")
        vc = oracle.to_f64(np.stack(vs), "f16")
        contiguous = oracle.attention_contiguous(oracle.to_f64(q, "f16"), kc, vc, 0.5)
        paged = oracle.paged_decode_seq(q, pool.k, pool.v, pool.tables[rid], pool.lens[rid], 0.5, bs, "f16")
        assert np.max(np.abs(paged - contiguous)) <= 1e-15
        # gather returns exactly the rows written, in order
        assert np.array_equal(oracle.gather(pool.k, pool.tables[rid], pool.lens[rid], bs), np.stack(ks))


# ------------------------------------------------------------------ cache write

def test_scatter_writes_exact_bits_and_nothing_else():
    rng = np.random.default_rng(11)
    nb, bs, hkv, d, T = 16, 16, 2, 8, 20
    kp = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    slots = rng.choice(nb * bs, size=T, replace=False)
    key = rng.integers(0, 1 << 16, size=(T, hkv, d), dtype=np.uint16)
    val = rng.integers(0, 1 << 16, size=(T, hkv, d), dtype=np.uint16)
    oracle.scatter(kp, vp, key, val, slots, bs)
    flat_k = kp.reshape(nb * bs, hkv, d)
    flat_v = vp.reshape(nb * bs, hkv, d)
    assert np.array_equal(flat_k[slots], key) and np.array_equal(flat_v[slots], val)
    untouched = np.setdiff1d(np.arange(nb * bs), slots)
    assert np.array_equal(flat_k[untouched], k0.reshape(nb * bs, hkv, d)[untouched])
    assert np.array_equal(flat_v[untouched], v0.reshape(nb * bs, hkv, d)[untouched])


def test_scatter_then_decode_matches_appending_token():
    """A decode step = write position L-1, then attend over L tokens."""
    rng = np.random.default_rng(12)
    hkv, g, d, L, bs = 2, 2, 8, 18, 16
    q, k, v, kp, vp, table = _tiny_case(rng, L, hkv * g, hkv, d, bs)
    ref = oracle.paged_decode_seq(q, kp, vp, table, L, 0.3, bs, "f16")
    slot = table[(L - 1) // bs] * bs + (L - 1) % bs
    kp[table[(L - 1) // bs], (L - 1) % bs] = 0x7E00
    vp[table[(L - 1) // bs], (L - 1) % bs] = 0x7E00
    oracle.scatter(kp, vp, k[L - 1:L], v[L - 1:L], [slot], bs)
    out = oracle.paged_decode_seq(q, kp, vp, table, L, 0.3, bs, "f16")
    assert np.array_equal(out, ref)
