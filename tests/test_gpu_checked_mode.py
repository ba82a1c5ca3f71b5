"""Checked mode (PAGEDKV_CHECK=1): bad block ids, lengths, slots, duplicate slots and
query offsets are caught on the device before anything is written, and valid inputs give
the same bits as the fast path."""

import math

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_68_amd as pk  # noqa: E402


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _setup(nb=40, hq=8, hkv=2, d=64):
    pool = pk.KVPool(1, nb, hkv, d, "f16")
    pool.memory.view(torch.int16).random_(-15000, 15000)
    lens = torch.tensor([5, 40, 100], dtype=torch.int32, device="cuda")
    tables = torch.tensor([[0, -1, -1, -1, -1, -1, -1], [1, 2, 3, -1, -1, -1, -1],
                           [4, 5, 6, 7, 8, 9, 10]], dtype=torch.int32, device="cuda")
    q = torch.randn(3, hq, d, device="cuda").half()
    return pool, lens, tables, q


def test_valid_inputs_same_bits(monkeypatch):
    _say("checked mode: valid decode and cache write")
    pool, lens, tables, q = _setup()
    out0 = pk.paged_attention_decode(pool, 0, torch.empty_like(q), q, tables, lens)
    monkeypatch.setenv("PAGEDKV_CHECK", "1")
    out1 = pk.paged_attention_decode(pool, 0, torch.empty_like(q), q, tables, lens)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    key = torch.randn(3, 2, 64, device="cuda").half()
    pk.reshape_and_cache(pool, 0, key, key, torch.tensor([-1, 5, 639], dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("case", ["bad_block", "negative_block", "long_length", "negative_length"])
def test_bad_tables_are_rejected_before_any_write(case, monkeypatch):
    _say(f"checked mode: {case}")
    pool, lens, tables, q = _setup()
    if case == "bad_block":
        tables[2, 6] = 40
    elif case == "negative_block":
        tables[1, 2] = -3
    elif case == "long_length":
        lens[0] = 7 * 16 + 1
    else:
        lens[1] = -2
    monkeypatch.setenv("PAGEDKV_CHECK", "1")
    out = torch.full_like(q, 3.0)
    with pytest.raises(pk.PagedKVError):
        pk.paged_attention_decode(pool, 0, out, q, tables, lens)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    qs = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    with pytest.raises(pk.PagedKVError):
        pk.paged_attention_prefill(pool, 0, out, q, qs, 1, tables, lens)
    # an unused entry past the length is not checked: padding stays legal
    if case == "bad_block":
        lens[2] = 96
        pk.paged_attention_decode(pool, 0, out, q, tables, lens)


@pytest.mark.parametrize("slots", [[0, 640, 3], [7, 9, 7]])
def test_bad_slots_are_rejected_before_any_write(slots, monkeypatch):
    _say(f"checked mode: slots {slots}")
    pool, _, _, _ = _setup()
    before = pool.memory.clone()
    monkeypatch.setenv("PAGEDKV_CHECK", "1")
    key = torch.randn(3, 2, 64, device="cuda").half()
    with pytest.raises(pk.PagedKVError):
        pk.reshape_and_cache(pool, 0, key, key, torch.tensor(slots, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(pool.memory, before)


def test_bad_query_offsets_are_rejected(monkeypatch):
    _say("checked mode: query offsets")
    pool, lens, tables, q = _setup()
    monkeypatch.setenv("PAGEDKV_CHECK", "1")
    out = torch.full_like(q, 3.0)
    monkeypatch.setenv("PAGEDKV_PREFILL_SPLITS", "2")      # the split entry point splits
    ws = pk.alloc_prefill_workspace(pool, 3, q.shape[1], q.shape[0], 2, tables.shape[1])
    assert ws is not None
    for qs in ([0, 2, 1, 3], [0, 3, 3, 3]):
        qs_d = torch.tensor(qs, dtype=torch.int32, device="cuda")
        with pytest.raises(pk.PagedKVError):
            pk.paged_attention_prefill(pool, 0, out, q, qs_d, 2, tables, lens, scale=1 / math.sqrt(64))
        with pytest.raises(pk.PagedKVError):
            pk.paged_attention_prefill_split(pool, 0, out, q, qs_d, 2, tables, lens,
                                             scale=1 / math.sqrt(64), workspace=ws)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def test_append_with_shared_last_slot_is_rejected(monkeypatch):
    """Two sequences whose position L - 1 falls in the same slot (a shared block before
    its copy) are rejected by the decode-with-append calls before anything is written;
    distinct slots pass and give the fast path's bits."""
    _say("checked mode: decode_append with a shared last slot")
    pool, lens, tables, q = _setup()
    key = torch.randn(3, 2, 64, device="cuda").half()
    val = torch.randn(3, 2, 64, device="cuda").half()
    ref_pool, _, _, _ = _setup()
    ref_pool.memory.copy_(pool.memory)
    out0 = pk.paged_attention_decode_append(ref_pool, 0, torch.empty_like(q), q, key, val, tables, lens)
    monkeypatch.setenv("PAGEDKV_CHECK", "1")
    out1 = pk.paged_attention_decode_append(pool, 0, torch.empty_like(q), q, key, val, tables, lens)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(pool.memory, ref_pool.memory)
    # sequence 0 (length 5, block 0) and sequence 2 cut to length 5 over the same block 0
    lens2 = lens.clone()
    lens2[2] = 5
    tables2 = tables.clone()
    tables2[2, 0] = 0
    before = pool.memory.clone()
    out = torch.full_like(q, 3.0)
    with pytest.raises(pk.PagedKVError):
        pk.paged_attention_decode_append(pool, 0, out, q, key, val, tables2, lens2)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    assert torch.equal(pool.memory, before)
