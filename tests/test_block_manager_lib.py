"""The library's C++ block manager against the oracle's (host logic, no GPU): the same
operations give the same tables, lengths, free list, reference counts, slots and
copy-on-write copies, bit for bit, and failing calls change nothing in either."""

import ctypes
import json
import os
import random

import numpy as np
import pytest

import oracle

pk = pytest.importorskip("paged_kv_cache_68_amd")
from paged_kv_cache_68_amd import _lib  # noqa: E402

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "block_manager_traces.json")))


def _state(m, rids):
    return (m.free_list(), [m.ref_count(b) for b in range(m.num_blocks)],
            {r: m.table(r) for r in rids}, {r: m.length(r) for r in rids})


def _same(lib_m, ora_m, rids):
    assert _state(lib_m, rids) == _state(ora_m, rids)


def test_hand_worked_example_trace():
    t = GOLDEN["hand_worked_example"]
    m = pk.BlockManager(t["num_blocks"], t["block_size"])
    ids = {"A": 1, "B": 2, "C": 3}
    for st in t["steps"][1:]:
        ev = st["event"]
        if ev[0] == "add":
            m.add_request(ids[ev[1]])
            m.append_batch([ids[ev[1]]], [ev[2]])
        elif ev[0] == "append":
            _, copies = m.append_batch([ids[ev[1]]], [ev[2]])
            assert copies.shape == (0, 3)
        elif ev[0] == "free":
            m.free(ids[ev[1]])
        assert {k: m.table(ids[k]) for k in st["tables"]} == st["tables"]
        assert {k: m.length(ids[k]) for k in st["tokens"]} == st["tokens"]
        assert m.free_list() == st["free"]
        assert m.num_free() == len(st["free"])


def test_prefix_sharing_trace():
    t = GOLDEN["prefix_sharing_example"]
    m = pk.BlockManager(t["num_blocks"], t["block_size"])
    ids = {"S1": 1, "S2": 2}
    for st in t["steps"]:
        ev = st["event"]
        copies = np.zeros((0, 3), dtype=np.int32)
        if ev[0] == "add":
            m.add_request(ids[ev[1]])
            _, copies = m.append_batch([ids[ev[1]]], [ev[2]])
        elif ev[0] == "fork":
            m.fork(ids[ev[1]], ids[ev[2]])
        elif ev[0] == "append":
            _, copies = m.append_batch([ids[ev[1]]], [ev[2]])
        assert copies.tolist() == st["copies"]
        assert {k: m.table(ids[k]) for k in st["tables"]} == st["tables"]
        assert [m.ref_count(b) for b in range(3)] == st["refs012"]
        assert m.free_list() == st["free"]


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_the_oracle(seed):
    rng = random.Random(100 + seed)
    B = rng.choice([1, 4, 16])
    nb = rng.choice([8, 24, 64])
    lib_m, ora_m = pk.BlockManager(nb, B), oracle.BlockManager(nb, B)
    live, next_rid = [], 0
    for _ in range(600):
        op = rng.choice(["add", "append", "append", "batch", "fork", "free"] if live else ["add"])
        if op == "add":
            lib_m.add_request(next_rid)
            ora_m.add_request(next_rid)
            live.append(next_rid)
            next_rid += 1
        elif op in ("append", "batch"):
            k = 1 if op == "append" else rng.randint(1, min(6, len(live)))
            rids = [rng.choice(live) for _ in range(k)]      # repeats allowed
            counts = [rng.randint(0, 2 * B + 1) for _ in rids]
            try:
                want = ora_m.append_batch(rids, counts)
            except oracle.OutOfBlocks:
                want = None
            if want is None:
                before = _state(lib_m, live)
                with pytest.raises(pk.OutOfBlocks):
                    lib_m.append_batch(rids, counts)
                assert _state(lib_m, live) == before
            else:
                slots, copies = lib_m.append_batch(rids, counts)
                assert slots.tolist() == want[0]
                assert [tuple(c) for c in copies.tolist()] == want[1]
        elif op == "fork":
            parent = rng.choice(live)
            lib_m.fork(parent, next_rid)
            ora_m.fork(parent, next_rid)
            live.append(next_rid)
            next_rid += 1
        else:
            rid = live.pop(rng.randrange(len(live)))
            lib_m.free(rid)
            ora_m.free(rid)
        _same(lib_m, ora_m, live)


def test_decode_step_batch_with_copy_on_write():
    """A 64-way fork of a prompt that ends mid-block, then one decode step for all 64:
    the first 63 copy the shared partial block, the last writes in place."""
    for m in (pk.BlockManager(400, 16), oracle.BlockManager(400, 16)):
        m.add_request(0)
        m.append_batch([0], [4096 + 7])
        for c in range(1, 64):
            m.fork(0, c)
        slots, copies = m.append_batch(list(range(64)))
        copies = [tuple(int(x) for x in c) for c in copies]
        assert len(copies) == 63
        assert all(c[2] == 7 for c in copies)                        # rows already written
        assert len({c[1] for c in copies}) == 63                      # distinct new blocks
        assert all(int(s) % 16 == 7 for s in slots)
        # every copy reads the old shared tail block, which the last request keeps
        assert {c[0] for c in copies} == {m.table(63)[-1]}
        assert int(slots[63]) // 16 == m.table(63)[-1]


def test_export_layout():
    m = pk.BlockManager(64, 16)
    for r, n in ((7, 40), (9, 1), (11, 0)):
        m.add_request(r)
        if n:
            m.append_batch([r], [n])
    tables, lens = m.export([9, 7, 11], 4)
    assert lens.tolist() == [1, 40, 0]
    assert tables.tolist() == [[3, -1, -1, -1], [0, 1, 2, -1], [-1, -1, -1, -1]]
    with pytest.raises(pk.PagedKVError):
        m.export([7], 2)                        # 3 blocks do not fit in 2 columns
    with pytest.raises(pk.PagedKVError):
        m.export([5], 4)                        # unknown request


def test_invalid_calls_change_nothing():
    m = pk.BlockManager(8, 4)
    m.add_request(1)
    m.append_batch([1], [5])
    before = _state(m, [1])
    for call in (lambda: m.add_request(1), lambda: m.fork(2, 3), lambda: m.fork(1, 1),
                 lambda: m.free(2), lambda: m.append_batch([1, 2], [1, 1]),
                 lambda: m.append_batch([1], [-1])):
        with pytest.raises(pk.PagedKVError):
            call()
        assert _state(m, [1]) == before
    # buffers that are too small are rejected before anything changes
    h = m.handle
    rids = np.array([1], dtype=np.int64)
    slots = np.empty(1, dtype=np.int64)
    copies = np.empty((1, 3), dtype=np.int32)
    nc = ctypes.c_int32()
    counts = np.array([3], dtype=np.int32)
    st = _lib.lib().kv_bm_append(h, rids.ctypes.data, counts.ctypes.data, 1, slots.ctypes.data, 2,
                                 copies.ctypes.data, 1, ctypes.byref(nc))
    assert st == _lib.KV_ERR_INVALID_ARG
    st = _lib.lib().kv_bm_append(h, rids.ctypes.data, None, 1, slots.ctypes.data, 1,
                                 copies.ctypes.data, 0, ctypes.byref(nc))
    assert st == _lib.KV_ERR_INVALID_ARG
    assert _state(m, [1]) == before
    assert _lib.lib().kv_bm_create(0, 4, ctypes.byref(ctypes.c_void_p())) == _lib.KV_ERR_INVALID_ARG
    assert _lib.lib().kv_bm_num_free(None) == -1


def test_copy_blocks_argument_checks():
    desc = pk.make_desc(2, 64, 2, 64, "f16")
    h = ctypes.c_void_p()
    fake = 1 << 40
    assert _lib.lib().kv_pool_create(ctypes.byref(desc), fake, pk.kv_pool_bytes(desc), ctypes.byref(h)) == 0
    lib = _lib.lib()
    assert lib.kv_copy_blocks(h, None, 0, None) == _lib.KV_OK
    assert lib.kv_copy_blocks(h, None, 3, None) == _lib.KV_ERR_INVALID_ARG
    assert lib.kv_copy_blocks(h, fake + 2, 3, None) == _lib.KV_ERR_INVALID_ARG
    assert lib.kv_copy_blocks(h, fake, -1, None) == _lib.KV_ERR_INVALID_ARG
    assert lib.kv_copy_blocks(None, fake, 1, None) == _lib.KV_ERR_INVALID_ARG
    lib.kv_pool_destroy(h)
