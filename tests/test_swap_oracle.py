"""Pins of the oracle's swap (moving requests between the device block manager and a
host one, and the block copies that go with it) against what the pages fix: the
victim's blocks go to the host pool and its GPU blocks return to the free list; on
resume the blocks come back and decoding goes on with nothing lost ("PagedAttention
and Virtual Memory Management", section 6, swapping policy); plus a worked example
derived by hand from the free-list rules, all-or-nothing failures and random traces in
which every request reads back what it wrote after any number of swaps."""

import random

import numpy as np
import pytest

import oracle
from oracle import BlockManager, OutOfBlocks, move_requests


def _state(m):
    return m.snapshot()


def test_worked_example_by_hand():
    """Device: 8 blocks of 4 slots; request 0 holds 10 tokens (blocks 0 1 2), request 1
    5 tokens (3 4), request 2 is a fork of 0.  Swapping 0 and 2 out copies blocks 0 1 2
    once each to host blocks 0 1 2 (counts 2 there); on the device the three blocks
    reach zero while request 2 is dropped and join the back of the free list."""
    dev, host = BlockManager(8, 4), BlockManager(6, 4)
    for rid, n in ((0, 10), (1, 5)):
        dev.add_request(rid)
        dev.append_batch([rid], [n])
    dev.fork(0, 2)
    assert dev.table(0) == [0, 1, 2] and dev.table(1) == [3, 4]
    pairs = move_requests(dev, host, [0, 2])
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    assert dev.free_list() == [5, 6, 7, 0, 1, 2]
    assert dev.ref_counts()[:5] == [0, 0, 0, 1, 1]
    assert host.table(0) == host.table(2) == [0, 1, 2] and host.length(2) == 10
    assert host.ref_counts() == [2, 2, 2, 0, 0, 0] and host.free_list() == [3, 4, 5]
    # request 1 grows into the freed blocks: 5 + 7 = 12 tokens take blocks 5 then 6
    dev.append_batch([1], [7])
    assert dev.table(1) == [3, 4, 5]
    # swap back in: new device blocks from the front of the free list (6, 7, 0)
    pairs = move_requests(host, dev, [2, 0])
    assert pairs == [(0, 6), (1, 7), (2, 0)]
    assert dev.table(0) == dev.table(2) == [6, 7, 0] and dev.length(0) == 10
    assert host.free_list() == [3, 4, 5, 0, 1, 2]
    dev.check_invariants()
    host.check_invariants()


def test_partial_swap_of_a_shared_prefix():
    """Only the child leaves: its three blocks are copied, but on the device they stay
    (the parent still names them) with their count back to one."""
    dev, host = BlockManager(8, 4), BlockManager(8, 4)
    dev.add_request(0)
    dev.append_batch([0], [9])
    dev.fork(0, 1)
    free_before = dev.free_list()
    pairs = move_requests(dev, host, [1])
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    assert dev.free_list() == free_before and dev.ref_counts()[:3] == [1, 1, 1]
    assert host.ref_counts()[:3] == [1, 1, 1]


def test_failures_change_nothing():
    dev, host = BlockManager(8, 4), BlockManager(2, 4)
    for rid in (0, 1):
        dev.add_request(rid)
        dev.append_batch([rid], [9])
    host.add_request(5)
    before = (_state(dev), _state(host))
    with pytest.raises(OutOfBlocks):
        move_requests(dev, host, [0])          # 3 blocks, host has 2 free
    with pytest.raises(KeyError):
        move_requests(dev, host, [7])          # unknown id
    with pytest.raises(KeyError):
        move_requests(dev, host, [1, 1])       # repeated id
    dev.add_request(5)
    with pytest.raises(KeyError):
        move_requests(dev, host, [5])          # exists in the destination
    dev.free(5)
    assert (_state(dev), _state(host)) == before


def test_swap_blocks_copies_whole_blocks_bit_for_bit():
    rng = np.random.default_rng(0)
    src = rng.integers(0, 2**16, (6, 4, 2, 3), dtype=np.uint16)
    dst = rng.integers(0, 2**16, (5, 4, 2, 3), dtype=np.uint16)
    want = dst.copy()
    pairs = [(4, 0), (1, 3), (4, 2)]
    oracle.swap_blocks(src, dst, pairs)
    for s, d in pairs:                         # element by element
        for t in range(4):
            for h in range(2):
                for e in range(3):
                    want[d, t, h, e] = src[s, t, h, e]
    assert np.array_equal(dst, want)
    back = np.zeros_like(src)
    oracle.swap_blocks(dst, back, [(d, s) for s, d in pairs[:2]])
    assert np.array_equal(back[[4, 1]], src[[4, 1]])


def _read(m, store, rid):
    B = m.block_size
    t = m.table(rid)
    return [int(store[t[p // B], p % B]) for p in range(m.length(rid))]


@pytest.mark.parametrize("seed", range(5))
def test_random_swaps_lose_nothing(seed):
    """500 operations over a device and a host manager (add, append, fork, free, swap
    out, swap in), with token ids standing in for the K/V rows: the copies the swaps
    return, applied to the two stores, keep every request reading back what it wrote."""
    rng = random.Random(seed)
    B = 4
    dev, host = BlockManager(20, B), BlockManager(24, B)
    dstore = np.full((20, B), -1, dtype=np.int64)
    hstore = np.full((24, B), -1, dtype=np.int64)
    where, hist = {}, {}
    nxt_rid, nxt_tok = 0, 0
    for _ in range(500):
        on_dev = [r for r in where if where[r] == "dev"]
        on_host = [r for r in where if where[r] == "host"]
        op = rng.choice(["add", "append", "append", "fork", "free", "out", "in"])
        if op == "add":
            dev.add_request(nxt_rid)
            where[nxt_rid], hist[nxt_rid] = "dev", []
            nxt_rid += 1
        elif op == "append" and on_dev:
            rid = rng.choice(on_dev)
            try:
                slots, copies = dev.append_batch([rid], [rng.randint(1, 6)])
            except OutOfBlocks:
                continue
            oracle.copy_blocks(dstore, copies)
            for s in slots:
                dstore[s // B, s % B] = nxt_tok
                hist[rid].append(nxt_tok)
                nxt_tok += 1
        elif op == "fork" and on_dev:
            parent = rng.choice(on_dev)
            dev.fork(parent, nxt_rid)
            where[nxt_rid], hist[nxt_rid] = "dev", list(hist[parent])
            nxt_rid += 1
        elif op == "free" and where:
            rid = rng.choice(list(where))
            (dev if where[rid] == "dev" else host).free(rid)
            del where[rid], hist[rid]
        elif op in ("out", "in"):
            pool = on_dev if op == "out" else on_host
            if not pool:
                continue
            rids = rng.sample(pool, rng.randint(1, min(3, len(pool))))
            src, dst = (dev, host) if op == "out" else (host, dev)
            ss, ds = (dstore, hstore) if op == "out" else (hstore, dstore)
            before = (_state(src), _state(dst))
            try:
                pairs = move_requests(src, dst, rids)
            except OutOfBlocks:
                assert (_state(src), _state(dst)) == before
                continue
            oracle.swap_blocks(ss, ds, pairs)
            for r in rids:
                where[r] = "host" if op == "out" else "dev"
        dev.check_invariants()
        host.check_invariants()
        for rid, w in where.items():
            m, st = (dev, dstore) if w == "dev" else (host, hstore)
            assert _read(m, st, rid) == hist[rid], rid
