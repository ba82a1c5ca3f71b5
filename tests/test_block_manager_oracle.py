"""Pins of the oracle's block manager against what the pages print and fix.

The traces come from tests/golden/block_manager_traces.json (each entry cites its page
and section).  The rest are invariants the pages state: no block lost, double-booked
or listed twice; reference counts equal the tables; every request reads back what it
wrote; a copy-on-write append that cannot get a block changes nothing; forking k
streams adds k - 1 references; paged reads equal one flat array.
"""

import json
import os
import random

import numpy as np
import pytest

import oracle
from oracle import BlockManager, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_manager_traces.json")
TRACES = json.load(open(GOLDEN))


def _apply(mgr, event):
    kind = event[0]
    if kind == "start":
        return []
    if kind == "add":
        mgr.add_request(event[1])
        return mgr.append_batch([event[1]], [event[2]])[1]
    if kind == "append":
        return mgr.append_batch([event[1]], [event[2]])[1]
    if kind == "free":
        mgr.free(event[1])
        return []
    if kind == "fork":
        mgr.fork(event[1], event[2])
        return []
    raise ValueError(kind)


def test_hand_worked_example_trace():
    t = TRACES["hand_worked_example"]
    mgr = BlockManager(t["num_blocks"], t["block_size"])
    for st in t["steps"]:
        copies = _apply(mgr, st["event"])
        assert copies == []
        assert {r: mgr.length(r) for r in mgr.requests()} == st["tokens"], st["step"]
        assert {r: mgr.table(r) for r in mgr.requests()} == st["tables"], st["step"]
        assert mgr.free_list() == st["free"], st["step"]
        assert mgr.wasted_slots() == st["wasted"], st["step"]
        mgr.check_invariants()


def test_prefix_sharing_trace():
    t = TRACES["prefix_sharing_example"]
    mgr = BlockManager(t["num_blocks"], t["block_size"])
    for st in t["steps"]:
        copies = _apply(mgr, st["event"])
        assert [list(c) for c in copies] == st["copies"]
        assert {r: mgr.table(r) for r in mgr.requests()} == st["tables"]
        assert mgr.ref_counts()[:3] == st["refs012"]
        assert mgr.free_list() == st["free"]
        mgr.check_invariants()


def test_parallel_sampling_shares_full_prompt_blocks():
    t = TRACES["parallel_sampling_example"]
    B, n = t["block_size"], t["prompt"]
    mgr = BlockManager(128, B)
    mgr.add_request("parent")
    mgr.append_batch(["parent"], [n])
    prompt = mgr.table("parent")
    mgr.fork("parent", "branch")          # two streams: the parent and one fork
    assert [mgr.ref_count(b) for b in prompt] == [2, 2]
    slots, copies = mgr.append_batch(["parent", "branch"])
    assert copies == []                   # the prompt's last block is full: nothing copied
    new_a, new_b = slots[0] // B, slots[1] // B
    assert new_a != new_b and new_a not in prompt and new_b not in prompt
    assert mgr.ref_count(new_a) == mgr.ref_count(new_b) == 1
    assert [mgr.ref_count(b) for b in prompt] == [2, 2]
    assert slots[0] % B == slots[1] % B == 0      # position 32 is slot 0 of a new block
    mgr.check_invariants()


@pytest.mark.parametrize("k", [2, 3, 8])
def test_fork_k_streams_adds_k_minus_one(k):
    mgr = BlockManager(64, 16)
    mgr.add_request(0)
    mgr.append_batch([0], [40])
    before = {b: mgr.ref_count(b) for b in mgr.table(0)}
    for c in range(1, k):
        mgr.fork(0, c)
    assert all(mgr.ref_count(b) == before[b] + (k - 1) for b in before)
    assert mgr.num_free() == 64 - 3       # forking allocates nothing
    mgr.check_invariants()


def _state(mgr):
    return mgr.snapshot()


def test_cow_append_without_a_free_block_changes_nothing():
    mgr = BlockManager(2, 4)
    mgr.add_request("a")
    mgr.append_batch(["a"], [6])          # blocks 0, 1: the pool is full
    mgr.fork("a", "b")
    before = _state(mgr)
    with pytest.raises(OutOfBlocks):
        mgr.append("a")                   # needs a copy of shared block 1
    assert _state(mgr) == before


def test_batch_is_all_or_nothing():
    mgr = BlockManager(3, 4)
    for r in "xyz":
        mgr.add_request(r)
    before = _state(mgr)
    with pytest.raises(OutOfBlocks):
        mgr.append_batch(["x", "y", "z", "x"], [4, 4, 4, 1])    # the fourth block is missing
    assert _state(mgr) == before
    slots, _ = mgr.append_batch(["x", "y", "z"], [4, 4, 4])
    assert slots == list(range(12))


def _check_read_back(mgr, store, history):
    for rid, hist in history.items():
        t = mgr.table(rid)
        got = [int(store[t[p // mgr.block_size], p % mgr.block_size]) for p in range(mgr.length(rid))]
        assert got == hist, rid


@pytest.mark.parametrize("seed", range(5))
def test_random_operations_keep_invariants_and_contents(seed):
    """400 mixed operations (add, append, fork, free); after each: invariants hold and
    every request reads back exactly the tokens it (or its ancestors) wrote."""
    rng = random.Random(seed)
    B, nb = 4, 24
    mgr = BlockManager(nb, B)
    store = np.full((nb, B), -1, dtype=np.int64)     # token ids stand in for K/V rows
    history = {}
    next_rid, next_tok = 0, 0
    for _ in range(400):
        live = list(history)
        op = rng.choice(["add", "append", "append", "append", "fork", "free"] if live else ["add"])
        if op == "add":
            mgr.add_request(next_rid)
            history[next_rid] = []
            next_rid += 1
        elif op == "append":
            rid = rng.choice(live)
            n = rng.randint(1, 6)
            before = _state(mgr)
            try:
                slots, copies = mgr.append_batch([rid], [n])
            except OutOfBlocks:
                assert _state(mgr) == before
                continue
            oracle.copy_blocks(store, copies)
            for s in slots:
                store[s // B, s % B] = next_tok
                history[rid].append(next_tok)
                next_tok += 1
        elif op == "fork":
            parent = rng.choice(live)
            mgr.fork(parent, next_rid)
            history[next_rid] = list(history[parent])
            next_rid += 1
        else:
            rid = rng.choice(live)
            mgr.free(rid)
            del history[rid]
        mgr.check_invariants()
        _check_read_back(mgr, store, history)


@pytest.mark.parametrize("block_size", [1, 3, 8, 16])
def test_reading_through_the_managers_tables_equals_one_flat_array(block_size):
    """Four requests (5, 17, 12 and 30 tokens) whose appends come in a shuffled order,
    so their blocks interleave in the pool; attention read through each table equals
    attention over the request's flat arrays ("Why AI servers waste memory", "Proof it
    works")."""
    rng = np.random.default_rng(4100 + block_size)
    d = 4
    mgr = BlockManager(80, block_size)
    kp = np.zeros((80, block_size, 1, d))
    vp = np.zeros((80, block_size, 1, d))
    targets = {10: 5, 11: 17, 12: 12, 13: 30}
    flat = {rid: ([], []) for rid in targets}
    for rid in targets:
        mgr.add_request(rid)
    order = np.repeat(list(targets), list(targets.values()))
    rng.shuffle(order)
    for rid in order.tolist():
        k, v = rng.standard_normal((1, d)), rng.standard_normal((1, d))
        (slot,), copies = mgr.append_batch([rid])
        assert copies == []
        kp[slot // block_size, slot % block_size] = k
        vp[slot // block_size, slot % block_size] = v
        flat[rid][0].append(k)
        flat[rid][1].append(v)
    mgr.check_invariants()
    q = rng.standard_normal((1, d))
    for rid, (ks, vs) in flat.items():
        table, L = mgr.table(rid), mgr.length(rid)
        assert L == targets[rid]
        paged = oracle.attention_contiguous(q, oracle.gather(kp, table, L, block_size),
                                            oracle.gather(vp, table, L, block_size), 0.5)
        ref = oracle.attention_contiguous(q, np.stack(ks), np.stack(vs), 0.5)
        assert np.allclose(paged, ref, rtol=0, atol=1e-12)
