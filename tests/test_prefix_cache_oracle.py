"""Pins of the oracle's prefix cache: the FNV-1a test vectors of its hash, the behaviour
the pages state (block-aligned matches of a 2,407-token prefix, the hash chain, the
salt, warm reuse after finishing, uncached-first / cached-oldest-first reuse of free
blocks, fail-before-change), and invariants under random operations."""

import random

import pytest

from oracle.prefix_cache import FNV_OFFSET, OutOfBlocks, PrefixCache, block_hash, fnv1a64


def test_fnv1a_test_vectors():
    assert fnv1a64(b"") == FNV_OFFSET == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def _state(pc):
    return pc.snapshot()


def test_shared_prefix_of_2407_tokens_matches_150_blocks():
    """Sixteen requests with the same 2,407-token prompt: the first computes it, each
    later one finds 2,400 tokens (150 full blocks); the 7-token tails stay private."""
    rng = random.Random(0)
    prompt = [rng.randrange(151936) for _ in range(2407)]
    pc = PrefixCache(400, 16)
    assert pc.add_request(0, prompt) == 0
    pc.append(0, prompt)
    found = []
    for r in range(1, 16):
        found.append(pc.add_request(r, prompt))
        pc.append(r, prompt[found[-1]:])
    assert found == [2400] * 15
    shared = pc.table(0)[:150]
    assert all(pc.table(r)[:150] == shared for r in range(16))
    assert all(pc.ref_count(b) == 16 for b in shared)
    tails = {pc.table(r)[150] for r in range(16)}
    assert len(tails) == 16 and all(pc.ref_count(b) == 1 for b in tails)
    assert pc.num_blocks - pc.num_free() == 150 + 16
    pc.check_invariants()


def test_a_match_needs_the_whole_prefix():
    pc = PrefixCache(32, 4)
    a = [1, 2, 3, 4, 5, 6, 7, 8]
    pc.add_request("a", a)
    pc.append("a", a)
    b = [9, 2, 3, 4, 5, 6, 7, 8]          # second block identical, first block not
    assert pc.add_request("b", b) == 0
    c = [1, 2, 3, 4, 0, 6, 7, 8]          # first block identical
    assert pc.add_request("c", c) == 4


def test_salt_separates_tenants():
    pc = PrefixCache(32, 4)
    p = list(range(12))
    pc.add_request("x", p, salt=7)
    pc.append("x", p)
    assert pc.add_request("y", p, salt=8) == 0
    assert pc.add_request("z", p, salt=7) == 12
    assert block_hash(0, p[:4], 7, first=True) != block_hash(0, p[:4], 8, first=True)
    assert block_hash(5, p[:4], 7) == block_hash(5, p[:4], 8)      # only the first block


def test_finished_prefix_stays_findable_until_evicted():
    pc = PrefixCache(8, 4)
    p = list(range(10))                    # blocks: 2 full (cached) + 1 partial
    pc.add_request(0, p)
    pc.append(0, p)
    full = pc.table(0)[:2]
    pc.free_request(0)
    assert all(pc.ref_count(b) == 0 and pc.block_hash_of(b) is not None for b in full)
    # hash-less partial block at the head, cached ones at the tail, last-walked first
    q = pc.free_queue()
    assert q[0] not in full and q[-2:] == [full[1], full[0]]
    assert pc.add_request(1, p) == 8        # warm: found, nothing computed
    assert all(b not in pc.free_queue() and pc.ref_count(b) == 1 for b in full)
    pc.check_invariants()


def test_uncached_blocks_are_reused_first_and_cached_ones_oldest_first():
    pc = PrefixCache(6, 2)
    pa, pb = [1, 1, 2, 2], [3, 3, 4, 4]
    for rid, p in (("a", pa), ("b", pb)):
        pc.add_request(rid, p)
        pc.append(rid, p)
    a0, a1 = pc.table("a")
    pc.free_request("a")                    # a's cached blocks join the tail first,
    pc.free_request("b")                    # each request's last block first
    assert pc.free_queue()[:2] == [4, 5]    # the never-used (hash-less) blocks lead
    assert pc.free_queue()[2:4] == [a1, a0] and pc.num_cached() == 4
    pc.add_request("c", [9])
    pc.append("c", [9, 9, 9, 9, 9])         # 3 blocks: the 2 uncached ones, then a's tail block
    assert pc.table("c") == [4, 5, a1] and pc.block_hash_of(a1) is None   # evicted; holds c's partial tail
    assert pc.num_cached() == 4 - 1 + 2     # one evicted, c's two full blocks cached
    assert pc.add_request("d", pa) == 2     # a's head block survives, its tail does not
    assert pc.add_request("e", pb) == 4     # b's prefix is still there


def test_append_without_enough_blocks_changes_nothing():
    pc = PrefixCache(3, 4)
    pc.add_request(0, [])
    pc.append(0, list(range(8)))
    before = _state(pc)
    with pytest.raises(OutOfBlocks):
        pc.append(0, list(range(8)))        # needs 2 blocks, 1 free
    assert _state(pc) == before


@pytest.mark.parametrize("seed", range(4))
def test_random_operations_keep_invariants(seed):
    rng = random.Random(seed)
    B = rng.choice([2, 4, 16])
    pc = PrefixCache(40, B)
    stems = [[rng.randrange(50) for _ in range(rng.randrange(0, 5 * B))] for _ in range(4)]
    live, nxt = [], 0
    for _ in range(300):
        op = rng.choice(["add", "append", "free"] if live else ["add"])
        if op == "add":
            prompt = rng.choice(stems) + [rng.randrange(50) for _ in range(rng.randrange(0, 2 * B))]
            found = pc.add_request(nxt, prompt, salt=rng.choice([0, 0, 1]))
            assert found % B == 0 and found <= len(prompt)
            try:
                pc.append(nxt, prompt[found:])
            except OutOfBlocks:
                pass
            live.append(nxt)
            nxt += 1
        elif op == "append":
            rid = rng.choice(live)
            before = _state(pc)
            try:
                pc.append(rid, [rng.randrange(50) for _ in range(rng.randrange(1, 3 * B))])
            except OutOfBlocks:
                assert _state(pc) == before
        else:
            pc.free_request(live.pop(rng.randrange(len(live))))
        pc.check_invariants()


def test_decode_step_equals_one_token_appends_in_order():
    """append_step is appending one token to each request in turn; a step that needs more
    blocks than are free, or names a request twice, changes nothing."""
    import copy
    rng = random.Random(7)
    pc = PrefixCache(12, 4)
    for rid, n in enumerate([4, 6, 3, 8]):       # lengths 4 and 8 end on a full block
        pc.add_request(rid, [rng.randrange(9) for _ in range(n)])
        pc.append(rid, [rng.randrange(9) for _ in range(n)])
    ref = copy.deepcopy(pc)
    toks = [11, 12, 13, 14]
    slots = pc.append_step([3, 0, 2, 1], toks)
    want = [ref.append(r, [t])[0] for r, t in zip([3, 0, 2, 1], toks)]
    assert slots == want
    assert pc.snapshot() == ref.snapshot()
    with pytest.raises(ValueError):
        pc.append_step([0, 0], [1, 2])
    with pytest.raises(ValueError):
        pc.append_step([9], [1])
    # drain the free list, then a step needing a block fails as a whole
    while pc.num_free():
        pc.append(0, [1] * (4 - pc.length(0) % 4))
    before = pc.snapshot()
    need_block = [r for r in pc.requests() if pc.length(r) % 4 == 0]
    assert need_block
    with pytest.raises(OutOfBlocks):
        pc.append_step(sorted(pc.requests()), [5] * len(pc.requests()))
    assert pc.snapshot() == before
