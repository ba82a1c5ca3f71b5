"""Plain reference model of the block manager that produces block tables, slots and
copy-on-write copies -- TEST INFRASTRUCTURE ONLY (tests/ may import it; the product
path never does, and this module imports nothing from it).

The model is written from the rules the pages state, as transitions of one immutable
state value: every operation computes the next state from the current one and the
manager adopts it only when the whole operation succeeded, so a call that fails has
changed nothing by construction.

Rules used (page title, then the section):

[P2] "Why AI servers waste memory, and how paging fixes it"
  - "The idea: a block table": the pool is cut into blocks once; a request owns a list
    of physical blocks in logical order; position p lives in entry p // B, slot p % B;
    a request that fills its last block gets one more from the free blocks; a finished
    request gives its blocks back.
  - "A hand-worked example": the next block handed out is the one at the front of the
    free list, and blocks given back go to its end; "wasted" counts allocated slots
    that hold no token.
  - "The real implementation": before an append changes anything it checks that a
    block is available when one is needed, and fails otherwise; a block returns to the
    free list only when no request names it any more.
  - "Sharing a prefix with copy-on-write": a fork starts with the parent's table, each
    block gaining a user; a write into a shared block that still has room first moves
    the writer to a private copy of it.
[P3] "PagedAttention and Virtual Memory Management", section 5: the reference count
  R[p] is the number of logical blocks mapped to p; forking k streams adds k - 1 to
  each shared block; a write at slot o of a block with R[p] = 1 happens in place, with
  R[p] > 1 a new block is allocated, the o token vectors already in p are copied to it,
  R[p] drops by one and the table entry is repointed.

Data model (ours):
  - a request is (blocks, length);
  - a block's reference count is not stored: it is the number of request tables that
    name it, counted when needed, so counts can never disagree with the tables;
  - the free blocks carry a ticket (a sequence number); the free block with the
    smallest ticket is handed out first, and a block given back gets the next,
    largest, ticket.  Tickets make "front of the list" and "back of the list" plain
    comparisons.

Readings:
  - Fork follows P2: one child per call, one more user per block, and the parent keeps
    running; P3's k-way fork is the parent plus k - 1 such forks.
  - The copy made on a write into a shared block moves the o = length mod B rows the
    block already holds (P3 section 5, case 2) and is reported as (src, dst, rows); a
    copy of the whole block (P2) leaves every readable value the same, since rows past
    o are written before they are read.
  - A batch of appends (one decode step, or a prompt) is applied token by token in the
    order given and adopted only if every token found its block.
  - A finished request's blocks that nobody names any more are given back in table
    order, front to back (P2's example returns a request's blocks in that order).

Swap (``move_requests``), from [P3] section 6 (swapping policy: a second pool of blocks
in host memory receives the victim's blocks, its GPU blocks return to the free list,
and on resume the blocks come back) and [P4] "2.1 PagedAttention" (preemption by
swapping the cache to CPU memory and back).  Readings:
  - The host pool is a second manager of the same kind; a swap moves a set of requests
    from one manager to the other.
  - Each distinct block the moved tables name gets one new block in the destination,
    handed out in first-seen order (requests in the order given, tables front to
    back); blocks the moved requests share stay shared there.  The (src, dst) pairs are
    the copies to make.
  - The source then drops the moved requests one after another as a finished request
    is dropped.  A block that a request left behind still names keeps its contents and
    its other users; its copy goes along anyway.
  - All or nothing: unknown or repeated ids, an id the destination already has, or too
    few free destination blocks change nothing.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Tuple

__all__ = ["OutOfBlocks", "BlockManager", "move_requests"]


class OutOfBlocks(Exception):
    """No free block for an append (or a swap) that needs one; nothing was changed."""


@dataclass(frozen=True)
class Request:
    blocks: Tuple[int, ...]   # physical blocks, logical order
    length: int               # tokens stored


@dataclass(frozen=True)
class State:
    """Everything the manager knows, as one value."""
    block_size: int
    num_blocks: int
    requests: Tuple[Tuple[object, Request], ...]   # (id, request), in the order added
    tickets: Tuple[Tuple[int, int], ...]           # (block, ticket) of every free block
    next_ticket: int

    # ---------------------------------------------------------------- queries
    def request(self, rid) -> Request:
        for r, req in self.requests:
            if r == rid:
                return req
        raise KeyError(f"unknown request {rid!r}")

    def has(self, rid) -> bool:
        return any(r == rid for r, _ in self.requests)

    def users(self, block: int) -> int:
        """Reference count: how many request tables name the block."""
        return sum(req.blocks.count(block) for _, req in self.requests)

    def free_in_order(self):
        return [b for b, _ in sorted(self.tickets, key=lambda bt: bt[1])]

    # ---------------------------------------------------------------- transitions
    def with_request(self, rid, req: Request) -> "State":
        rest = tuple((r, q) for r, q in self.requests if r != rid)
        if len(rest) == len(self.requests):
            return replace(self, requests=self.requests + ((rid, req),))
        return replace(self, requests=tuple((r, req if r == rid else q) for r, q in self.requests))

    def without_request(self, rid) -> "State":
        return replace(self, requests=tuple((r, q) for r, q in self.requests if r != rid))

    def take_block(self) -> Tuple["State", int]:
        """Hand out the free block at the front (smallest ticket)."""
        if not self.tickets:
            raise OutOfBlocks("no free block")
        block = min(self.tickets, key=lambda bt: bt[1])[0]
        return replace(self, tickets=tuple(bt for bt in self.tickets if bt[0] != block)), block

    def give_back(self, blocks) -> "State":
        """Put blocks nobody names at the back of the free list, in the order given."""
        tickets, t = list(self.tickets), self.next_ticket
        for b in blocks:
            tickets.append((b, t))
            t += 1
        return replace(self, tickets=tuple(tickets), next_ticket=t)


def initial_state(num_blocks: int, block_size: int) -> State:
    return State(block_size, num_blocks, (), tuple((b, b) for b in range(num_blocks)), num_blocks)


def add_request(s: State, rid) -> State:
    if s.has(rid):
        raise KeyError(f"request {rid!r} exists")
    return s.with_request(rid, Request((), 0))


def fork(s: State, parent, child) -> State:
    """The child starts with the parent's table and length: every block gains a user,
    nothing is allocated or copied."""
    src = s.request(parent)
    if s.has(child):
        raise KeyError(f"request {child!r} exists")
    return s.with_request(child, src)


def drop(s: State, rid) -> State:
    """A finished request: its blocks lose a user; those left with none are given back,
    front of the table first."""
    blocks = s.request(rid).blocks
    s = s.without_request(rid)
    return s.give_back([b for b in blocks if s.users(b) == 0])


def append_token(s: State, rid):
    """Next state after storing one more token of ``rid``, the token's slot, and the
    copy-on-write copy it needs (None or (src, dst, rows))."""
    B = s.block_size
    req = s.request(rid)
    n = req.length
    slot_in_block = n % B
    blocks, copy = req.blocks, None
    if slot_in_block == 0:                         # past the last block (or no block yet)
        s, fresh = s.take_block()
        blocks = blocks + (fresh,)
    elif s.users(blocks[-1]) > 1:                  # shared block with room: private copy
        s, fresh = s.take_block()
        copy = (blocks[-1], fresh, slot_in_block)
        blocks = blocks[:-1] + (fresh,)
    s = s.with_request(rid, Request(blocks, n + 1))
    return s, blocks[n // B] * B + slot_in_block, copy


class BlockManager:
    """Holds the current ``State``; each call adopts the next one only on success."""

    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.state = initial_state(num_blocks, block_size)

    # ------------------------------------------------------------ requests
    def add_request(self, rid) -> None:
        self.state = add_request(self.state, rid)

    def fork(self, parent, child) -> None:
        self.state = fork(self.state, parent, child)

    def free(self, rid) -> None:
        self.state = drop(self.state, rid)

    def append(self, rid):
        """Reserve the slot of the request's next token: (slot, copy), slot = physical
        block * B + offset, copy None or (src, dst, rows) -- the first `rows` token rows
        of src go to dst before the token is written there."""
        s, slot, copy = append_token(self.state, rid)
        self.state = s
        return slot, copy

    def append_batch(self, rids, counts=None):
        """counts[i] tokens for rids[i], request after request.  Returns (slots, copies)
        in that order; on OutOfBlocks the manager keeps its state before the call."""
        counts = [1] * len(rids) if counts is None else list(counts)
        if len(counts) != len(rids):
            raise ValueError("rids and counts differ in length")
        s, slots, copies = self.state, [], []
        for rid, c in zip(rids, counts):
            for _ in range(c):
                s, slot, copy = append_token(s, rid)
                slots.append(slot)
                if copy is not None:
                    copies.append(copy)
        self.state = s
        return slots, copies

    # ------------------------------------------------------------ views
    def requests(self):
        return [r for r, _ in self.state.requests]

    def table(self, rid):
        return list(self.state.request(rid).blocks)

    def length(self, rid) -> int:
        return self.state.request(rid).length

    def ref_count(self, block: int) -> int:
        return self.state.users(block)

    def ref_counts(self):
        return [self.state.users(b) for b in range(self.num_blocks)]

    def free_list(self):
        """Free blocks, the next one handed out first."""
        return self.state.free_in_order()

    def num_free(self) -> int:
        return len(self.state.tickets)

    def snapshot(self):
        """A comparable summary: (free list, reference counts, tables, lengths)."""
        return (self.free_list(), self.ref_counts(), {r: self.table(r) for r in self.requests()},
                {r: self.length(r) for r in self.requests()})

    def wasted_slots(self) -> int:
        """Allocated slots that hold no token (P2's "wasted" column); a shared block
        holds as many tokens as the fullest table that names it."""
        B = self.block_size
        used: Dict[int, int] = {}
        for _, req in self.state.requests:
            for j, b in enumerate(req.blocks):
                used[b] = max(used.get(b, 0), min(B, req.length - j * B))
        return B * len(used) - sum(used.values())

    def check_invariants(self) -> None:
        """Every block is either free (once) or named by some table; tables fit their
        lengths and name a block at most once."""
        s = self.state
        free = [b for b, _ in s.tickets]
        assert len(free) == len(set(free)), "a block is listed twice"
        assert len({t for _, t in s.tickets}) == len(s.tickets), "two blocks share a ticket"
        for rid, req in s.requests:
            assert len(req.blocks) == -(-req.length // self.block_size), f"table of {rid!r} does not fit its length"
            assert len(set(req.blocks)) == len(req.blocks), f"table of {rid!r} names a block twice"
        for b in range(self.num_blocks):
            assert (b in free) == (s.users(b) == 0), f"block {b} lost or double-booked"


def move_requests(src: BlockManager, dst: BlockManager, rids):
    """Move requests from ``src`` to ``dst`` (swap out or in).  Returns the block copies
    [(src block, dst block), ...]; raises OutOfBlocks or KeyError with nothing changed."""
    rids = list(rids)
    if len(set(rids)) != len(rids):
        raise KeyError("a request id is repeated")
    if src.block_size != dst.block_size:
        raise ValueError("block sizes differ")
    s, d = src.state, dst.state
    moved = [(rid, s.request(rid)) for rid in rids]
    for rid in rids:
        if d.has(rid):
            raise KeyError(f"request {rid!r} exists in the destination")
    mapping: Dict[int, int] = {}
    for _, req in moved:
        for b in req.blocks:
            if b not in mapping:
                d, mapping[b] = d.take_block()
    for rid, req in moved:
        d = d.with_request(rid, Request(tuple(mapping[b] for b in req.blocks), req.length))
    for rid in rids:
        s = drop(s, rid)
    src.state, dst.state = s, d
    return list(mapping.items())
