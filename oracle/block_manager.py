"""Plain reference model of the block manager that produces block tables, slots and
copy-on-write copies -- TEST INFRASTRUCTURE ONLY (tests/ may import it; the product
path never does, and this module imports nothing from it).

Sources (page title, then the section used):

[P2] "Why AI servers waste memory, and how paging fixes it" -- "The idea: a block
     table" (cut the pool into blocks once, keep a free list, append a block to a
     request's table when its last block is full, return blocks when it finishes),
     "A hand-worked example" (new blocks come from the front of the free list, freed
     blocks join the back; "wasted" = allocated slots minus stored tokens),
     "The real implementation" (the manager's state; append with the missing-block
     check first, so a failing call changes nothing; free returns a block only when
     no table points at it), "Sharing a prefix with copy-on-write" (fork copies the
     table and adds one reference per block; a write into a shared block with room
     first copies that block).
[P3] "PagedAttention and Virtual Memory Management" -- section 5 (reference counts
     R[p], forking k streams adds k - 1 to each shared block's count, case 1 writes in
     place, case 2 allocates p_new, copies the o token vectors already in p, drops
     R[p] by one, repoints the table and writes slot o of p_new).

Readings:
* Fork follows P2: one child per call, +1 per block, and the parent keeps running;
  P3's k-way fork is the parent plus k - 1 such forks, which adds k - 1.
* The copy made on a write into a shared block moves the o = length mod B rows the
  block already holds (P3 section 5 case 2).  P2's listing copies the whole block;
  the rows past o are never read before they are written, so both readings leave
  every readable value the same.  The copy is reported as (src, dst, rows).
* ``append_batch`` (one decode step over many requests) is a sequence of appends in
  the order given; if any of them cannot get a block, the manager is left exactly as
  it was before the batch (the pages' check-before-mutate rule, applied to the batch).
* Free walks the request's table front to back (P2 "The real implementation"),
  so blocks freed together join the free list in table order (P2's example, step 7).

Swap (``move_requests``), from [P3] section 6 (swapping policy: a second pool of
blocks in host memory; the victim's blocks are copied there, the freed GPU blocks go
back to the active pool, and on resume the blocks are copied back and decoding goes
on where it stopped) and [P4] "2.1 PagedAttention" (preemption: swap moves the cache
to CPU memory and back instead of recomputing it).  Readings:
* The host pool is a second manager of the same kind; a swap moves a set of requests
  from one manager to the other (out: device to host; in: host to device).
* Every distinct block the moved tables name gets one new block in the destination,
  taken from its free list in first-seen order (requests in the order given, each
  table front to back); a block the moved requests share stays shared there, with
  the same count.  The (src, dst) pairs are the copies to make.
* The source then drops the moved requests as ``free`` does, request after request,
  table front to back.  A block still named by a request that stays behind keeps
  its contents and its remaining references; its copy goes along anyway.
* All or nothing: unknown or repeated ids, or an id the destination already has,
  change nothing; so does a destination free list shorter than the distinct blocks.
"""

from __future__ import annotations

import copy as _copy
from collections import deque

__all__ = ["OutOfBlocks", "BlockManager", "move_requests"]


class OutOfBlocks(Exception):
    """No free block for an append that needs one; nothing was changed."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_list = deque(range(num_blocks))   # take from the front, give back at the back
        self.ref_count = [0] * num_blocks           # tables that name each block
        self.tables: dict = {}                      # request id -> physical blocks in logical order
        self.lengths: dict = {}                     # request id -> tokens stored

    # ------------------------------------------------------------ requests

    def add_request(self, rid) -> None:
        if rid in self.tables:
            raise KeyError(f"request {rid!r} exists")
        self.tables[rid] = []
        self.lengths[rid] = 0

    def fork(self, parent, child) -> None:
        """The child starts as a copy of the parent's table and length; every block
        they name gains one reference.  No block is allocated or copied."""
        if parent not in self.tables:
            raise KeyError(f"unknown request {parent!r}")
        if child in self.tables:
            raise KeyError(f"request {child!r} exists")
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for block in self.tables[child]:
            self.ref_count[block] += 1

    def free(self, rid) -> None:
        if rid not in self.tables:
            raise KeyError(f"unknown request {rid!r}")
        for block in self.tables.pop(rid):
            self.ref_count[block] -= 1
            if self.ref_count[block] == 0:
                self.free_list.append(block)
        del self.lengths[rid]

    # ------------------------------------------------------------ writes

    def _take_block(self) -> int:
        block = self.free_list.popleft()
        assert self.ref_count[block] == 0
        self.ref_count[block] = 1
        return block

    def append(self, rid):
        """Reserve the slot of the request's next token.

        Returns (slot, copy): slot = physical block * B + offset, and copy is None or
        (src, dst, rows) when the last block was shared and had room, so that its
        first `rows` token rows must be copied to the new block before the token is
        written there."""
        if rid not in self.tables:
            raise KeyError(f"unknown request {rid!r}")
        table, n = self.tables[rid], self.lengths[rid]
        offset = n % self.block_size
        last_is_full = offset == 0                   # also true for an empty table
        last_is_shared = not last_is_full and self.ref_count[table[-1]] > 1
        if (last_is_full or last_is_shared) and not self.free_list:
            raise OutOfBlocks(rid)                   # checked before anything changes
        copy = None
        if last_is_full:
            table.append(self._take_block())
        elif last_is_shared:
            old, new = table[-1], self._take_block()
            self.ref_count[old] -= 1
            table[-1] = new
            copy = (old, new, offset)
        self.lengths[rid] = n + 1
        return table[-1] * self.block_size + offset, copy

    def append_batch(self, rids, counts=None):
        """Appends counts[i] tokens to rids[i], request after request, in order.
        Returns (slots, copies) in that order.  All or nothing: on OutOfBlocks the
        manager is restored to its state before the call."""
        counts = [1] * len(rids) if counts is None else list(counts)
        if len(counts) != len(rids):
            raise ValueError("rids and counts differ in length")
        saved = (deque(self.free_list), list(self.ref_count), _copy.deepcopy(self.tables),
                 dict(self.lengths))
        slots, copies = [], []
        try:
            for rid, c in zip(rids, counts):
                for _ in range(c):
                    slot, cp = self.append(rid)
                    slots.append(slot)
                    if cp is not None:
                        copies.append(cp)
        except Exception:
            self.free_list, self.ref_count, self.tables, self.lengths = saved
            raise
        return slots, copies

    # ------------------------------------------------------------ views

    def table(self, rid):
        return list(self.tables[rid])

    def length(self, rid) -> int:
        return self.lengths[rid]

    def num_free(self) -> int:
        return len(self.free_list)

    def wasted_slots(self) -> int:
        """Allocated slots minus stored tokens (P2's "wasted" column); a shared block's
        tokens count once, as many as the fullest table that names it."""
        filled = {}
        for rid, table in self.tables.items():
            n = self.lengths[rid]
            for j, block in enumerate(table):
                valid = min(self.block_size, n - j * self.block_size)
                filled[block] = max(filled.get(block, 0), valid)
        return len(filled) * self.block_size - sum(filled.values())

    def check_invariants(self) -> None:
        """No block lost, double-booked or listed twice; reference counts equal the
        number of tables naming each block; every table covers its length exactly."""
        free = list(self.free_list)
        assert len(free) == len(set(free)), "a block is listed twice"
        counts = [0] * self.num_blocks
        for rid, table in self.tables.items():
            n = self.lengths[rid]
            assert len(table) == -(-n // self.block_size), f"table of {rid!r} does not fit its length"
            assert len(table) == len(set(table)), f"table of {rid!r} names a block twice"
            for block in table:
                counts[block] += 1
        assert counts == self.ref_count, "reference counts do not match the tables"
        free_set = set(free)
        for block in range(self.num_blocks):
            in_free = block in free_set
            assert in_free == (counts[block] == 0), f"block {block} lost or double-booked"


def move_requests(src: BlockManager, dst: BlockManager, rids):
    """Move requests from ``src`` to ``dst`` (swap out or in).  Returns the block
    copies [(src block, dst block), ...] to make; raises OutOfBlocks (nothing changed)
    if ``dst`` has too few free blocks, KeyError for a bad id."""
    rids = list(rids)
    if len(set(rids)) != len(rids):
        raise KeyError("a request id is repeated")
    for rid in rids:
        if rid not in src.tables:
            raise KeyError(f"unknown request {rid!r}")
        if rid in dst.tables:
            raise KeyError(f"request {rid!r} exists in the destination")
    if src.block_size != dst.block_size:
        raise ValueError("block sizes differ")
    order = []                                   # distinct source blocks, first seen first
    for rid in rids:
        for block in src.tables[rid]:
            if block not in order:
                order.append(block)
    if len(order) > dst.num_free():
        raise OutOfBlocks(rids)
    new = {block: dst.free_list.popleft() for block in order}
    for rid in rids:
        dst.tables[rid] = [new[b] for b in src.tables[rid]]
        dst.lengths[rid] = src.lengths[rid]
        for b in dst.tables[rid]:
            dst.ref_count[b] += 1
    for rid in rids:
        src.free(rid)
    return [(b, new[b]) for b in order]
