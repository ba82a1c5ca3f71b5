"""Plain reference model of automatic prefix caching on a paged block pool -- TEST
INFRASTRUCTURE ONLY (tests/ may import it; the product path never does, and this module
imports nothing from it).

Sources (page title, then the section used):

[P1] "PagedAttention: Treating KV Memory Like Virtual Memory" -- "A separate mechanism:
     automatic prefix caching": a block is hashed when it fills up, from the previous
     block's hash, the block's token ids and extras; the hashes form a chain, so a match
     means agreement from the first token; a match ends on a block boundary (a
     2,407-token prefix shares 150 full blocks, 2,400 tokens, and its 7-token tail is
     nobody else's); a hit copies nothing and raises the block's count, finishing lowers
     it, and at zero the block returns to the free list with its hash intact; the free
     list hands out uncached blocks first and cached ones oldest first; a cache_salt
     mixed into the first block's hash keeps requests with different salts apart.
[P4] "2.1 PagedAttention", section 9 (BlockPool / KVCacheManager): new blocks are
     taken from the head of a doubly linked free queue, failing before any change if
     there are not enough; free lowers the counts of a request's blocks in reverse order
     and puts the blocks that reach zero back, hash-less ones at the head (reused first)
     and hashed ones at the tail (evicted last); a hit on a free cached block removes it
     from the middle of the queue ("touch"); allocating a cached free block evicts its
     hash.

Readings:
* Hash: 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3) over the
  little-endian bytes of the previous block's hash (0 before the first block), the
  block's token ids (4 bytes each) and, for the first block only, the 8-byte salt.
* A lookup matches full blocks of the prompt only, as many leading ones as the table
  holds, and may cover the whole prompt when its length is a multiple of B.
* When a block fills and its hash is already in the table (another block holds the same
  prefix), the new block stays uncached; the table keeps the first block.
* prepend / append of several blocks keep their order: the group freed together sits at
  the head (or the tail) in the order the request's blocks were walked, last first.
* Appends are all or nothing, like the block manager's.
"""

from __future__ import annotations

import struct

__all__ = ["fnv1a64", "block_hash", "OutOfBlocks", "PrefixCache"]

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(prev: int, tokens, salt: int = 0, first: bool = False) -> int:
    data = struct.pack("<Q", prev & MASK64) + b"".join(struct.pack("<i", int(t)) for t in tokens)
    if first:
        data += struct.pack("<Q", salt & MASK64)
    return fnv1a64(data)


class OutOfBlocks(Exception):
    """Not enough free blocks; nothing was changed."""


class PrefixCache:
    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.hash = [None] * num_blocks
        self.free = list(range(num_blocks))      # head first
        self.cached = {}                         # hash -> block
        self.tables = {}
        self.lengths = {}
        self.tokens = {}                         # token ids written so far
        self.salts = {}
        self.last_hash = {}                      # hash of the request's last full block

    # ------------------------------------------------------------ pool
    def _take(self, n: int):
        if n > len(self.free):
            raise OutOfBlocks(n)
        out = self.free[:n]
        del self.free[:n]
        for b in out:
            if self.hash[b] is not None:         # a cached free block: evict its hash
                del self.cached[self.hash[b]]
                self.hash[b] = None
            assert self.ref[b] == 0
            self.ref[b] = 1
        return out

    def _touch(self, blocks):
        for b in blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1

    def _release(self, ordered):
        for b in ordered:
            self.ref[b] -= 1
        to_free = [b for b in ordered if self.ref[b] == 0]
        no_hash = [b for b in to_free if self.hash[b] is None]
        has_hash = [b for b in to_free if self.hash[b] is not None]
        self.free = no_hash + self.free + has_hash

    # ------------------------------------------------------------ requests
    def chain(self, tokens, salt: int = 0):
        """Hashes of the full blocks of a token sequence."""
        B = self.block_size
        out, prev = [], 0
        for j in range(len(tokens) // B):
            prev = block_hash(prev, tokens[j * B:(j + 1) * B], salt, first=(j == 0))
            out.append(prev)
        return out

    def add_request(self, rid, prompt, salt: int = 0) -> int:
        """Start a request; the leading full blocks of `prompt` already cached become its
        first blocks.  Returns the number of prompt tokens found (a multiple of B)."""
        if rid in self.tables:
            raise KeyError(rid)
        matched = []
        for h in self.chain(prompt, salt):
            b = self.cached.get(h)
            if b is None:
                break
            matched.append(b)
        self._touch(matched)
        n = len(matched) * self.block_size
        self.tables[rid] = list(matched)
        self.lengths[rid] = n
        self.tokens[rid] = list(prompt[:n])
        self.salts[rid] = salt
        self.last_hash[rid] = self.hash[matched[-1]] if matched else 0
        return n

    def append(self, rid, tokens):
        """Slots for the request's next tokens (their ids given); blocks that fill up
        are hashed and cached.  All or nothing."""
        B = self.block_size
        n0 = self.lengths[rid]
        need = (n0 + len(tokens) + B - 1) // B - (n0 + B - 1) // B
        new = self._take(need)                  # raises before any change
        table = self.tables[rid]
        slots = []
        for t in tokens:
            n = self.lengths[rid]
            if n % B == 0:
                table.append(new.pop(0))
            slots.append(table[-1] * B + n % B)
            self.tokens[rid].append(int(t))
            self.lengths[rid] = n + 1
            if (n + 1) % B == 0:                # the block is full: hash and cache it
                j = n // B
                h = block_hash(self.last_hash[rid], self.tokens[rid][j * B:(j + 1) * B],
                               self.salts[rid], first=(j == 0))
                self.last_hash[rid] = h
                blk = table[-1]
                if h not in self.cached and self.hash[blk] is None:
                    self.cached[h] = blk
                    self.hash[blk] = h
        return slots

    def append_step(self, rids, tokens):
        """A decode step: token tokens[i] for request rids[i], the requests distinct;
        appending one token to each in turn, after checking the whole step first (the
        requests whose last block is full each need a block).  All or nothing."""
        rids = [int(r) for r in rids]
        if len(set(rids)) != len(rids) or any(r not in self.lengths for r in rids):
            raise ValueError("unknown or repeated request")
        need = sum(1 for r in rids if self.lengths[r] % self.block_size == 0)
        if need > len(self.free):
            raise OutOfBlocks(need)
        return [self.append(r, [t])[0] for r, t in zip(rids, tokens)]

    def free_request(self, rid):
        table = self.tables.pop(rid)
        self._release(list(reversed(table)))
        for d in (self.lengths, self.tokens, self.salts, self.last_hash):
            del d[rid]

    # ------------------------------------------------------------ checks
    def check_invariants(self):
        counts = [0] * self.num_blocks
        for t in self.tables.values():
            for b in t:
                counts[b] += 1
        assert counts == self.ref
        assert len(self.free) == len(set(self.free))
        assert set(self.free) == {b for b in range(self.num_blocks) if self.ref[b] == 0}
        for h, b in self.cached.items():
            assert self.hash[b] == h
        assert sum(h is not None for h in self.hash) == len(self.cached)
