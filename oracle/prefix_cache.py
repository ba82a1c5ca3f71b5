"""Plain reference model of automatic prefix caching on a paged block pool -- TEST
INFRASTRUCTURE ONLY (tests/ may import it; the product path never does, and this module
imports nothing from it).

Written from the rules the pages state (page title, then the section):

[P1] "PagedAttention: Treating KV Memory Like Virtual Memory" -- "A separate mechanism:
     automatic prefix caching":
       - a block gets a hash when it fills up, computed from the previous block's hash,
         the block's token ids and extras, so the hashes form a chain and a match means
         agreement from the first token; matches end on block boundaries (a
         2,407-token prefix shares its 150 full blocks, 2,400 tokens);
       - a hit copies nothing, it only gives the block one more user; when a block's
         last user finishes it becomes free but keeps its hash and can still be found;
       - free blocks without a hash are reused before cached ones, and cached ones are
         reused oldest first; a cache salt mixed into the first block's hash keeps
         requests with different salts apart.
[P4] "2.1 PagedAttention", section 9 (BlockPool / KVCacheManager):
       - new blocks come from the head of the free queue, and a request that needs more
         than are free fails before anything changes;
       - a finishing request's blocks are released last block first; those nobody uses
         any more re-enter the queue, hash-less ones at the head (reused first) and
         cached ones at the tail (evicted last);
       - a hit on a free cached block takes it out of the queue;
       - reusing a cached free block for new data drops its hash from the cache.

Data model (ours): the free queue is a map from block to an ordering key, the head
being the smallest key; putting a group at the head gives it keys below every key in
use, putting it at the tail keys above them.  A block's number of users is not stored:
it is counted from the request tables when needed.  Each request keeps its token ids
and the chain of hashes of its full blocks.  Every call first works out what it will do
from the current state, checks that it can, and only then applies it.

Readings:
* Hash: 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3, the
  published parameters) over the little-endian bytes of the previous block's hash (0
  before the first block), the block's token ids (4 bytes each) and, for the first
  block only, the 8-byte salt.
* A lookup matches leading full blocks of the prompt, as many as are cached, and may
  cover the whole prompt when its length is a multiple of B.
* When a block fills and its hash is already cached (another block holds the same
  prefix), the new block stays uncached: the cache keeps the block it already has.
* A group released together keeps the order in which the finishing request's blocks
  were walked (last block first), at the head or at the tail.
* Appends are all or nothing; the blocks an append needs are taken (and their hashes
  dropped) before its tokens are placed.
"""

from __future__ import annotations

import struct

__all__ = ["fnv1a64", "block_hash", "OutOfBlocks", "PrefixCache"]

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64 bits: for each byte, xor it in, then multiply by the prime."""
    for byte in data:
        h = ((h ^ byte) * FNV_PRIME) & MASK64
    return h


def block_hash(prev: int, tokens, salt: int = 0, first: bool = False) -> int:
    data = struct.pack("<Q", prev & MASK64) + struct.pack(f"<{len(tokens)}i", *[int(t) for t in tokens])
    if first:
        data += struct.pack("<Q", salt & MASK64)
    return fnv1a64(data)


class OutOfBlocks(Exception):
    """Not enough free blocks; nothing was changed."""


class _Request:
    __slots__ = ("blocks", "tokens", "salt", "chain")

    def __init__(self, blocks, tokens, salt, chain):
        self.blocks = blocks      # physical blocks, logical order
        self.tokens = tokens      # token ids stored so far
        self.salt = salt
        self.chain = chain        # hashes of the full blocks, in order


class PrefixCache:
    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.queue = {b: b for b in range(num_blocks)}   # free block -> ordering key
        self.by_hash = {}                                # cached hash -> block
        self.hash_of = {}                                # cached block -> hash
        self.reqs = {}

    # ------------------------------------------------------------ helpers
    def users(self, block: int) -> int:
        return sum(r.blocks.count(block) for r in self.reqs.values())

    def _head_blocks(self, n: int):
        """The n free blocks at the head of the queue (checked: enough are free)."""
        if n > len(self.queue):
            raise OutOfBlocks(n)
        return sorted(self.queue, key=self.queue.get)[:n]

    def _claim(self, blocks) -> None:
        """Blocks leave the queue for new data; a cached one loses its hash."""
        for b in blocks:
            del self.queue[b]
            h = self.hash_of.pop(b, None)
            if h is not None:
                del self.by_hash[h]

    def chain(self, tokens, salt: int = 0):
        """Hashes of the full blocks of a token sequence."""
        B = self.block_size
        out, prev = [], 0
        for j in range(len(tokens) // B):
            prev = block_hash(prev, tokens[j * B:(j + 1) * B], salt, first=(j == 0))
            out.append(prev)
        return out

    # ------------------------------------------------------------ requests
    def add_request(self, rid, prompt, salt: int = 0) -> int:
        """Start a request; the leading full blocks of `prompt` that are cached become
        its first blocks.  Returns the number of prompt tokens found (a multiple of B)."""
        if rid in self.reqs:
            raise KeyError(rid)
        hits, hashes = [], []
        for h in self.chain(prompt, salt):
            if h not in self.by_hash:
                break
            hits.append(self.by_hash[h])
            hashes.append(h)
        for b in hits:                      # a free cached block leaves the queue
            self.queue.pop(b, None)
        n = len(hits) * self.block_size
        self.reqs[rid] = _Request(list(hits), [int(t) for t in prompt[:n]], salt, hashes)
        return n

    def append(self, rid, tokens):
        """Slots for the request's next tokens (their ids given); blocks that fill up
        are hashed and cached.  All or nothing."""
        B = self.block_size
        req = self.reqs[rid]
        n0 = len(req.tokens)
        have = -(-n0 // B)
        fresh = self._head_blocks(-(-(n0 + len(tokens)) // B) - have)
        self._claim(fresh)
        req.blocks.extend(fresh)
        slots = []
        for t in tokens:
            n = len(req.tokens)
            slots.append(req.blocks[n // B] * B + n % B)
            req.tokens.append(int(t))
            if (n + 1) % B == 0:            # block n // B is now full
                j = n // B
                h = block_hash(req.chain[-1] if req.chain else 0, req.tokens[j * B:], req.salt,
                               first=(j == 0))
                req.chain.append(h)
                if h not in self.by_hash:
                    self.by_hash[h] = req.blocks[j]
                    self.hash_of[req.blocks[j]] = h
        return slots

    def append_step(self, rids, tokens):
        """A decode step: token tokens[i] for request rids[i], the requests distinct;
        one token to each in turn, after the whole step is checked (each request whose
        last block is full needs a block).  All or nothing."""
        rids = [int(r) for r in rids]
        if len(set(rids)) != len(rids) or any(r not in self.reqs for r in rids):
            raise ValueError("unknown or repeated request")
        need = sum(len(self.reqs[r].tokens) % self.block_size == 0 for r in rids)
        self._head_blocks(need)             # raises before any change
        return [self.append(r, [t])[0] for r, t in zip(rids, tokens)]

    def free_request(self, rid) -> None:
        req = self.reqs.pop(rid)
        walk = [b for b in reversed(req.blocks) if self.users(b) == 0]
        plain = [b for b in walk if b not in self.hash_of]
        cached = [b for b in walk if b in self.hash_of]
        lo = min(self.queue.values(), default=0)
        hi = max(self.queue.values(), default=0)
        for i, b in enumerate(plain):       # the head, in walk order
            self.queue[b] = lo - len(plain) + i
        for i, b in enumerate(cached):      # the tail, in walk order
            self.queue[b] = hi + 1 + i

    # ------------------------------------------------------------ views
    def requests(self):
        return list(self.reqs)

    def table(self, rid):
        return list(self.reqs[rid].blocks)

    def length(self, rid) -> int:
        return len(self.reqs[rid].tokens)

    def tokens(self, rid):
        return list(self.reqs[rid].tokens)

    def free_queue(self):
        """Free blocks, head (next reused) first."""
        return sorted(self.queue, key=self.queue.get)

    def num_free(self) -> int:
        return len(self.queue)

    def ref_count(self, block: int) -> int:
        return self.users(block)

    def block_hash_of(self, block: int):
        """The block's cached hash, or None."""
        return self.hash_of.get(block)

    def cached(self):
        return dict(self.by_hash)

    def num_cached(self) -> int:
        return len(self.by_hash)

    def snapshot(self):
        """(free queue, per-block (users, hash), tables, token ids, cached map)."""
        return (self.free_queue(), [(self.users(b), self.hash_of.get(b)) for b in range(self.num_blocks)],
                {r: self.table(r) for r in self.reqs}, {r: self.tokens(r) for r in self.reqs},
                self.cached())

    # ------------------------------------------------------------ checks
    def check_invariants(self) -> None:
        for b in range(self.num_blocks):
            assert (b in self.queue) == (self.users(b) == 0), f"block {b} lost or double-booked"
        assert len(set(self.queue.values())) == len(self.queue), "two free blocks share a key"
        assert {b: h for h, b in self.by_hash.items()} == self.hash_of, "hash maps disagree"
        for rid, req in self.reqs.items():
            assert len(req.blocks) == -(-len(req.tokens) // self.block_size), rid
            assert len(req.chain) == len(req.tokens) // self.block_size, rid
