"""Oracle prefix caching: chained block hashes, longest-hit lookup, LRU.

TEST INFRASTRUCTURE (see the package header).

What it follows:
  * [DEEPSONAR] §2.4 (V1's block pool and hash chain): a block's key is a
    chained hash, SHA-256 over the parent block's hash, the block's token ids
    and extra keys, so two prefixes that differ in one token differ in every
    later key.  The free queue doubles as the LRU list: freed blocks join its
    tail, allocation takes its head, and a head block that still holds cached
    content is first dropped from the hash table.
  * [CSDN] §5.2 (find_longest_cache_hit): walk the request's chain block by
    block and stop at the first key that is not cached; at most
    max_length // B blocks.  §5.3: max_length is the prompt length minus one
    (the last token is always computed again), only full blocks are cached
    (cache_full_blocks) and only those past the request's count of blocks
    already cached (the blocks it took over count as cached), and a block
    records its key when it is cached.
  * [CSDN] §3.2.1 / §3.2.2: a block taken from the free queue loses its key
    (eviction); §3.2.3 (touch): a hit on a block with no holder takes it out
    of the free queue and counts it.
  * [PUFANYI] "共享前缀，分叉时 Copy-on-write", its paragraphs on automatic
    prefix caching: only whole prefixes match; the key includes the
    previous block's key, the block's tokens and identifiers such as a LoRA
    id; only full blocks are cached.

Readings where the pages are silent:
  * Serialisation of the hashed message: parent key (32 bytes) || token ids
    as little-endian int32 || extra key bytes; the first block's parent key is
    32 zero bytes.  The extra key bytes of a request enter every block's key.
  * A key already mapped to another block keeps its first block; the second
    block is not cached (its content is equal, either serves).
  * Everything else is the allocator of oracle.allocator (FIFO free queue,
    freed blocks to the tail, tail first).

Pinned by tests/test_oracle_prefix_cache.py: SHA-256 against the FIPS 180
example digests, the chaining property, first-miss stop, the n - 1 cap,
full blocks only, LRU order of evictions and touch leaving the queue.
"""

from __future__ import annotations

import hashlib
import struct

from .allocator import OraclePool

ROOT_KEY = bytes(32)


def block_key(parent: bytes, tokens, extra: bytes = b"") -> bytes:
    """SHA-256 of parent key || int32 LE token ids || extra key bytes."""
    msg = parent + b"".join(struct.pack("<i", int(t)) for t in tokens) + extra
    return hashlib.sha256(msg).digest()


def key_chain(tokens, block_size: int, extra: bytes = b"") -> list:
    """Keys of every full block of a token sequence, each chained on the last."""
    keys, parent = [], ROOT_KEY
    for j in range(len(tokens) // block_size):
        parent = block_key(parent, tokens[j * block_size:(j + 1) * block_size], extra)
        keys.append(parent)
    return keys


class OraclePrefixPool(OraclePool):
    """The allocator with a prefix cache over its blocks."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.key_of = [None] * num_blocks  # cached key of each block
        self.cached = {}                    # key -> block
        self.tokens: dict[int, list] = {}
        self.extra: dict[int, bytes] = {}
        self.num_cached_blocks: dict[int, int] = {}  # per request
        self.num_evicted = 0

    def _take(self) -> int:
        blk = self.free[0]
        key = self.key_of[blk]
        if key is not None:  # the LRU head still holds cached content: evict it
            if self.cached.get(key) == blk:
                del self.cached[key]
            self.key_of[blk] = None
            self.num_evicted += 1
        return super()._take()

    def _touch(self, blk: int) -> None:
        if self.ref[blk] == 0:
            self.free.remove(blk)
        self.ref[blk] += 1

    def longest_hit(self, keys, max_length: int) -> list:
        """Blocks of the longest cached prefix of ``keys`` (first miss stops)."""
        hit = []
        for key in keys[:max_length // self.block_size]:
            blk = self.cached.get(key)
            if blk is None:
                break
            hit.append(blk)
        return hit

    def add_seq_cached(self, seq: int, prompt, extra: bytes = b"") -> int:
        """New sequence for ``prompt``: its longest cached prefix (at most
        len(prompt) - 1 tokens) is taken over; returns the tokens computed."""
        self.add_seq(seq)
        self.tokens[seq] = []
        self.extra[seq] = extra
        hit = self.longest_hit(key_chain(prompt, self.block_size, extra), len(prompt) - 1)
        for blk in hit:
            self._touch(blk)
        self.tables[seq] = list(hit)
        self.num_cached_blocks[seq] = len(hit)
        n = len(hit) * self.block_size
        self.lens[seq] = n
        self.tokens[seq] = list(prompt[:n])
        return n

    def append_tokens(self, seq: int, tokens):
        """Append token ids to ``seq`` (slots and copy pairs as append)."""
        slots, cow = self.append(seq, len(tokens))
        self.tokens[seq].extend(int(t) for t in tokens)
        return slots, cow

    def fork(self, parent: int, child: int) -> None:
        super().fork(parent, child)
        self.tokens[child] = list(self.tokens.get(parent, []))
        self.extra[child] = self.extra.get(parent, b"")
        self.num_cached_blocks[child] = self.num_cached_blocks.get(parent, 0)

    def free_seq(self, seq: int) -> None:
        super().free_seq(seq)
        self.tokens.pop(seq, None)
        self.extra.pop(seq, None)
        self.num_cached_blocks.pop(seq, None)

    def cache_full_blocks(self, seq: int) -> int:
        """Register the full blocks of ``seq`` past its count of cached blocks
        under their keys; returns how many blocks were newly cached."""
        keys = key_chain(self.tokens[seq], self.block_size, self.extra[seq])
        n = 0
        start = self.num_cached_blocks[seq]
        self.num_cached_blocks[seq] = max(start, len(keys))
        for j in range(start, len(keys)):
            key = keys[j]
            blk = self.tables[seq][j]
            if blk is None or self.key_of[blk] is not None:
                continue
            if key in self.cached:  # another block already holds this content
                continue
            self.key_of[blk] = key
            self.cached[key] = blk
            n += 1
        return n
