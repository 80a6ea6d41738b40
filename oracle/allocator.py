"""Oracle block pool: fixed-size blocks, reference counts, block-level COW.

TEST INFRASTRUCTURE (see the package header).

What it follows:
  * [PUFANYI] "按 Block 分配": a sequence of T tokens holds ceil(T/B) blocks;
    new tokens fill the tail block first and a block is taken from the pool
    only once the tail is full; a finished request drops its references and
    blocks nobody references go back to the pool.
  * [VLLBC] walk-through of paper §4.2: the 7-token, B=4 prompt occupies
    physical blocks 7 and 1, the first decode token uses the spare slot of
    logical block 1, the second one takes a fresh block 3.
  * [VLLBC] paper §4.4 / Fig. 8 and [PUFANYI] "共享前缀，分叉时 Copy-on-write":
    sharing bumps a per-block reference count; a writer whose tail block is
    shared (count > 1) first copies the block to a fresh one, moves its own
    mapping there and decrements the old count; the last holder writes in
    place.
  * [CSDN] §3.2.1: new blocks come from the head of the free queue and an
    allocation that does not fit fails without side effects (§3.1.1 returns
    None / §3.2.1 raises when the pool is short).
  * [CSDN] §3.1.2 / §3.2.4: a request's blocks are released tail first; every
    block whose count reaches zero is appended to the tail of the free queue.
  * [CSDN] §3.2.3 (touch): sharing increments the count of every shared block.

  * [CSDN] §3.1.1 / §3.3.1 (sliding window): before new slots are
    allocated, the blocks that lie wholly before the window are released;
    their number is the count of skipped tokens divided by B, rounded down.

Readings where the pages are silent or disagree:
  * The free queue is a FIFO seeded with an explicit initial order, freed
    blocks go to its tail, and there is no reserved null block ([CSDN] §2.4
    reserves block 0, [PUFANYI] uses P0 as an ordinary block; [VLLBC]'s V1
    notes put uncached blocks at the front).  With the initial order
    [7, 1, 3, 4, 5, 0, 2, 6] this reproduces the [VLLBC] examples exactly.
  * Only the first appended token of a shared partial tail can trigger a
    copy; a full shared tail is never copied (a new block is opened instead).
  * Sliding window W: after N computed tokens the next query (position N)
    sees positions N - W + 1 .. N, so max(0, N - W + 1) tokens are skipped.
    A released block leaves a hole (None) in the table, is dropped like a
    freed block (count down, to the queue tail at zero), and the holes are
    released tail first, as a freed request's blocks are.

Pinned by: tests/test_oracle_allocator.py against the pages' worked examples
(tests/golden/*.txt) and by closed-form block / slot counts.
"""

from __future__ import annotations

from collections import deque


class PoolExhausted(Exception):
    """The pool holds fewer free blocks than an operation needs."""


class OraclePool:
    """A pool of ``num_blocks`` physical blocks of ``block_size`` token slots."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be >= 1")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free = deque(order)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.num_cow = 0

    # ---- queries -------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def block_table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        return self.lens[seq]

    # ---- mutations -----------------------------------------------------
    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise ValueError(f"sequence {seq} already exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def _take(self) -> int:
        blk = self.free.popleft()
        assert self.ref[blk] == 0
        self.ref[blk] = 1
        return blk

    def blocks_needed(self, seq: int, n: int) -> int:
        """Fresh blocks that appending ``n`` tokens to ``seq`` would take."""
        B = self.block_size
        length = self.lens[seq]
        table = self.tables[seq]
        need = 0
        if n > 0 and length % B != 0 and self.ref[table[-1]] > 1:
            need += 1  # copy-on-write of the shared, partly filled tail
        held = -(-length // B)
        need += -(-(length + n) // B) - held
        return need

    def append(self, seq: int, n: int):
        """Append ``n`` tokens to ``seq``.

        Returns ``(slots, cow_pairs)``: the physical slot of every new token in
        order, and the (src, dst) block copies the writer must perform before
        writing.  All-or-nothing: raises PoolExhausted with no state change.
        """
        if n < 1:
            raise ValueError("n must be >= 1")
        if self.blocks_needed(seq, n) > len(self.free):
            raise PoolExhausted(f"sequence {seq} needs more blocks than are free")
        B = self.block_size
        table = self.tables[seq]
        slots, cow = [], []
        for _ in range(n):
            length = self.lens[seq]
            if length % B == 0:
                table.append(self._take())
            elif self.ref[table[-1]] > 1:
                old = table[-1]
                new = self._take()
                self.ref[old] -= 1
                table[-1] = new
                cow.append((old, new))
                self.num_cow += 1
            blk = table[length // B]
            slots.append(blk * B + length % B)
            self.lens[seq] = length + 1
        return slots, cow

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (counts go up by one)."""
        if child in self.tables:
            raise ValueError(f"sequence {child} already exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            if blk is not None:
                self.ref[blk] += 1

    def remove_skipped(self, seq: int, num_computed: int, window: int) -> list:
        """Release the blocks of ``seq`` that lie wholly before the window of
        its next query; returns the released block ids in release order."""
        table = self.tables[seq]
        skipped_blocks = num_skipped_tokens(num_computed, window) // self.block_size
        released = []
        for j in reversed(range(min(skipped_blocks, len(table)))):
            blk = table[j]
            if blk is None:
                continue
            table[j] = None
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
            released.append(blk)
        return released

    def free_seq(self, seq: int) -> None:
        """Drop ``seq``; blocks are released tail first."""
        table = self.tables.pop(seq)
        del self.lens[seq]
        for blk in reversed(table):
            if blk is None:
                continue
            self.ref[blk] -= 1
            if self.ref[blk] < 0:
                raise AssertionError(f"block {blk} released more often than taken")
            if self.ref[blk] == 0:
                self.free.append(blk)

    # ---- invariants ------------------------------------------------------
    def check_invariants(self) -> None:
        mapped = [0] * self.num_blocks
        for table in self.tables.values():
            for blk in table:
                if blk is not None:
                    mapped[blk] += 1
        assert mapped == self.ref, "reference counts differ from the table mappings"
        free = set(self.free)
        assert len(free) == len(self.free), "a block is queued twice"
        for blk in range(self.num_blocks):
            assert (blk in free) == (self.ref[blk] == 0), f"block {blk} free/referenced mismatch"
        for seq, table in self.tables.items():
            assert len(table) == -(-self.lens[seq] // self.block_size)


def num_skipped_tokens(num_computed: int, window: int) -> int:
    """Tokens no future query sees once ``num_computed`` tokens are computed
    (window W: the next query, at position num_computed, starts at
    num_computed - W + 1); 0 without a window."""
    return max(0, num_computed - window + 1) if window > 0 else 0


def sharing_saving(tables) -> float:
    """Block saving of a set of tables, as the [VLLBC] simulator defines it:
    (logical mappings - distinct physical blocks) / logical mappings."""
    mappings = sum(len(t) for t in tables)
    distinct = len({b for t in tables for b in t})
    return (mappings - distinct) / mappings


def tail_fragmentation(lengths, block_size: int):
    """Blocks, slots and empty slots when each length gets ceil(L/B) blocks
    ([PUFANYI] "按 Block 分配"; [VLLBC] §7.2 example)."""
    blocks = sum(-(-L // block_size) for L in lengths)
    slots = blocks * block_size
    empty = slots - sum(lengths)
    return blocks, slots, empty, empty / slots
