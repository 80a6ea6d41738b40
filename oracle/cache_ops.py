"""Oracle cache writes: scatter of new tokens, and whole-block copies.

TEST INFRASTRUCTURE (see the package header).

Cache layout (a reading; the pages do not fix the in-block layout): both the
key and the value cache are arrays [num_blocks, num_kv_heads, B, head_size],
so slot s addresses row (s div B, :, s mod B, :).

What it follows:
  * [VLLBC] walk-through of paper §4.2 and [PUFANYI] "按 Block 分配": a new
    token's key and value are stored at its slot, filling the tail block.
  * [VLLBC] paper §4.4 / Fig. 8 and [PUFANYI] "共享前缀，分叉时 Copy-on-write":
    copy-on-write duplicates one whole physical block (all heads, all slots)
    into the fresh block before the writer appends to it.

Both functions move raw storage elements (bit copies); they reject inputs
whose result would depend on the order of writes (a slot written twice, a
copy destination that repeats or is also a source).

Pinned by: tests/test_oracle_slots.py (gather of written slots returns the
input bytes, untouched rows unchanged, copied block byte-equal to its source,
order-dependent inputs rejected, the Fig. 8 sharing example replayed on data).
"""

from __future__ import annotations

import numpy as np


def reshape_and_cache(key_cache: np.ndarray, value_cache: np.ndarray,
                      key: np.ndarray, value: np.ndarray, slot_mapping,
                      block_size: int) -> None:
    """key/value: [T, num_kv_heads, head_size]; slots < 0 are skipped."""
    seen = set()
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        if slot in seen:
            raise ValueError(f"slot {slot} written twice in one scatter")
        seen.add(slot)
        blk, off = divmod(slot, block_size)
        key_cache[blk, :, off, :] = key[i]
        value_cache[blk, :, off, :] = value[i]


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray, block_mapping) -> None:
    """block_mapping: iterable of (src, dst) physical block pairs."""
    pairs = [(int(s), int(d)) for s, d in block_mapping]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("a destination block repeats")
    if set(dsts) & {s for s, _ in pairs}:
        raise ValueError("a destination block is also a source")
    for src, dst in pairs:
        key_cache[dst] = key_cache[src]
        value_cache[dst] = value_cache[src]
