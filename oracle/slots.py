"""Oracle slot mapping: logical token position -> physical cache slot.

TEST INFRASTRUCTURE (see the package header).

What it follows:
  * [PUFANYI] "按 Block 分配": position p lives in logical block p div B; the
    block table names its physical block; inside that block it sits at
    offset p mod B (the [3, 0, 4] example sends position 8 to P4, offset 0).
  * [CSDN] §2.3 (slot-mapping kernel, context-parallel world size 1): the
    slot id is physical_block * B + offset, one entry per scheduled token, the
    tokens of request r being those between query_start_loc[r] and
    query_start_loc[r + 1].

Readings where the pages are silent:
  * The padding id the kernel writes for unused entries is -1 (the page names
    a PAD_ID constant but not its value), and entries from the number of
    scheduled tokens up to the buffer length are filled with it.

Context parallelism ([CSDN] §2.3, the same kernel with world size > 1):
world ranks share one block table; a virtual block holds B * world
consecutive positions; offset o inside it belongs to rank (o div I) mod world
(I = interleave size), which stores it in the same-numbered block of its own
pool at local offset (o div (world * I)) * I + o mod I; on other ranks the
token maps to the padding id.

Kernel blocks ([CSDN] §3.4, hybrid block sizes): when the allocator's blocks
hold k smaller blocks of the attention kernel, manager block b stands for
kernel blocks b*k .. b*k + k - 1, in order.

Pinned by: tests/test_oracle_slots.py (the [3, 0, 4] example, the 7-token
growth example, bijection onto the occupied slots of random pools, and for
context parallelism: world 1 equals the plain mapping, hand-computed
interleaves, every position on exactly one rank, each rank's local offsets
filled in position order; the manager-to-kernel example [0, 1, 2] x 2 ->
[0..5] and slot numbers that agree under both block sizes).
"""

from __future__ import annotations

PAD_SLOT = -1


def slot_of(table_row, pos: int, block_size: int) -> int:
    """Physical slot of logical position ``pos`` of one sequence."""
    logical_block = pos // block_size
    offset = pos % block_size
    return int(table_row[logical_block]) * block_size + offset


def compute_slot_mapping(query_start_loc, positions, block_tables, block_size: int,
                         max_num_tokens: int):
    """Slot of every scheduled token; entries past the last token are PAD_SLOT.

    query_start_loc: [S + 1] ints; positions: [T] ints; block_tables: S rows.
    Returns a Python list of length ``max_num_tokens``.
    """
    num_reqs = len(query_start_loc) - 1
    num_tokens = int(query_start_loc[num_reqs])
    if num_tokens > max_num_tokens:
        raise ValueError("more tokens than the slot buffer holds")
    out = [PAD_SLOT] * max_num_tokens
    for r in range(num_reqs):
        for i in range(int(query_start_loc[r]), int(query_start_loc[r + 1])):
            out[i] = slot_of(block_tables[r], int(positions[i]), block_size)
    return out


def cp_owner_and_offset(offset_in_virtual_block: int, world: int, interleave: int):
    """(rank, local offset) of an offset inside a virtual block of B * world
    positions, following the interleave of [CSDN] §2.3."""
    o = offset_in_virtual_block
    rank = (o // interleave) % world
    local = (o // (world * interleave)) * interleave + o % interleave
    return rank, local


def compute_slot_mapping_cp(query_start_loc, positions, block_tables, block_size: int,
                            max_num_tokens: int, world: int, rank: int, interleave: int):
    """Rank ``rank``'s slot of every scheduled token (PAD_SLOT when another
    rank stores it); entries past the last token are PAD_SLOT."""
    num_reqs = len(query_start_loc) - 1
    num_tokens = int(query_start_loc[num_reqs])
    if num_tokens > max_num_tokens:
        raise ValueError("more tokens than the slot buffer holds")
    virtual = block_size * world
    out = [PAD_SLOT] * max_num_tokens
    for r in range(num_reqs):
        for i in range(int(query_start_loc[r]), int(query_start_loc[r + 1])):
            pos = int(positions[i])
            vblock, off = divmod(pos, virtual)
            owner, local = cp_owner_and_offset(off, world, interleave)
            if owner == rank:
                out[i] = int(block_tables[r][vblock]) * block_size + local
    return out


def cp_local_length(length: int, block_size: int, world: int, rank: int,
                    interleave: int) -> int:
    """How many of a sequence's first ``length`` positions rank ``rank`` holds."""
    return sum(1 for p in range(length)
               if cp_owner_and_offset(p % (block_size * world), world, interleave)[0] == rank)


def map_to_kernel_blocks(manager_ids, blocks_per_kv_block: int):
    """Kernel block ids of a row of manager block ids ([CSDN] §3.4: manager
    block b covers kernel blocks b*k .. b*k + k - 1)."""
    k = int(blocks_per_kv_block)
    out = []
    for b in manager_ids:
        for j in range(k):
            out.append(int(b) * k + j)
    return out
