"""Pins of the oracle slot mapping and cache writes."""

from __future__ import annotations

import numpy as np
import pytest

from conftest import ints, load_golden
from oracle.allocator import OraclePool
from oracle.cache_ops import copy_blocks, reshape_and_cache
from oracle.slots import PAD_SLOT, compute_slot_mapping


def test_slot_mapping_table_example():
    g = load_golden("t_table")
    table = ints(g["A_table"])
    B = int(g["block_size"][0])
    out = compute_slot_mapping([0, 1], [int(g["query_pos"][0])], [table], B, 4)
    assert out == [int(g["query_slot"][0]), PAD_SLOT, PAD_SLOT, PAD_SLOT]


def test_slot_mapping_growth_example():
    g = load_golden("t_grow")
    B = int(g["block_size"][0])
    table = ints(g["table_after_decode2"])
    positions = list(range(int(g["prompt_len"][0]) + 2))
    out = compute_slot_mapping([0, len(positions)], positions, [table], B, len(positions))
    assert out == ints(g["prompt_slots"]) + ints(g["decode1_slot"]) + ints(g["decode2_slot"])


def test_slot_mapping_is_a_bijection_onto_occupied_slots():
    rng = np.random.default_rng(11)
    for B in (1, 3, 4, 16):
        nb = 64
        pool = OraclePool(nb, B, rng.permutation(nb))
        lens = rng.integers(1, 5 * B, size=5)
        for s, L in enumerate(lens):
            pool.add_seq(s)
            pool.append(s, int(L))
        qsl = np.concatenate([[0], np.cumsum(lens)])
        positions = np.concatenate([np.arange(L) for L in lens])
        tables = [pool.block_table(s) for s in range(len(lens))]
        out = compute_slot_mapping(qsl, positions, tables, B, int(qsl[-1]) + 3)
        real = out[: int(qsl[-1])]
        assert out[int(qsl[-1]):] == [PAD_SLOT] * 3
        assert len(set(real)) == len(real)
        # every slot lies in a block of its own sequence, in order of position
        for s in range(len(lens)):
            seq_slots = real[qsl[s]: qsl[s + 1]]
            assert [x // B for x in seq_slots] == [tables[s][p // B] for p in range(lens[s])]
            assert [x % B for x in seq_slots] == [p % B for p in range(lens[s])]


def test_slot_mapping_rejects_overflow():
    with pytest.raises(ValueError):
        compute_slot_mapping([0, 3], [0, 1, 2], [[0]], 4, 2)


def test_scatter_round_trip_and_untouched_rows():
    rng = np.random.default_rng(5)
    nb, hkv, B, D = 6, 2, 4, 8
    kc = rng.integers(0, 2**16, size=(nb, hkv, B, D), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(nb, hkv, B, D), dtype=np.uint16)
    kc0, vc0 = kc.copy(), vc.copy()
    slots = [5, -1, 17, 0, 23]
    k = rng.integers(0, 2**16, size=(5, hkv, D), dtype=np.uint16)
    v = rng.integers(0, 2**16, size=(5, hkv, D), dtype=np.uint16)
    reshape_and_cache(kc, vc, k, v, slots, B)
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc[s // B, :, s % B, :], k[i])
        assert np.array_equal(vc[s // B, :, s % B, :], v[i])
        written.add(s)
    for s in range(nb * B):
        if s not in written:
            assert np.array_equal(kc[s // B, :, s % B, :], kc0[s // B, :, s % B, :])
            assert np.array_equal(vc[s // B, :, s % B, :], vc0[s // B, :, s % B, :])


def test_scatter_rejects_duplicate_slot():
    kc = np.zeros((2, 1, 2, 2), np.float32)
    with pytest.raises(ValueError):
        reshape_and_cache(kc, kc.copy(), np.ones((2, 1, 2), np.float32),
                          np.ones((2, 1, 2), np.float32), [3, 3], 2)


def test_copy_blocks_copies_whole_blocks_only():
    rng = np.random.default_rng(9)
    kc = rng.standard_normal((8, 2, 4, 8)).astype(np.float32)
    vc = rng.standard_normal((8, 2, 4, 8)).astype(np.float32)
    kc0, vc0 = kc.copy(), vc.copy()
    copy_blocks(kc, vc, [(1, 3), (6, 0)])
    assert np.array_equal(kc[3], kc0[1]) and np.array_equal(vc[3], vc0[1])
    assert np.array_equal(kc[0], kc0[6]) and np.array_equal(vc[0], vc0[6])
    for b in (1, 2, 4, 5, 6, 7):
        assert np.array_equal(kc[b], kc0[b]) and np.array_equal(vc[b], vc0[b])


@pytest.mark.parametrize("pairs", [[(1, 2), (3, 2)], [(1, 2), (2, 3)]])
def test_copy_blocks_rejects_order_dependent_pairs(pairs):
    kc = np.zeros((4, 1, 2, 2), np.float32)
    with pytest.raises(ValueError):
        copy_blocks(kc, kc.copy(), pairs)


def test_cow_copy_then_scatter_matches_sharing_example():
    """Fig. 8 replay on data: after the copy and both appends, A and B read the
    same prompt and differ only in their own new token."""
    g = load_golden("t_sharing")
    B = int(g["block_size"][0])
    pool = OraclePool(int(g["num_blocks"][0]), B, ints(g["free_order"]))
    nb, hkv, D = pool.num_blocks, 1, 4
    kc = np.zeros((nb, hkv, B, D), np.float32)
    vc = np.zeros_like(kc)
    pool.add_seq(0)
    slots, _ = pool.append(0, 7)
    prompt = np.arange(7 * D, dtype=np.float32).reshape(7, hkv, D) + 1
    reshape_and_cache(kc, vc, prompt, -prompt, slots, B)
    pool.fork(0, 1)
    new_tok = {0: np.full((1, hkv, D), 100.0, np.float32), 1: np.full((1, hkv, D), 200.0, np.float32)}
    for s in (0, 1):
        slots, cow = pool.append(s, 1)
        copy_blocks(kc, vc, cow)
        reshape_and_cache(kc, vc, new_tok[s], -new_tok[s], slots, B)
    for s in (0, 1):
        table = pool.block_table(s)
        seq = np.stack([kc[table[p // B], :, p % B, :] for p in range(8)])
        assert np.array_equal(seq[:7], prompt)
        assert np.array_equal(seq[7], new_tok[s][0])


# ---- context parallelism ------------------------------------------------------

from oracle.slots import compute_slot_mapping_cp, cp_local_length, cp_owner_and_offset  # noqa: E402


def test_cp_world_one_is_the_plain_mapping():
    rng = np.random.default_rng(3)
    for B, I in ((4, 1), (16, 4), (8, 8)):
        tables = [list(rng.permutation(20)[:6]) for _ in range(3)]
        lens = [5, 17, 23]
        qsl = np.concatenate([[0], np.cumsum(lens)])
        pos = np.concatenate([np.arange(L) for L in lens])
        pos = np.minimum(pos, 6 * B - 1)
        assert compute_slot_mapping_cp(qsl, pos, tables, B, len(pos), 1, 0, I) == \
            compute_slot_mapping(qsl, pos, tables, B, len(pos))


def test_cp_interleave_hand_examples():
    # B = 4, two ranks: virtual block of 8 positions
    # interleave 1: ranks alternate; local offsets 0,0,1,1,2,2,3,3
    got = [cp_owner_and_offset(o, 2, 1) for o in range(8)]
    assert got == [(0, 0), (1, 0), (0, 1), (1, 1), (0, 2), (1, 2), (0, 3), (1, 3)]
    # interleave 2: pairs alternate; local offsets 0,1,0,1,2,3,2,3
    got = [cp_owner_and_offset(o, 2, 2) for o in range(8)]
    assert got == [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3)]
    # interleave = B: each rank takes one whole block's worth in turn
    got = [cp_owner_and_offset(o, 2, 4) for o in range(8)]
    assert got == [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0), (1, 1), (1, 2), (1, 3)]


@pytest.mark.parametrize("world,I,B", [(2, 1, 4), (4, 2, 8), (3, 1, 2), (8, 16, 16)])
def test_cp_every_position_on_exactly_one_rank_in_order(world, I, B):
    rng = np.random.default_rng(world * 100 + I)
    L = 5 * B * world + 3
    table = list(rng.permutation(64)[: -(-L // (B * world))])
    pos = list(range(L))
    owners = {}
    for r in range(world):
        slots = compute_slot_mapping_cp([0, L], pos, [table], B, L, world, r, I)
        local = [(p, s) for p, s in zip(pos, slots) if s != PAD_SLOT]
        for p, s in local:
            assert p not in owners
            owners[p] = (r, s)
        # the rank's tokens fill local offsets of each (same-numbered) block in order
        flat = [(table.index(s // B), s % B) for _, s in local]
        assert flat == [(j // B, j % B) for j in range(len(local))]
        assert len(local) == cp_local_length(L, B, world, r, I)
    assert sorted(owners) == pos


# ---- kernel blocks ------------------------------------------------------------

from oracle.slots import map_to_kernel_blocks  # noqa: E402


def test_kernel_block_example():
    g = load_golden("t_k2k")
    k = int(g["blocks_per_kv_block"][0])
    assert k == int(g["manager_block_size"][0]) // int(g["kernel_block_size"][0])
    assert map_to_kernel_blocks(ints(g["manager_ids"]), k) == ints(g["kernel_ids"])


def test_kernel_blocks_one_per_manager_block_is_identity():
    assert map_to_kernel_blocks([7, 3, 0, 9], 1) == [7, 3, 0, 9]


@pytest.mark.parametrize("k,Bk", [(2, 16), (4, 4), (8, 1), (3, 5)])
def test_kernel_block_slots_equal_manager_block_slots(k, Bk):
    """A position's slot is the same number under the manager table at block
    size k * Bk and under the kernel table at block size Bk."""
    rng = np.random.default_rng(k * 10 + Bk)
    Bm = k * Bk
    lens = [1, Bm - 1, Bm, 3 * Bm + 2, 7 * Bm]
    tables = [list(rng.permutation(40)[: -(-L // Bm)]) for L in lens]
    qsl = np.concatenate([[0], np.cumsum(lens)])
    pos = np.concatenate([np.arange(L) for L in lens])
    manager = compute_slot_mapping(qsl, pos, tables, Bm, len(pos))
    kernel = compute_slot_mapping(qsl, pos, [map_to_kernel_blocks(t, k) for t in tables], Bk,
                                  len(pos))
    assert manager == kernel
