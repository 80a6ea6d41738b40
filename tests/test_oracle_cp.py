"""Pins of the oracle's context-parallel attention (CPU only).

The ranks of a context-parallel group store disjoint shares of every
sequence ([CSDN] §2.3 slot mapping with world size > 1).  Each rank's
(m, l, o) over its share, merged with the split-K merge, must equal dense
softmax attention over the whole sequence, and each share's (m, l, o) must
equal the one computed straight from the positions the rank owns.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle.attention import (attention_partial, merge_rank_partials,
                              paged_attention_partials)
from oracle.cache_ops import reshape_and_cache
from oracle.slots import compute_slot_mapping_cp, cp_local_length, cp_owner_and_offset
from test_oracle_attention import _dense


def _cp_case(rng, lens, hkv, G, D, B, world):
    """Logical K/V per sequence, virtual-block tables and a query."""
    vbs = B * world
    need = [-(-L // vbs) for L in lens]
    nb = sum(need) + 2
    perm = rng.permutation(nb)
    tables, k = [], 0
    for n in need:
        tables.append(list(perm[k:k + n]))
        k += n
    W = max(max(need), 1)
    bt = np.full((len(lens), W), -1, dtype=np.int64)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    Klog = [rng.standard_normal((hkv, L, D)) for L in lens]
    Vlog = [rng.standard_normal((hkv, L, D)) for L in lens]
    q = rng.standard_normal((len(lens), hkv * G, D))
    return q, bt, nb, Klog, Vlog


def _rank_cache(rank, world, I, B, nb, bt, Klog, Vlog, lens):
    """This rank's cache, written token by token through its slot mapping."""
    hkv, D = Klog[0].shape[0], Klog[0].shape[2]
    kc = np.full((nb, hkv, B, D), np.nan)  # slots nobody writes poison the result
    vc = np.full((nb, hkv, B, D), np.nan)
    qsl = np.concatenate([[0], np.cumsum(lens)])
    pos = np.concatenate([np.arange(L) for L in lens])
    T = int(qsl[-1])
    slots = compute_slot_mapping_cp(qsl, pos, bt, B, T, world, rank, I)
    k = np.concatenate([Klog[s].transpose(1, 0, 2) for s in range(len(lens))])
    v = np.concatenate([Vlog[s].transpose(1, 0, 2) for s in range(len(lens))])
    reshape_and_cache(kc, vc, k, v, slots, B)
    local = [cp_local_length(L, B, world, rank, I) for L in lens]
    return kc, vc, local


CASES = [  # world, interleave, block size, group
    (1, 1, 4, 1), (2, 1, 4, 1), (2, 4, 4, 2), (3, 2, 4, 1), (4, 1, 2, 2), (4, 8, 8, 1),
]


@pytest.mark.parametrize("world,I,B,G", CASES)
def test_rank_partials_merge_to_dense_attention(world, I, B, G):
    rng = np.random.default_rng(7 * world + 3 * I + B + G)
    # short sequences leave some ranks without any token
    lens = [1, 2, 3, B * world - 1, B * world + 1, 3 * B * world + 5]
    hkv, D = 2, 8
    q, bt, nb, Klog, Vlog = _cp_case(rng, lens, hkv, G, D, B, world)
    scale = 0.29
    parts = []
    for r in range(world):
        kc, vc, local = _rank_cache(r, world, I, B, nb, bt, Klog, Vlog, lens)
        parts.append(paged_attention_partials(q, kc, vc, bt, local, scale, "f64"))
    m = np.stack([p[0] for p in parts])
    l = np.stack([p[1] for p in parts])
    o = np.stack([p[2] for p in parts])
    got = merge_rank_partials(m, l, o)
    want = _dense(q, Klog, Vlog, float(np.float32(scale)), G)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    if world > 1:  # the shortest sequence leaves ranks 1.. empty
        assert all(l[r, 0, 0] == 0 and m[r, 0, 0] == -np.inf for r in range(1, world))


@pytest.mark.parametrize("world,I,B,G", CASES)
def test_rank_partial_is_the_partial_over_owned_positions(world, I, B, G):
    rng = np.random.default_rng(11 * world + I + B)
    lens = [5, 2 * B * world + 3]
    hkv, D = 1, 4
    q, bt, nb, Klog, Vlog = _cp_case(rng, lens, hkv, G, D, B, world)
    scale = 0.5
    sc = float(np.float32(scale))
    for r in range(world):
        kc, vc, local = _rank_cache(r, world, I, B, nb, bt, Klog, Vlog, lens)
        m, l, o = paged_attention_partials(q, kc, vc, bt, local, scale, "f64")
        for s, L in enumerate(lens):
            owned = [p for p in range(L)
                     if cp_owner_and_offset(p % (B * world), world, I)[0] == r]
            assert len(owned) == local[s]
            for h in range(hkv * G):
                wm, wl, wo = attention_partial(q[s, h], Klog[s][h // G][owned],
                                               Vlog[s][h // G][owned], sc)
                assert m[s, h] == pytest.approx(wm, abs=1e-12) or m[s, h] == wm
                assert l[s, h] == pytest.approx(wl, rel=1e-12, abs=0)
                np.testing.assert_allclose(o[s, h], wo, rtol=0, atol=1e-12)


def test_empty_partial_and_merge_special_cases():
    m, l, o = attention_partial(np.ones(3), np.zeros((0, 3)), np.zeros((0, 3)), 1.0)
    assert m == -np.inf and l == 0.0 and not o.any()
    # one part merges to itself; an empty part beside it changes nothing
    rng = np.random.default_rng(0)
    o1 = rng.standard_normal((1, 1, 1, 4))
    m1, l1 = np.array([[[0.7]]]), np.array([[[2.5]]])
    np.testing.assert_array_equal(merge_rank_partials(m1, l1, o1)[0, 0], o1[0, 0, 0])
    m2 = np.concatenate([m1, [[[-np.inf]]]])
    l2 = np.concatenate([l1, [[[0.0]]]])
    o2 = np.concatenate([o1, np.zeros((1, 1, 1, 4))])
    np.testing.assert_allclose(merge_rank_partials(m2, l2, o2)[0, 0], o1[0, 0, 0], atol=1e-15)
    # no key anywhere: the row is zero
    assert not merge_rank_partials(np.full((2, 1, 1), -np.inf), np.zeros((2, 1, 1)),
                                   np.zeros((2, 1, 1, 4))).any()
