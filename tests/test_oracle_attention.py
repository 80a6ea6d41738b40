"""Pins of the oracle attention: library brute force, closed forms, invariances."""

from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle.attention import (merge_partials, paged_attention, paged_attention_split,
                              split_partials)
from oracle.dtypes import decode


def _place(logical, tables, num_blocks, B):
    """Build a paged cache [NB, H_kv, B, D] from logical rows [S][H_kv, L, D]
    by copying whole logical blocks (slices) into their physical blocks."""
    hkv, D = logical[0].shape[0], logical[0].shape[2]
    cache = np.full((num_blocks, hkv, B, D), np.nan)  # unused slots poison the result
    for s, rows in enumerate(logical):
        L = rows.shape[1]
        for j, phys in enumerate(tables[s]):
            n = min(B, L - j * B)
            cache[phys, :, :n, :] = rows[:, j * B: j * B + n, :]
    return cache


def _random_case(rng, S, H, hkv, D, B, lens, spare=3):
    need = [-(-L // B) for L in lens]
    nb = sum(need) + spare
    perm = rng.permutation(nb)
    tables, k = [], 0
    for n in need:
        tables.append(list(perm[k:k + n]))
        k += n
    W = max(need)
    bt = np.full((S, W), -1, dtype=np.int64)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    Klog = [rng.standard_normal((hkv, L, D)) for L in lens]
    Vlog = [rng.standard_normal((hkv, L, D)) for L in lens]
    q = rng.standard_normal((S, H, D))
    kc = _place(Klog, tables, nb, B)
    vc = _place(Vlog, tables, nb, B)
    return q, kc, vc, bt, Klog, Vlog


def _dense(q, Klog, Vlog, scale, G):
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    for s in range(S):
        for h in range(H):
            g = h // G
            p = softmax(scale * (Klog[s][g] @ q[s, h]))
            out[s, h] = p @ Vlog[s][g]
    return out


@pytest.mark.parametrize("B", [1, 2, 3, 4])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_brute_force_equals_dense_softmax(B, G):
    rng = np.random.default_rng(100 * B + G)
    hkv, D = 2, 8
    lens = list(range(1, 14))
    q, kc, vc, bt, Klog, Vlog = _random_case(rng, len(lens), hkv * G, hkv, D, B, lens)
    scale = 0.37
    sc = float(np.float32(scale))
    got = paged_attention(q, kc, vc, bt, lens, scale, "f64")
    want = _dense(q, Klog, Vlog, sc, G)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_hand_computed_two_tokens():
    # x = [0, ln 3] -> weights 1 : 3 -> out = (v0 + 3 v1) / 4
    kc = np.zeros((2, 1, 1, 2))
    vc = np.zeros((2, 1, 1, 2))
    kc[1, 0, 0] = [0.0, 0.0]
    kc[0, 0, 0] = [math.log(3.0), 0.0]
    vc[1, 0, 0] = [4.0, 0.0]
    vc[0, 0, 0] = [0.0, 8.0]
    q = np.array([[[1.0, 0.0]]])
    out = paged_attention(q, kc, vc, np.array([[1, 0]]), [2], 1.0, "f64")
    np.testing.assert_allclose(out[0, 0], [1.0, 6.0], rtol=0, atol=1e-14)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(3)
    kc = rng.standard_normal((5, 1, 4, 16))
    vc = rng.standard_normal((5, 1, 4, 16))
    q = rng.standard_normal((1, 1, 16))
    out = paged_attention(q, kc, vc, np.array([[3]]), [1], 0.125, "f64")
    assert np.array_equal(out[0, 0], vc[3, 0, 0])


@pytest.mark.parametrize("mode", ["equal_keys", "zero_scale"])
def test_uniform_weights_give_mean_of_values(mode):
    rng = np.random.default_rng(4)
    B, L, D = 4, 11, 8
    kc = rng.standard_normal((4, 1, B, D))
    vc = rng.standard_normal((4, 1, B, D))
    table = np.array([[2, 0, 3]])
    if mode == "equal_keys":
        kc[:] = kc[0, 0, 0]
        scale = 0.5
    else:
        scale = 0.0
    q = rng.standard_normal((1, 1, D))
    out = paged_attention(q, kc, vc, table, [L], scale, "f64")
    rows = np.stack([vc[table[0, t // B], 0, t % B] for t in range(L)])
    np.testing.assert_allclose(out[0, 0], rows.mean(axis=0), rtol=0, atol=1e-14)


def test_large_logits_do_not_overflow():
    # x = [1000, 999]: weights e : 1, finite only if the max is subtracted
    kc = np.zeros((1, 1, 2, 1))
    vc = np.zeros((1, 1, 2, 1))
    kc[0, 0, :, 0] = [1000.0, 999.0]
    vc[0, 0, :, 0] = [1.0, 0.0]
    out = paged_attention(np.ones((1, 1, 1)), kc, vc, np.array([[0]]), [2], 1.0, "f64")
    np.testing.assert_allclose(out[0, 0, 0], math.e / (math.e + 1.0), rtol=1e-14)


def test_physical_permutation_invariance_is_exact():
    rng = np.random.default_rng(21)
    B, lens = 4, [5, 9, 16, 3]
    q, kc, vc, bt, _, _ = _random_case(rng, 4, 4, 2, 8, B, lens)
    base = paged_attention(q, kc, vc, bt, lens, 0.3, "f64")
    pi = rng.permutation(kc.shape[0])
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1)
    moved = paged_attention(q, kc2, vc2, bt2, lens, 0.3, "f64")
    assert np.array_equal(base, moved)


def test_shared_prefix_identity():
    """Two sequences whose KV is the same logical data in different blocks, or
    the same blocks (shared), read identical attention."""
    rng = np.random.default_rng(8)
    B, D, L = 4, 8, 10
    rows = rng.standard_normal((1, L, D))
    t_a, t_b = [5, 1, 7], [0, 6, 2]
    kc = _place([rows, rows], [t_a, t_b], 8, B)
    vc = _place([-rows, -rows], [t_a, t_b], 8, B)
    q = rng.standard_normal(D)
    query = np.stack([q, q, q])[:, None, :]
    bt = np.array([t_a, t_b, t_a])  # third row shares A's blocks
    out = paged_attention(query, kc, vc, bt, [L, L, L], 0.4, "f64")
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(12)
    G, hkv, B, lens = 4, 2, 4, [7, 13]
    q, kc, vc, bt, _, _ = _random_case(rng, 2, G * hkv, hkv, 8, B, lens)
    gqa = paged_attention(q, kc, vc, bt, lens, 0.35, "f64")
    mha = paged_attention(q, np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1), bt, lens,
                          0.35, "f64")
    assert np.array_equal(gqa, mha)
    # and a different head-to-group rule (h mod H_kv) gives a different answer
    alt = np.concatenate([kc] * G, axis=1), np.concatenate([vc] * G, axis=1)
    assert not np.allclose(gqa, paged_attention(q, alt[0], alt[1], bt, lens, 0.35, "f64"))


@pytest.mark.parametrize("P", [1, 4, 8, 12, 64])
def test_split_merge_equals_single_pass(P):
    rng = np.random.default_rng(P)
    B, lens = 4, [1, 4, 9, 33, 40]
    q, kc, vc, bt, _, _ = _random_case(rng, 5, 2, 1, 16, B, lens)
    one = paged_attention(q, kc, vc, bt, lens, 0.25, "f64")
    split, partials = paged_attention_split(q, kc, vc, bt, lens, 0.25, "f64", P)
    np.testing.assert_allclose(split, one, rtol=1e-13, atol=1e-13)
    for (s, h), (m, l, o) in partials.items():
        assert len(m) == -(-lens[s] // P)  # only non-empty partitions exist


def test_split_with_one_partition_is_the_single_pass():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((9, 4))
    V = rng.standard_normal((9, 4))
    q = rng.standard_normal(4)
    m, l, o = split_partials(q, K, V, 0.5, 16)
    assert len(m) == 1
    p = softmax(0.5 * (K @ q))
    np.testing.assert_allclose(merge_partials(m, l, o), p @ V, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l[0], np.exp(0.5 * (K @ q) - m[0]).sum(), rtol=1e-15)


def test_merge_weights_partitions_by_their_mass():
    # two partitions with equal maxima and masses 1 and 3 -> weights 1/4, 3/4
    m = np.array([2.0, 2.0])
    l = np.array([1.0, 3.0])
    o = np.array([[4.0], [8.0]])
    assert merge_partials(m, l, o)[0] == pytest.approx(7.0, abs=1e-15)
    # a partition whose max is lower by ln 3 has its mass scaled by 1/3
    m = np.array([0.0, -math.log(3.0)])
    l = np.array([1.0, 3.0])
    assert merge_partials(m, l, o)[0] == pytest.approx(6.0, abs=1e-14)


def test_rejects_empty_context():
    with pytest.raises(ValueError):
        paged_attention(np.zeros((1, 1, 2)), np.zeros((1, 1, 1, 2)), np.zeros((1, 1, 1, 2)),
                        np.array([[0]]), [0], 1.0, "f64")


def test_storage_decode_reaches_attention():
    """bf16 and fp16 inputs give the attention of their exact decoded values."""
    rng = np.random.default_rng(2)
    kc32 = rng.standard_normal((3, 1, 4, 8)).astype(np.float32)
    vc32 = rng.standard_normal((3, 1, 4, 8)).astype(np.float32)
    q32 = rng.standard_normal((1, 1, 8)).astype(np.float32)
    bt = np.array([[2, 0]])
    for dt, enc in (("f16", lambda a: a.astype(np.float16)),
                    ("bf16", lambda a: (a.view(np.uint32) >> 16).astype(np.uint16))):
        got = paged_attention(enc(q32), enc(kc32), enc(vc32), bt, [6], 0.3, dt)
        want = paged_attention(decode(enc(q32), dt), decode(enc(kc32), dt),
                               decode(enc(vc32), dt), bt, [6], 0.3, "f64")
        assert np.array_equal(got, want)


# ---- several new tokens per sequence (causal over the new tokens) ----------

from oracle.attention import paged_attention_multi  # noqa: E402


def _dense_causal(qrows, Klog, Vlog, scale, G, lens, qsl):
    """Dense reference: scipy softmax over the keys of a boolean causal mask."""
    T, H, D = qrows.shape
    out = np.zeros((T, H, D))
    for s, L in enumerate(lens):
        n = qsl[s + 1] - qsl[s]
        pos = np.arange(L)
        for i in range(n):
            me = L - n + i
            mask = pos <= me
            for h in range(H):
                g = h // G
                x = scale * (Klog[s][g] @ qrows[qsl[s] + i, h])
                p = softmax(np.where(mask, x, -np.inf))
                out[qsl[s] + i, h] = p @ Vlog[s][g]
    return out


@pytest.mark.parametrize("G", [1, 2, 4])
def test_multi_query_equals_dense_causal_softmax(G):
    rng = np.random.default_rng(40 + G)
    B, hkv, D = 4, 2, 8
    lens = [1, 3, 6, 9, 13]
    nq = [1, 3, 2, 5, 4]
    qsl = np.concatenate([[0], np.cumsum(nq)])
    _, kc, vc, bt, Klog, Vlog = _random_case(rng, len(lens), hkv * G, hkv, D, B, lens)
    q = rng.standard_normal((int(qsl[-1]), hkv * G, D))
    got = paged_attention_multi(q, kc, vc, bt, lens, qsl, 0.41, "f64")
    want = _dense_causal(q, Klog, Vlog, float(np.float32(0.41)), G, lens, qsl)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_multi_query_last_token_is_the_decode_result():
    rng = np.random.default_rng(5)
    lens, nq = [7, 12, 4], [3, 1, 4]
    qsl = np.concatenate([[0], np.cumsum(nq)])
    _, kc, vc, bt, _, _ = _random_case(rng, 3, 4, 2, 8, 4, lens)
    q = rng.standard_normal((int(qsl[-1]), 4, 8))
    multi = paged_attention_multi(q, kc, vc, bt, lens, qsl, 0.3, "f64")
    last = q[qsl[1:] - 1]
    single = paged_attention(last, kc, vc, bt, lens, 0.3, "f64")
    assert np.array_equal(multi[qsl[1:] - 1], single)


def test_multi_query_prefill_from_empty_context():
    """All L tokens are new: token 0 sees only itself, so its output is v0
    exactly; token i sees tokens 0..i."""
    rng = np.random.default_rng(6)
    L = 6
    _, kc, vc, bt, Klog, Vlog = _random_case(rng, 1, 1, 1, 4, 2, [L])
    q = rng.standard_normal((L, 1, 4))
    out = paged_attention_multi(q, kc, vc, bt, [L], [0, L], 0.5, "f64")
    assert np.array_equal(out[0, 0], Vlog[0][0][0])
    for i in range(L):
        p = softmax(float(np.float32(0.5)) * (Klog[0][0][: i + 1] @ q[i, 0]))
        np.testing.assert_allclose(out[i, 0], p @ Vlog[0][0][: i + 1], rtol=0, atol=1e-13)


def test_multi_query_rejects_more_queries_than_context():
    with pytest.raises(ValueError):
        paged_attention_multi(np.zeros((3, 1, 2)), np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)),
                              np.array([[0]]), [2], [0, 3], 1.0, "f64")
