"""Pins of the oracle's decode functions (one new query per sequence against a
cache) against facts that do not come from the decode code itself: brute-force
selection by enumeration, the dense softmax written out with loops, the
uniform-attention closed form, cache contents past the length never mattering,
and the forward's row n_b - 1 (the forward oracle is pinned on its own). CPU
only."""
import itertools
import math

import numpy as np
import pytest

from oracle import msa_oracle as O


def _caches(rng, B, C, Hkv, G, D, Di, lo=-2, hi=2):
    k_idx = rng.integers(lo, hi + 1, size=(B, C, Di)).astype(np.float64)
    q_idx = rng.integers(lo, hi + 1, size=(B, Hkv, Di)).astype(np.float64)
    k = rng.standard_normal((B, C, Hkv, D))
    v = rng.standard_normal((B, C, Hkv, D))
    q = rng.standard_normal((B, Hkv * G, D))
    return q_idx, k_idx, q, k, v


def _brute_select(q_row, keys, n, Bk, k):
    """Kept blocks of the query at position n - 1, by loops and by enumerating
    every subset of the competing blocks (the subset whose members all outrank
    every non-member under score desc, id asc)."""
    i = n - 1
    L = i // Bk
    m = []
    for j in range(L):
        best = -math.inf
        for t in range(j * Bk, (j + 1) * Bk):
            s = sum(float(q_row[d]) * float(keys[t][d]) for d in range(len(q_row)))
            best = max(best, s)
        m.append(best)
    size = min(k - 1, L)
    found = [sub for sub in itertools.combinations(range(L), size)
             if all(m[a] > m[b] or (m[a] == m[b] and a < b)
                    for a in sub for b in range(L) if b not in sub)]
    assert len(found) == 1
    ids = sorted(list(found[0]) + [L])
    return ids + [-1] * (k - len(ids))


@pytest.mark.parametrize("seed,B,C,Bk,k,Di,Hkv", [
    (0, 4, 30, 4, 3, 3, 2),      # many ties
    (1, 5, 23, 3, 5, 2, 1),      # k - 1 above the candidates of short sequences
    (2, 3, 17, 4, 1, 3, 2),      # k = 1: the local block only
])
def test_decode_selection_matches_brute_force(seed, B, C, Bk, k, Di, Hkv):
    rng = np.random.default_rng(seed)
    q_idx, k_idx, _, _, _ = _caches(rng, B, C, Hkv, 1, 4, Di)
    lens = rng.integers(1, C + 1, size=B)
    lens[0] = C
    got = O.decode_index_topk(q_idx, k_idx, lens, Bk, k)
    for b in range(B):
        for g in range(Hkv):
            assert got[b, g].tolist() == _brute_select(q_idx[b, g], k_idx[b], int(lens[b]), Bk, k), (b, g)


def _dense_row(qh, keys, vals, n, scale):
    """Softmax attention of one query over keys 0..n-1 written out with loops."""
    z = [scale * sum(qh[d] * keys[t][d] for d in range(len(qh))) for t in range(n)]
    mx = max(z)
    w = [math.exp(x - mx) for x in z]
    s = sum(w)
    o = [sum(w[t] * vals[t][d] for t in range(n)) / s for d in range(len(vals[0]))]
    return o, mx + math.log(s)


def test_decode_dense_when_k_covers_every_block():
    """k >= the number of visible blocks: every cached token is attended, so the
    output is plain causal softmax attention of the new query."""
    rng = np.random.default_rng(5)
    B, C, Hkv, G, D, Di, Bk = 3, 40, 2, 2, 4, 3, 8
    q_idx, k_idx, q, k, v = _caches(rng, B, C, Hkv, G, D, Di)
    lens = np.array([40, 17, 1])
    bi = O.decode_index_topk(q_idx, k_idx, lens, Bk, 8)
    o, lse = O.decode_attention(q, k, v, lens, bi, Bk)
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv * G):
            g = h // G
            want_o, want_l = _dense_row(q[b, h], k[b, :, g], v[b, :, g], n, scale)
            np.testing.assert_allclose(o[b, h], want_o, rtol=1e-12, atol=1e-12)
            assert abs(lse[b, h] - want_l) < 1e-12


def test_decode_uniform_attention_closed_form():
    """Q = 0: every selected token gets the same weight, so LSE = ln |T| with
    |T| = (min(k, L+1) - 1) Bk + (i mod Bk) + 1, and O is the mean of V over T."""
    rng = np.random.default_rng(6)
    B, C, Hkv, G, D, Di, Bk, k = 4, 60, 2, 2, 3, 3, 8, 3
    q_idx, k_idx, q, kc, v = _caches(rng, B, C, Hkv, G, D, Di)
    q[:] = 0.0
    lens = np.array([60, 9, 8, 1])
    bi = O.decode_index_topk(q_idx, k_idx, lens, Bk, k)
    o, lse = O.decode_attention(q, kc, v, lens, bi, Bk)
    for b in range(B):
        i = int(lens[b]) - 1
        L = i // Bk
        count = (min(k, L + 1) - 1) * Bk + (i % Bk) + 1
        for g in range(Hkv):
            toks = [t for j in bi[b, g] if j >= 0 for t in range(j * Bk, min((j + 1) * Bk, i + 1))]
            assert len(toks) == count
            for h in range(g * G, (g + 1) * G):
                assert abs(lse[b, h] - math.log(count)) < 1e-12
                np.testing.assert_allclose(o[b, h], v[b, toks, g].mean(axis=0), atol=1e-12)


def test_decode_ignores_cache_past_length():
    rng = np.random.default_rng(7)
    B, C, Hkv, G, D, Di, Bk, k = 3, 50, 2, 2, 4, 3, 8, 3
    q_idx, k_idx, q, kc, v = _caches(rng, B, C, Hkv, G, D, Di)
    lens = np.array([31, 50, 8])
    bi = O.decode_index_topk(q_idx, k_idx, lens, Bk, k)
    o, lse = O.decode_attention(q, kc, v, lens, bi, Bk)
    k_idx2, kc2, v2 = k_idx.copy(), kc.copy(), v.copy()
    for b in range(B):
        n = int(lens[b])
        k_idx2[b, n:] = 99.0
        kc2[b, n:] = 1e3
        v2[b, n:] = -1e3
    bi2 = O.decode_index_topk(q_idx, k_idx2, lens, Bk, k)
    o2, lse2 = O.decode_attention(q, kc2, v2, lens, bi2, Bk)
    assert np.array_equal(bi, bi2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_decode_invalid_lengths():
    rng = np.random.default_rng(8)
    B, C, Hkv, G, D, Di, Bk, k = 3, 20, 1, 2, 4, 3, 8, 2
    q_idx, k_idx, q, kc, v = _caches(rng, B, C, Hkv, G, D, Di)
    lens = np.array([0, 21, 20])
    bi = O.decode_index_topk(q_idx, k_idx, lens, Bk, k)
    assert (bi[:2] == -1).all() and bi[2, 0, -1] == (20 - 1) // Bk
    o, lse = O.decode_attention(q, kc, v, lens, bi, Bk)
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all() and np.isfinite(lse[2]).all()


def test_decode_is_the_forward_row():
    """Placing each new query at row n_b - 1 of a full-sequence problem, the
    forward oracle's row n_b - 1 gives the decode result."""
    rng = np.random.default_rng(9)
    B, C, Hkv, G, D, Di, Bk, k = 3, 70, 2, 4, 8, 6, 8, 4
    q_idx, k_idx, q, kc, v = _caches(rng, B, C, Hkv, G, D, Di, lo=-3, hi=3)
    lens = np.array([70, 33, 8])
    q_full = rng.standard_normal((B, C, Hkv * G, D))
    qi_full = rng.integers(-3, 4, size=(B, C, Hkv, Di)).astype(np.float64)
    for b in range(B):
        q_full[b, lens[b] - 1] = q[b]
        qi_full[b, lens[b] - 1] = q_idx[b]
    bi_full = O.index_topk(qi_full, k_idx, Bk, k)            # [B, Hkv, C, k]
    o_full, lse_full = O.sparse_attention(q_full, kc, v, bi_full, Bk)
    bi = O.decode_index_topk(q_idx, k_idx, lens, Bk, k)
    o, lse = O.decode_attention(q, kc, v, lens, bi, Bk)
    for b in range(B):
        i = int(lens[b]) - 1
        assert np.array_equal(bi[b], bi_full[b, :, i])
        np.testing.assert_allclose(o[b], o_full[b, i], atol=1e-12)
        np.testing.assert_allclose(lse[b], lse_full[b, :, i], atol=1e-12)


def test_decode_planted_mistakes_are_caught():
    """A decode that queried position n_b (off by one) or kept the cache's last
    block instead of the query's would fail the pins above: show that both
    change the result on this input."""
    rng = np.random.default_rng(10)
    B, C, Hkv, G, D, Di, Bk, k = 2, 40, 1, 2, 4, 3, 8, 2
    q_idx, k_idx, q, kc, v = _caches(rng, B, C, Hkv, G, D, Di)
    lens = np.array([16, 24])          # the query ends a block: one more token opens the next
    good = O.decode_index_topk(q_idx, k_idx, lens, Bk, k)
    off_by_one = O.decode_index_topk(q_idx, k_idx, lens + 1, Bk, k)
    assert not np.array_equal(good, off_by_one)
    o, _ = O.decode_attention(q, kc, v, lens, good, Bk)
    o_next, _ = O.decode_attention(q, kc, v, lens + 1, off_by_one, Bk)
    assert np.abs(o - o_next).max() > 1e-3
    last_block = good.copy()
    last_block[:, :, -1] = (C - 1) // Bk
    o_bad, _ = O.decode_attention(q, kc, v, lens, last_block, Bk)
    assert np.abs(o - o_bad).max() > 1e-3


def test_multi_query_decode_is_the_forward_rows():
    """R new tokens per sequence: row r (position n_b - R + r) is the forward
    oracle's row there; rows at negative positions do not exist."""
    rng = np.random.default_rng(12)
    B, C, Hkv, G, D, Di, Bk, k, R = 3, 70, 2, 4, 8, 6, 8, 4, 3
    _, k_idx, _, kc, v = _caches(rng, B, C, Hkv, G, D, Di, lo=-3, hi=3)
    lens = np.array([70, 33, 2])
    q_full = rng.standard_normal((B, C, Hkv * G, D))
    qi_full = rng.integers(-3, 4, size=(B, C, Hkv, Di)).astype(np.float64)
    q_new = np.zeros((B, R, Hkv * G, D))
    qi_new = np.zeros((B, R, Hkv, Di))
    for b in range(B):
        for r in range(R):
            i = lens[b] - R + r
            if i >= 0:
                q_new[b, r], qi_new[b, r] = q_full[b, i], qi_full[b, i]
    bi_full = O.index_topk(qi_full, k_idx, Bk, k)
    o_full, lse_full = O.sparse_attention(q_full, kc, v, bi_full, Bk)
    bi = O.decode_index_topk(qi_new, k_idx, lens, Bk, k)            # [B, Hkv, R, k]
    o, lse = O.decode_attention(q_new, kc, v, lens, bi, Bk)         # [B, R, Hq, D], [B, Hq, R]
    for b in range(B):
        for r in range(R):
            i = int(lens[b]) - R + r
            if i < 0:
                assert (bi[b, :, r] == -1).all() and (o[b, r] == 0).all() and np.isneginf(lse[b, :, r]).all()
                continue
            assert np.array_equal(bi[b, :, r], bi_full[b, :, i])
            np.testing.assert_allclose(o[b, r], o_full[b, i], atol=1e-12)
            np.testing.assert_allclose(lse[b, :, r], lse_full[b, :, i], atol=1e-12)
    # the last row alone is the single-query decode
    bi1 = O.decode_index_topk(qi_new[:, -1], k_idx, lens, Bk, k)
    assert np.array_equal(bi1, bi[:, :, -1])
