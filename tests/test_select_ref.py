"""Pins of the block-selection reference (CPU).

The scoring rule is a reading (the pages name the step but not its
formula), so these pins fix that the reference computes that rule: scores
built by construction, special cases, invariances and the defining
property of a top-k. Parity of the rule itself against the pages is
unpinned.
"""
import itertools

import numpy as np
import pytest

from oracle import select_ref as R


def _paged(keys_seq, P, NP, rng):
    """Scatter per-sequence keys [B][L_s, Hkv, 128] into a shuffled paged cache."""
    Hkv = keys_seq[0].shape[1]
    cache = np.full((NP, Hkv, P, 128), np.nan)
    pages = rng.permutation(NP)
    MP = max(-(-k.shape[0] // P) for k in keys_seq)
    bt = np.full((len(keys_seq), MP), -1, dtype=np.int32)
    nxt = 0
    for s, k in enumerate(keys_seq):
        for i in range(-(-k.shape[0] // P)):
            bt[s, i] = pages[nxt]
            nxt += 1
            rows = k[i * P:(i + 1) * P]
            cache[bt[s, i], :, :rows.shape[0]] = rows.transpose(1, 0, 2)
    return cache, bt


def _designed(L, Hkv, w, rng, spot=None):
    """Keys whose block maxima are w[b, g] for q = e_0: one spot token per block holds w, the rest -1000."""
    nb = -(-L // 128)
    k = np.zeros((L, Hkv, 128))
    k[:, :, 0] = -1000.0
    for b in range(nb):
        n = min(128, L - 128 * b)
        j = 128 * b + (int(rng.integers(n)) if spot is None else min(spot, n - 1))
        k[j, :, 0] = w[b]
    k[:, :, 1:] = rng.standard_normal((L, Hkv, 127))  # ignored by q = e_0
    return k


def test_scores_equal_the_designed_block_maxima_and_topk_their_order():
    rng = np.random.default_rng(1)
    Hkv, P, L, topk = 2, 64, 1000, 5
    nb = -(-L // 128)
    w = rng.permutation(nb * Hkv).reshape(nb, Hkv).astype(float) * 3.0 - 7.0
    keys = _designed(L, Hkv, w, rng)
    cache, bt = _paged([keys], P, 20, rng)
    q = np.zeros((1, Hkv, 128))
    q[:, :, 0] = 1.0
    cu, used = [0, 1], [L]
    sel, sc = R.select_blocks(q, cache, bt, cu, used, P, causal=False, topk=topk, force_local=False)
    assert np.array_equal(sc[0, :, :nb], w.T)
    assert np.all(sc[0, :, nb:] == -np.inf)
    for g in range(Hkv):
        assert list(sel[0, g]) == list(np.argsort(-w[:, g], kind="stable")[:topk])


def test_force_local_comes_first_even_when_it_scores_lowest():
    rng = np.random.default_rng(2)
    Hkv, P, L = 1, 128, 900
    nb = -(-L // 128)
    w = np.arange(nb, 0, -1, dtype=float)[:, None]   # block 0 best, the last block worst
    keys = _designed(L, Hkv, w, rng, spot=0)
    cache, bt = _paged([keys], P, 10, rng)
    q = np.zeros((1, Hkv, 128))
    q[:, :, 0] = 2.0
    sel, _ = R.select_blocks(q, cache, bt, [0, 1], [L], P, causal=False, topk=3)
    assert list(sel[0, 0]) == [nb - 1, 0, 1]


def test_causal_hides_tokens_after_the_position():
    rng = np.random.default_rng(3)
    Hkv, P, L, Tq = 1, 64, 512, 4                    # positions 508..511, local block 3
    w = np.array([[1.0], [2.0], [3.0], [4.0]])
    keys = _designed(L, Hkv, w, rng, spot=127)       # block 3's spot is token 511
    cache, bt = _paged([keys], P, 8, rng)
    q = np.zeros((Tq, Hkv, 128))
    q[:, :, 0] = 1.0
    sel, sc = R.select_blocks(q, cache, bt, [0, Tq], [L], P, causal=True, topk=2)
    assert np.all(sc[:3, 0, 3] == -1000.0) and sc[3, 0, 3] == 4.0  # only t=3 (pos 511) sees it
    assert np.all(sc[:, 0, :3] == w[:3, 0])
    for t in range(Tq):
        assert list(sel[t, 0]) == [3, 2]


def test_top_k_is_the_k_best_by_brute_force():
    # every size-k subset is compared: the chosen one has the largest score
    # multiset, and the list is in descending order with ties by block id
    rng = np.random.default_rng(4)
    for trial in range(200):
        nb, k = int(rng.integers(1, 7)), int(rng.integers(1, 5))
        row = rng.integers(-3, 4, size=nb).astype(float)   # many ties
        row[rng.random(nb) < 0.2] = -np.inf
        sc = row[None, None, :]
        sel = R.select_topk(sc, k, [0, 1], [nb * 128], causal=False, force_local=False)[0, 0]
        got = [b for b in sel if b >= 0]
        vis = [b for b in range(nb) if row[b] > -np.inf]
        assert len(got) == min(k, len(vis)) and len(set(got)) == len(got)
        best = max(itertools.combinations(vis, len(got)), key=lambda c: sorted((row[b] for b in c), reverse=True))
        assert sorted(row[b] for b in got) == sorted(row[b] for b in best)
        keyed = [(-row[b], b) for b in got]
        assert keyed == sorted(keyed)
        assert all(b == -1 for b in sel[len(got):])


def test_invariances():
    rng = np.random.default_rng(5)
    Hkv, P = 2, 64
    lens, tqs = [700, 300, 1100], [3, 1, 5]
    keys = [rng.standard_normal((L, Hkv, 128)) for L in lens]
    q = rng.standard_normal((sum(tqs), Hkv, 128))
    cu = np.concatenate([[0], np.cumsum(tqs)])
    c1, bt1 = _paged(keys, P, 60, np.random.default_rng(6))
    c2, bt2 = _paged(keys, P, 60, np.random.default_rng(7))    # another page placement
    for causal in (False, True):
        s1, sc1 = R.select_blocks(q, c1, bt1, cu, lens, P, causal, topk=4)
        s2, sc2 = R.select_blocks(q, c2, bt2, cu, lens, P, causal, topk=4)
        assert np.array_equal(sc1, sc2) and np.array_equal(s1, s2)
        s3, sc3 = R.select_blocks(2.5 * q, c1, bt1, cu, lens, P, causal, topk=4)  # positive scale
        assert np.allclose(sc3, 2.5 * sc1) and np.array_equal(s3, s1)
        # every pick is visible, distinct, and the local block leads
        seq, pos = R._positions(cu, lens, len(q), causal)
        for t in range(len(q)):
            for g in range(Hkv):
                picks = [b for b in s1[t, g] if b >= 0]
                assert picks[0] == pos[t] // 128
                assert len(set(picks)) == len(picks)
                assert all(128 * b <= pos[t] for b in picks)


def test_few_visible_blocks_pad_and_empty_sequences_select_nothing():
    rng = np.random.default_rng(8)
    Hkv, P = 1, 64
    keys = [rng.standard_normal((200, Hkv, 128)), rng.standard_normal((64, Hkv, 128))]
    cache, bt = _paged(keys, P, 8, rng)
    q = rng.standard_normal((3, Hkv, 128))
    cu = [0, 2, 2, 3]                    # sequence 1 has no queries
    used = [200, 64, 0]                  # sequence 2 has no keys
    bt = np.vstack([bt, np.full((1, bt.shape[1]), -1, np.int32)])
    sel, sc = R.select_blocks(q, cache, bt, cu, used, P, causal=False, topk=4)
    assert sorted(sel[0, 0, :2]) == [0, 1] and list(sel[0, 0, 2:]) == [-1, -1]
    assert list(sel[2, 0]) == [-1, -1, -1, -1] and np.all(sc[2] == -np.inf)
