"""Reference of block selection (index-key scoring, then top-k) -- TEST INFRASTRUCTURE.

Only the test suite and the benchmark's CPU-baseline leg may import this
module; the product library never imports, links or runs it and shares no
code with it.

The selection produces ``selected [Tq, Hkv, topk]``, the input of the
block-sparse pass. The pages name it -- the MSA README's "How It Works" and
"Highlighted Details" list sparse top-k selection beside the dense and
sparse attention kernels, and the sglang pull request "Speed up MiniMax-M3
sparse attention on Hopper" ("Changes to existing code") keeps a sparse
index K cache beside the K/V caches, stored in fp8 on Hopper with fp8 KV --
but the scoring itself is in a document they only link. The scoring below is
therefore a reading, and its parity is UNPINNED against the pages: the pins
fix that this code computes the rule written here, not that the rule is
MiniMax's.

Readings:
  * Each (query token t, KV head g) has one index query ``q_idx[t, g, :128]``.
    Each cached token j of sequence s has index keys ``k_idx(s, g, j)`` in a
    paged cache laid out like the attention K cache,
    ``[num_pages, Hkv, page_size, 128]``, read through the same page table.
  * Token j is visible to t when ``j < L_s`` and, when causal,
    ``j <= pos(t) = L_s - Tq_s + (t - cu[s])`` (the attention pass's
    bottom-right alignment).
  * The score of logical block b (tokens ``[128 b, 128 b + 128)``) is the
    largest ``q_idx[t, g] . k_idx(s, g, j)`` over its visible tokens; a block
    with no visible token scores -inf and is never selected.
  * ``selected[t, g, :]`` lists at most topk blocks: with ``force_local``,
    first the token's own block (the block of pos(t) when causal, the last
    block of the sequence when not), then the other blocks by descending
    score, equal scores by ascending block id; -1 pads the rest.
"""
from __future__ import annotations

import numpy as np

BLK = 128


def _positions(cu, used, Tq, causal):
    """(sequence, pos) of every query token; sequence -1 outside every range."""
    seq = np.full(Tq, -1, dtype=np.int64)
    pos = np.zeros(Tq, dtype=np.int64)
    cu = np.asarray(cu, dtype=np.int64)
    used = np.asarray(used, dtype=np.int64)
    for s in range(len(used)):
        a, b = int(cu[s]), int(cu[s + 1])
        L = int(used[s])
        for t in range(max(a, 0), min(b, Tq)):
            seq[t] = s
            pos[t] = L - (b - a) + (t - a) if causal else L - 1
    return seq, pos


def block_scores(q_idx, k_cache, block_tables, cu, used, page_size, causal, nb_cap=None, tokens=None):
    """float64 scores [Tq, Hkv, nb_cap] of the rule in the module docstring.

    q_idx: [Tq, Hkv, 128] and k_cache: [NP, Hkv, P, 128], float arrays holding
    the stored values exactly; block_tables: [B, MP]; cu: [B + 1]; used: [B].
    nb_cap defaults to ceil(MP * P / 128), the most blocks a sequence can hold.
    With ``tokens`` (query token ids) only those rows are computed; the
    others stay -inf.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    bt = np.asarray(block_tables, dtype=np.int64)
    Tq, Hkv, _ = q.shape
    P = int(page_size)
    if nb_cap is None:
        nb_cap = -(-bt.shape[1] * P // BLK)
    out = np.full((Tq, Hkv, nb_cap), -np.inf)
    seq, pos = _positions(cu, used, Tq, causal)
    wanted = np.ones(Tq, dtype=bool) if tokens is None else np.isin(np.arange(Tq), np.asarray(tokens))
    for s in range(len(used)):
        L = int(used[s])
        toks = np.nonzero((seq == s) & wanted)[0]
        if L <= 0 or toks.size == 0:
            continue
        j = np.arange(L)
        keys = kc[bt[s, j // P], :, j % P, :]          # [L, Hkv, 128], de-paged
        nb = -(-L // BLK)
        for t in toks:
            visible = j <= pos[t]                          # j < L holds by construction
            for g in range(Hkv):
                logits = keys[:, g, :] @ q[t, g]           # [L]
                pooled = np.full(nb * BLK, -np.inf)
                pooled[:L] = np.where(visible, logits, -np.inf)
                out[t, g, :nb] = pooled.reshape(nb, BLK).max(axis=1)
    return out


def select_topk(scores, topk, cu, used, causal, force_local=True):
    """int32 selected [Tq, Hkv, topk] from scores [Tq, Hkv, nb_cap] (any float dtype).

    The comparisons are made in the scores' own precision, so a caller that
    passes float32 scores gets the decisions a float32 implementation takes.
    """
    sc = np.asarray(scores)
    Tq, Hkv, nb_cap = sc.shape
    out = np.full((Tq, Hkv, topk), -1, dtype=np.int32)
    seq, pos = _positions(cu, used, Tq, causal)
    for t in range(Tq):
        if seq[t] < 0 or pos[t] < 0:
            continue
        local = int(pos[t]) // BLK
        for g in range(Hkv):
            row = sc[t, g]
            cand = [b for b in range(nb_cap) if row[b] > -np.inf]
            picks = []
            if force_local and local in cand and topk > 0:
                picks.append(local)
                cand.remove(local)
            cand.sort(key=lambda b: (-row[b], b))
            picks += cand[:topk - len(picks)]
            out[t, g, :len(picks)] = picks
    return out


def select_blocks(q_idx, k_cache, block_tables, cu, used, page_size, causal, topk, force_local=True):
    """(selected, scores): the whole step on exact values, in float64."""
    sc = block_scores(q_idx, k_cache, block_tables, cu, used, page_size, causal)
    return select_topk(sc, topk, cu, used, causal, force_local), sc
