"""Brute-force dense attention over de-paged K/V -- TEST INFRASTRUCTURE.

When a token selects every block of its sequence, block-sparse attention is
ordinary (optionally causal) softmax attention over keys 0..L-1. That is the
situation of the fw-ai/minimax-kernels README "Quick start" example (one
query picks both 128-token blocks of a 256-token sequence). This module
computes that case with library primitives only: the page table is undone by
fancy indexing, scores come from one numpy matmul, and the causal mask is an
explicit bottom-right mask (key j is visible to query i of a sequence with
Tq_s queries and L keys when j <= L - Tq_s + i).
"""
from __future__ import annotations

import numpy as np
import torch


def depage(cache: torch.Tensor, table_row, L: int, g: int) -> np.ndarray:
    """[L, 128] fp64 rows of KV head g for logical tokens 0..L-1."""
    P = cache.shape[2]
    j = np.arange(L)
    pages = np.asarray(table_row, dtype=np.int64)[j // P]
    return cache[torch.from_numpy(pages), g, torch.from_numpy(j % P)].double().numpy()


def attention(q, k_cache, v_cache, block_tables, cu_seqlens_q, used_kv_lens, causal: bool):
    """Dense attention for every token over all keys of its sequence.

    Returns ``out [Tq, Hq, 128]`` and ``lse [Hq, Tq]`` in fp64.
    """
    qd = q.detach().cpu().double().numpy()
    Tq, Hq, _ = qd.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    cu = cu_seqlens_q.detach().cpu().numpy().astype(np.int64)
    used = used_kv_lens.detach().cpu().numpy().astype(np.int64)
    bt = block_tables.detach().cpu().numpy()
    out = np.zeros((Tq, Hq, 128))
    lse = np.full((Hq, Tq), -np.inf)
    scale = 1.0 / np.sqrt(128.0)
    for s in range(len(used)):
        q0, q1, L = int(cu[s]), int(cu[s + 1]), int(used[s])
        if q1 <= q0 or L <= 0:
            continue
        Tq_s = q1 - q0
        for g in range(Hkv):
            K = depage(k_cache, bt[s], L, g)
            V = depage(v_cache, bt[s], L, g)
            Q = qd[q0:q1, g * G:(g + 1) * G, :].reshape(Tq_s * G, 128)
            S = scale * (Q @ K.T)  # [Tq_s*G, L]
            if causal:
                qpos = L - Tq_s + np.repeat(np.arange(Tq_s), G)
                S = np.where(np.arange(L)[None, :] <= qpos[:, None], S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            m = np.where(np.isfinite(m), m, 0.0)
            W = np.exp(S - m)
            tot = W.sum(axis=1, keepdims=True)
            O = (W @ V) / np.where(tot > 0, tot, 1.0)
            O[~ok] = 0.0
            l = np.where(ok, m[:, 0] + np.log(np.where(tot[:, 0] > 0, tot[:, 0], 1.0)), -np.inf)
            out[q0:q1, g * G:(g + 1) * G, :] = O.reshape(Tq_s, G, 128)
            lse[g * G:(g + 1) * G, q0:q1] = l.reshape(Tq_s, G).T
    return out, lse
