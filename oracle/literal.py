"""Second oracle: the attention definition in pure-Python loops -- TEST INFRASTRUCTURE.

For tiny inputs only (a few tokens, a few hundred keys). It is written
independently of ``msa_oracle.c`` to cross-check it: values are converted to
fp64 by torch's own dtype conversion, the key set is built with a Python set,
and every sum is an explicit loop. Follows fw-ai/minimax-kernels README,
intro (each query attends only to the keys of the blocks it selected) and
"Quick start" (paged cache [pages, Hkv, page_size, 128], page table, output
[Tq, Hq, 128], fp32 LSE [Hq, Tq]).
"""
from __future__ import annotations

import math

import torch


def attention(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens,
              causal: bool, scale: float | None = None):
    qd = q.detach().cpu().double().tolist()
    kd = k_cache.detach().cpu().double()
    vd = v_cache.detach().cpu().double()
    sel = selected.detach().cpu().tolist()
    bt = block_tables.detach().cpu().tolist()
    cu = [int(x) for x in cu_seqlens_q.detach().cpu().tolist()]
    used = [int(x) for x in used_kv_lens.detach().cpu().tolist()]
    Tq, Hq = len(qd), len(qd[0]) if len(qd) else 0
    Hkv, P = kd.shape[1], kd.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(128.0)
    out = [[[0.0] * 128 for _ in range(Hq)] for _ in range(Tq)]
    lse = [[-math.inf] * Tq for _ in range(Hq)]
    for s in range(len(used)):
        L = used[s]
        Tq_s = cu[s + 1] - cu[s]
        nblk = (L + 127) // 128
        for t in range(cu[s], cu[s + 1]):
            pos = L - Tq_s + (t - cu[s])
            for h in range(Hq):
                g = h // G
                keys = set()
                for b in sel[t][g]:
                    if 0 <= b < nblk:
                        for j in range(128 * b, min(128 * b + 128, L)):
                            if (not causal) or j <= pos:
                                keys.add(j)
                if not keys:
                    continue
                J = sorted(keys)
                xs = []
                for j in J:
                    page = bt[s][j // P]
                    krow = kd[page, g, j % P].tolist()
                    xs.append(scale * sum(a * b for a, b in zip(qd[t][h], krow)))
                m = max(xs)
                ws = [math.exp(x - m) for x in xs]
                tot = sum(ws)
                lse[h][t] = m + math.log(tot)
                acc = [0.0] * 128
                for w, j in zip(ws, J):
                    page = bt[s][j // P]
                    vrow = vd[page, g, j % P].tolist()
                    for d in range(128):
                        acc[d] += w * vrow[d]
                out[t][h] = [a / tot for a in acc]
    return torch.tensor(out, dtype=torch.float64).numpy(), torch.tensor(lse, dtype=torch.float64).numpy()
