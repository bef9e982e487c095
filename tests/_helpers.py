"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

ATOL_O = 1e-2
RTOL_O = 1e-2
ATOL_LSE = 1e-3


def device_inputs(wl: W.Workload, dev="cuda", poison=None):
    k, v = W.kv_pool(wl, device=dev, poison=poison)
    return dict(
        q=wl.q.to(dev),
        k_cache=k,
        v_cache=v,
        selected=torch.from_numpy(wl.selected).to(dev),
        block_tables=torch.from_numpy(wl.block_tables).to(dev),
        cu_seqlens_q=torch.from_numpy(wl.cu_seqlens_q).to(dev),
        used_kv_lens=torch.from_numpy(wl.used_kv_lens).to(dev),
    )


def run_gpu(wl: W.Workload, inputs=None, dev="cuda"):
    import block_sparse_attention_selection_amd as msa

    inputs = inputs or device_inputs(wl, dev)
    out, lse = msa.kvouter_attention(
        inputs["q"], inputs["k_cache"], inputs["v_cache"], inputs["selected"], inputs["block_tables"],
        cu_seqlens_q=inputs["cu_seqlens_q"], used_kv_lens=inputs["used_kv_lens"],
        page_size=wl.page_size, causal=wl.causal, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def oracle_pairs(wl: W.Workload, pairs):
    """Oracle results for (t, g) pairs, one KV head at a time on a compacted cache.

    Returns ``out [n, G, 128]`` and ``lse [n, G]`` in fp64, in the order of ``pairs``.
    """
    import oracle

    pairs = np.asarray(pairs, dtype=np.int64)
    G = wl.G
    out = np.empty((pairs.size, G, 128))
    lse = np.empty((pairs.size, G))
    for g in np.unique(pairs % wl.Hkv):
        idx = np.nonzero(pairs % wl.Hkv == g)[0]
        toks = pairs[idx] // wl.Hkv
        k, v, bt = W.compact_cache(wl, heads=[int(g)])
        q = wl.q[:, g * G:(g + 1) * G, :].contiguous()
        sel = np.ascontiguousarray(wl.selected[:, g:g + 1, :])
        o, l = oracle.attention(q, k, v, sel, bt, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal,
                                pairs=toks)
        out[idx] = o
        lse[idx] = l
    return out, lse


def all_pairs(wl: W.Workload):
    return np.arange(wl.Tq * wl.Hkv, dtype=np.int64)


def sample_pairs(wl: W.Workload, n: int, seed=0):
    rng = np.random.default_rng(seed)
    tot = wl.Tq * wl.Hkv
    base = {0, tot - 1, (wl.Tq // 2) * wl.Hkv}
    # tokens at sequence boundaries
    for s in range(wl.B):
        for t in (wl.cu_seqlens_q[s], wl.cu_seqlens_q[s + 1] - 1):
            if 0 <= t < wl.Tq:
                base.add(int(t) * wl.Hkv + int(rng.integers(wl.Hkv)))
    extra = rng.choice(tot, size=min(n, tot), replace=False)
    return np.array(sorted(base | set(int(x) for x in extra)), dtype=np.int64)


def compare(wl: W.Workload, out, lse, pairs, ref_out, ref_lse):
    """Element-wise tolerance check; returns (max |dO|, max |dLSE|)."""
    G = wl.G
    pairs = np.asarray(pairs, dtype=np.int64)
    t = pairs // wl.Hkv
    g = pairs % wl.Hkv
    heads = g[:, None] * G + np.arange(G)[None, :]
    o = out.float().cpu().double().numpy()[t[:, None], heads]          # [n, G, 128]
    l = lse.cpu().double().numpy()[heads, t[:, None]]                  # [n, G]
    assert not np.isnan(o).any(), "NaN in output"
    assert not np.isnan(l).any(), "NaN in lse"
    err_o = np.abs(o - ref_out)
    bad = err_o > ATOL_O + RTOL_O * np.abs(ref_out)
    assert not bad.any(), f"out mismatch at {np.argwhere(bad)[:5].tolist()} max err {err_o.max():.3e}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), fin), "lse finiteness differs"
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse))
    err_l = np.abs(l[fin] - ref_lse[fin]) if fin.any() else np.zeros(1)
    assert err_l.max() <= ATOL_LSE, f"lse max err {err_l.max():.3e}"
    return float(err_o.max()), float(err_l.max())


def product_tiles(wl: W.Workload):
    """Tile and unit-window sizes the library uses for a prefill-shaped call:
    tiles of min(128, 256/G) tokens, windows of min(8 max(1, 128/G), 512)."""
    G = wl.G
    return min(128, max(1, 256 // G)), min(8 * max(1, 128 // G), 512)


def stratified_pairs(wl: W.Workload, per_tile: int = 3, seed: int = 0):
    """(t, g) pairs that reach every tile item of the tile kernel (the first,
    the last and random tokens of every tile, for every KV head) and every
    KV-outer window of the unit kernel (its first and last token), at the
    tile and window sizes the library uses. Every item of the work queues,
    whatever XCD range it falls in, is then compared."""
    from oracle import index_ref

    rng = np.random.default_rng(seed)
    T, Tu = product_tiles(wl)
    pairs = set()
    cu = wl.cu_seqlens_q
    for s in range(wl.B):
        for t0 in range(int(cu[s]), int(cu[s + 1]), T):
            t1 = min(t0 + T, int(cu[s + 1]))
            toks = {t0, t1 - 1} | set(int(x) for x in rng.integers(t0, t1, size=max(0, per_tile - 2)))
            for g in range(wl.Hkv):
                pairs.update(t * wl.Hkv + g for t in toks)
    nb_max = (wl.block_tables.shape[1] * wl.page_size + 127) // 128
    ref = index_ref.build(wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, T, Tu, nb_max, wl.G,
                          list_all_tiles=True)
    HK = wl.Hkv * wl.topk
    for r in range(ref.row_off.size - 1):
        a, b = int(ref.row_off[r]), int(ref.row_off[r + 1])
        for w0 in range(a, b, Tu):
            for e in (w0, min(w0 + Tu, b) - 1):
                slot = int(ref.ent[e])
                pairs.add((slot // HK) * wl.Hkv + (slot // wl.topk) % wl.Hkv)
    return np.array(sorted(pairs), dtype=np.int64)
