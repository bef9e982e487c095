"""Seeded synthetic inputs for block-sparse attention (shared by tests, bench and smoke).

This module only draws inputs: sequence lengths, page tables, block
selections and N(0,1) values. It contains none of the attention arithmetic
and imports neither the oracle nor the GPU library.

Five named workloads (sizes and pick rules in ``CONFIGS`` below):
  tiny            1 seq, Tq=4, Hq=16, Hkv=1, L=512, page 64 (8 permuted pages),
                  2 of 4 blocks per (token, kv head), non-causal, bf16
  decode_gqa      64 seqs x 1 token, Hq=64, Hkv=8, L ~ U{8192..32768}, page 64,
                  last block + 15 uniform picks, causal, bf16
  prefill_shared  1 seq, Tq=L=16384, Hq=64, Hkv=8, page 128, top-k 16; chunks
                  of 64 queries share 12 of 16 picks, diagonal block always
                  picked, causal, bf16
  varlen_mqa      16 seqs, Tq_s lognormal (median 256, sigma 1) clipped to
                  [1, 2048], L = U{4096..131072} + Tq_s, Hq=32, Hkv=1, page 128,
                  top-k 32 (diagonal + 31 uniform), causal, fp16
  decode_fp8      256 seqs x 1 token, L=65536, Hq=64, Hkv=8, page 64, top-k 16
                  uniform picks, K/V e4m3fn (clamp to +-448 then cast), q bf16
  decode_mqa      256 seqs x 1 token, Hq=32, Hkv=1 (MQA), otherwise as
                  decode_gqa
  decode_fp4      decode_fp8's batch with MXFP4 K/V caches (below)
  prefill_fp4     prefill_shared's recipe with MXFP4 K/V caches

Values are float32 N(0,1) draws converted with torch: bf16 / fp16 by
round-to-nearest-even ``.to()``, e4m3fn by ``.clamp(-448, 448).to(...)``,
the cast rule stated in the sglang pull request "Speed up MiniMax-M3 sparse
attention on Hopper", section "Verification".

MXFP4 caches (``kv_dtype`` torch.uint8) hold, per K or V row, 64 bytes of
e2m1 codes drawn uniformly (every byte value) and 4 e8m0 scale bytes drawn
uniformly from MXFP4_SCALES, each from its own seeded stream; the poison of
such a row is the scale byte 0xFF. Their values are the oracle's to decode.

Only the (physical page, KV head) slices that some pick can touch receive
drawn values; the rest of the pool is filled on the device (NaN poison for
correctness runs, zeros for timing). Rows of a sequence's last page beyond
its used length are poisoned too when ``poison`` is set.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 128
HEAD_DIM = 128

_POISON_BITS = {torch.bfloat16: 0x7FC0, torch.float16: 0x7E00, torch.float8_e4m3fn: 0x7F,
                torch.float32: 0x7FC00000}

# e8m0 scale bytes of drawn MXFP4 rows (scales 2^-3 .. 2^0), and the poison
MXFP4_SCALES = (124, 125, 126, 127)
MXFP4_POISON = 0xFF

CONFIGS = {
    "tiny": dict(seed=1001),
    "decode_gqa": dict(seed=1002),
    "prefill_shared": dict(seed=1003),
    "varlen_mqa": dict(seed=1004),
    "decode_fp8": dict(seed=1005),
    "dense_causal": dict(seed=1006),
    "decode_mqa": dict(seed=1010),
    "decode_fp4": dict(seed=1011),
    "prefill_fp4": dict(seed=1012),
}


@dataclass
class Workload:
    name: str
    seed: int
    Hq: int
    Hkv: int
    page_size: int
    topk: int
    causal: bool
    q_dtype: torch.dtype
    kv_dtype: torch.dtype
    cu_seqlens_q: np.ndarray     # [B+1] int64
    used_kv_lens: np.ndarray     # [B] int32
    block_tables: np.ndarray     # [B, max_pages] int32 (-1 = unused)
    selected: np.ndarray         # [Tq, Hkv, topk] int32
    num_pages: int
    q: torch.Tensor              # [Tq, Hq, 128] cpu
    slice_page: np.ndarray       # [n] physical page of each drawn slice
    slice_head: np.ndarray       # [n] kv head of each drawn slice
    k_vals: torch.Tensor         # [n, page_size, 128] cpu, kv_dtype
    v_vals: torch.Tensor
    poison: bool = True
    meta: dict = field(default_factory=dict)
    k_scales: torch.Tensor | None = None  # MXFP4 caches: [n, page_size, 4] e8m0 bytes
    v_scales: torch.Tensor | None = None

    @property
    def mxfp4(self):
        return self.kv_dtype == torch.uint8

    @property
    def B(self):
        return int(self.used_kv_lens.shape[0])

    @property
    def Tq(self):
        return int(self.q.shape[0])

    @property
    def G(self):
        return self.Hq // self.Hkv


# ----------------------------------------------------------------------------
# value conversion
# ----------------------------------------------------------------------------
def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == torch.float8_e4m3fn:
        return t.clamp(-448, 448).to(torch.float8_e4m3fn)
    return t.to(dtype)


def filled(shape, dtype: torch.dtype, poison: bool, device="cpu") -> torch.Tensor:
    """A tensor of the given dtype filled with NaN poison or zeros."""
    if dtype == torch.float8_e4m3fn:
        raw = torch.full(shape, _POISON_BITS[dtype] if poison else 0, dtype=torch.uint8, device=device)
        return raw.view(torch.float8_e4m3fn)
    if dtype == torch.float32:
        raw = torch.full(shape, _POISON_BITS[dtype] if poison else 0, dtype=torch.int32, device=device)
        return raw.view(dtype)
    raw = torch.full(shape, _POISON_BITS[dtype] if poison else 0, dtype=torch.int16, device=device)
    return raw.view(dtype)


# ----------------------------------------------------------------------------
# structure helpers
# ----------------------------------------------------------------------------
def _page_tables(rng, used, page_size, max_pages=None, extra_pages=0):
    """Random permutation of every page the sequences need, handed out in order."""
    npages = [(int(L) + page_size - 1) // page_size for L in used]
    total = int(sum(npages)) + int(extra_pages)
    perm = rng.permutation(total).astype(np.int32)
    MP = max(npages) if max_pages is None else max_pages
    MP = max(MP, 1)
    bt = np.full((len(used), MP), -1, dtype=np.int32)
    off = 0
    for s, n in enumerate(npages):
        bt[s, :n] = perm[off:off + n]
        off += n
    return bt, total


def _draw_slices(seed, wl_pages, wl_heads, page_size, kv_dtype, poison_rows=None):
    n = len(wl_pages)
    kr = np.random.default_rng([seed, 2])
    vr = np.random.default_rng([seed, 3])
    kv = []
    for r in (kr, vr):
        out = torch.empty((n, page_size, HEAD_DIM), dtype=kv_dtype)
        step = max(1, (1 << 24) // (page_size * HEAD_DIM))
        for i in range(0, n, step):
            x = r.standard_normal((min(step, n - i), page_size, HEAD_DIM), dtype=np.float32)
            out[i:i + x.shape[0]] = to_dtype(x, kv_dtype)
        if poison_rows is not None:
            bits = out.view(torch.uint8) if kv_dtype == torch.float8_e4m3fn else out.view(torch.int16)
            for i, first_bad in poison_rows:
                bits[i, first_bad:] = _POISON_BITS[kv_dtype]
        kv.append(out)
    return kv[0], kv[1]


def _draw_mxfp4(seed, n, page_size, poison_rows=None):
    """MXFP4 codes [n, P, 64] and scales [n, P, 4] of K, then of V."""
    out = []
    for stream in (4, 5):
        r = np.random.default_rng([seed, stream])
        codes = torch.from_numpy(r.integers(0, 256, size=(n, page_size, HEAD_DIM // 2), dtype=np.uint8))
        scales = torch.from_numpy(r.choice(np.asarray(MXFP4_SCALES, dtype=np.uint8), size=(n, page_size, 4)))
        if poison_rows is not None:
            for i, first_bad in poison_rows:
                scales[i, first_bad:] = MXFP4_POISON
        out.append((codes, scales))
    return out


def needed_slices(block_tables, used, selected, cu, page_size, Hkv, all_pages=False, num_pages=0):
    """(page, head) slices that some pick with 0 <= b < ceil(L/128) can read."""
    if all_pages:
        pages = np.repeat(np.arange(num_pages), Hkv)
        heads = np.tile(np.arange(Hkv), num_pages)
        return pages.astype(np.int64), heads.astype(np.int64)
    keys = set()
    Tq = selected.shape[0]
    cu = np.asarray(cu)
    for s in range(len(used)):
        L = int(used[s])
        nblk = (L + BLOCK - 1) // BLOCK
        q0, q1 = int(cu[s]), int(cu[s + 1])
        if q1 <= q0:
            continue
        picks = selected[q0:q1]  # [Tq_s, Hkv, K]
        for g in range(Hkv):
            for b in np.unique(picks[:, g, :]):
                b = int(b)
                if b < 0 or b >= nblk:
                    continue
                lp0 = (BLOCK * b) // page_size
                lp1 = (min(BLOCK * b + BLOCK, L) + page_size - 1) // page_size
                for lp in range(lp0, lp1):
                    keys.add((int(block_tables[s, lp]), g))
    arr = np.array(sorted(keys), dtype=np.int64).reshape(-1, 2)
    return arr[:, 0], arr[:, 1]


def _poison_rows(slice_page, block_tables, used, page_size):
    """Slices holding rows at or beyond a sequence's used length."""
    owner = {}
    for s in range(block_tables.shape[0]):
        L = int(used[s])
        n = (L + page_size - 1) // page_size
        if n and L % page_size:
            owner[int(block_tables[s, n - 1])] = L % page_size
    return [(i, owner[int(p)]) for i, p in enumerate(slice_page) if int(p) in owner]


def assemble(name, seed, Hq, Hkv, page_size, topk, causal, q_dtype, kv_dtype, cu, used, bt,
             selected, num_pages, poison=True, all_pages=False, meta=None):
    cu = np.asarray(cu, dtype=np.int64)
    used = np.asarray(used, dtype=np.int32)
    selected = np.ascontiguousarray(selected, dtype=np.int32)
    Tq = int(selected.shape[0])
    qr = np.random.default_rng([seed, 1])
    q = to_dtype(qr.standard_normal((Tq, Hq, HEAD_DIM), dtype=np.float32), q_dtype)
    pages, heads = needed_slices(bt, used, selected, cu, page_size, Hkv, all_pages, num_pages)
    prow = _poison_rows(pages, bt, used, page_size) if poison else None
    ks = vs = None
    if kv_dtype == torch.uint8:  # MXFP4
        (kv, ks), (vv, vs) = _draw_mxfp4(seed, len(pages), page_size, prow)
    else:
        kv, vv = _draw_slices(seed, pages, heads, page_size, kv_dtype, prow)
    return Workload(name=name, seed=seed, Hq=Hq, Hkv=Hkv, page_size=page_size, topk=topk,
                    causal=causal, q_dtype=q_dtype, kv_dtype=kv_dtype, cu_seqlens_q=cu,
                    used_kv_lens=used, block_tables=bt, selected=selected, num_pages=num_pages,
                    q=q, slice_page=pages, slice_head=heads, k_vals=kv, v_vals=vv,
                    poison=poison, meta=dict(meta or {}), k_scales=ks, v_scales=vs)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
def make_tiny(seed=1001, poison=True):
    rng = np.random.default_rng(seed)
    L, P = 512, 64
    bt = rng.permutation(8).astype(np.int32)[None, :]
    sel = np.stack([rng.permutation(4)[:2] for _ in range(4 * 1)]).reshape(4, 1, 2)
    return assemble("tiny", seed, 16, 1, P, 2, False, torch.bfloat16, torch.bfloat16,
                    [0, 4], [L], bt, sel, 8, poison, all_pages=True)


def make_decode_gqa(seed=1002, poison=True, batch=64):
    rng = np.random.default_rng(seed)
    P, Hkv, K = 64, 8, 16
    used = rng.integers(8192, 32768, size=batch, endpoint=True).astype(np.int32)
    bt, NP = _page_tables(rng, used, P, max_pages=32768 // P)
    sel = np.empty((batch, Hkv, K), dtype=np.int32)
    for s in range(batch):
        nblk = (int(used[s]) + BLOCK - 1) // BLOCK
        for g in range(Hkv):
            picks = np.concatenate([[nblk - 1], rng.choice(nblk - 1, size=K - 1, replace=False)])
            sel[s, g] = rng.permutation(picks)
    return assemble("decode_gqa", seed, 64, Hkv, P, K, True, torch.bfloat16, torch.bfloat16,
                    np.arange(batch + 1), used, bt, sel, NP, poison)


def make_decode_mqa(seed=1010, poison=True, batch=256, Hq=32):
    """MQA decode: batch sequences x 1 query token, Hq query heads on one KV
    head, L ~ U{8192..32768}, page 64, last block + 15 uniform picks,
    causal, bf16 (decode_gqa's lengths and picks with Hkv = 1)."""
    rng = np.random.default_rng(seed)
    P, Hkv, K = 64, 1, 16
    used = rng.integers(8192, 32768, size=batch, endpoint=True).astype(np.int32)
    bt, NP = _page_tables(rng, used, P, max_pages=32768 // P)
    sel = np.empty((batch, Hkv, K), dtype=np.int32)
    for s in range(batch):
        nblk = (int(used[s]) + BLOCK - 1) // BLOCK
        picks = np.concatenate([[nblk - 1], rng.choice(nblk - 1, size=K - 1, replace=False)])
        sel[s, 0] = rng.permutation(picks)
    return assemble("decode_mqa", seed, Hq, Hkv, P, K, True, torch.bfloat16, torch.bfloat16,
                    np.arange(batch + 1), used, bt, sel, NP, poison)


def make_prefill_shared(seed=1003, poison=True, seqlen=16384):
    rng = np.random.default_rng(seed)
    P, Hkv, K, C = 128, 8, 16, 64
    T = L = seqlen
    bt, NP = _page_tables(rng, [L], P)
    sel = np.full((T, Hkv, K), -1, dtype=np.int32)
    for c in range(T // C):
        d = (C * c) // BLOCK
        for g in range(Hkv):
            shared = [d] + list(rng.choice(d, size=min(11, d), replace=False)) if d > 0 else [d]
            rest = np.setdiff1d(np.arange(d + 1), shared)
            for i in range(C):
                t = C * c + i
                n_extra = min(4, d + 1 - len(shared))
                extra = list(rng.choice(rest, size=n_extra, replace=False)) if n_extra > 0 else []
                picks = rng.permutation(np.array(shared + extra, dtype=np.int64))
                sel[t, g, :picks.size] = picks
    return assemble("prefill_shared", seed, 64, Hkv, P, K, True, torch.bfloat16, torch.bfloat16,
                    [0, T], [L], bt, sel, NP, poison, all_pages=True)


def make_varlen_mqa(seed=1004, poison=True, batch=16):
    rng = np.random.default_rng(seed)
    P, K = 128, 32
    tq = np.clip(np.rint(np.exp(rng.normal(np.log(256.0), 1.0, size=batch))), 1, 2048).astype(np.int64)
    prefix = rng.integers(4096, 131072, size=batch, endpoint=True)
    used = (prefix + tq).astype(np.int32)
    bt, NP = _page_tables(rng, used, P)
    cu = np.concatenate([[0], np.cumsum(tq)]).astype(np.int64)
    sel = np.empty((int(cu[-1]), 1, K), dtype=np.int32)
    for s in range(batch):
        for i in range(int(tq[s])):
            pos = int(used[s]) - int(tq[s]) + i
            d = pos // BLOCK
            picks = np.concatenate([[d], rng.choice(d, size=K - 1, replace=False)])
            sel[cu[s] + i, 0] = rng.permutation(picks)
    return assemble("varlen_mqa", seed, 32, 1, P, K, True, torch.float16, torch.float16,
                    cu, used, bt, sel, NP, poison, all_pages=True)


def make_decode_fp8(seed=1005, poison=True, batch=256):
    rng = np.random.default_rng(seed)
    P, Hkv, K, L = 64, 8, 16, 65536
    used = np.full(batch, L, dtype=np.int32)
    bt, NP = _page_tables(rng, used, P)
    nblk = L // BLOCK
    sel = np.empty((batch, Hkv, K), dtype=np.int32)
    for s in range(batch):
        for g in range(Hkv):
            sel[s, g] = rng.permutation(rng.choice(nblk, size=K, replace=False))
    return assemble("decode_fp8", seed, 64, Hkv, P, K, True, torch.bfloat16, torch.float8_e4m3fn,
                    np.arange(batch + 1), used, bt, sel, NP, poison)


def make_decode_fp4(seed=1011, poison=True, batch=256):
    """decode_fp8's batch (256 seqs x 1 token, L=65536, Hq=64, Hkv=8, page
    64, top-k 16 uniform picks, causal, q bf16) with MXFP4 K/V caches."""
    rng = np.random.default_rng(seed)
    P, Hkv, K, L = 64, 8, 16, 65536
    used = np.full(batch, L, dtype=np.int32)
    bt, NP = _page_tables(rng, used, P)
    nblk = L // BLOCK
    sel = np.empty((batch, Hkv, K), dtype=np.int32)
    for s in range(batch):
        for g in range(Hkv):
            sel[s, g] = rng.permutation(rng.choice(nblk, size=K, replace=False))
    return assemble("decode_fp4", seed, 64, Hkv, P, K, True, torch.bfloat16, torch.uint8,
                    np.arange(batch + 1), used, bt, sel, NP, poison)


def make_prefill_fp4(seed=1012, poison=True):
    """prefill_shared's recipe (seed 1012) with MXFP4 K/V caches."""
    wl = to_mxfp4(make_prefill_shared(seed=seed, poison=poison))
    wl.name = "prefill_fp4"
    return wl


def make_dense_causal(seed=1006, poison=True, seqlen=8192):
    """Dense causal attention as the case where every visible block is
    selected: 1 sequence, Tq = L = seqlen, Hq 64, Hkv 8, page 128, top-64
    (every block a token can see), bf16."""
    rng = np.random.default_rng(seed)
    P, Hkv, K = 128, 8, 64
    T = L = seqlen
    assert (L + BLOCK - 1) // BLOCK <= K, "every block must fit in the top-k"
    bt, NP = _page_tables(rng, [L], P)
    sel = np.full((T, Hkv, K), -1, dtype=np.int32)
    for t in range(T):
        vis = t // BLOCK + 1
        sel[t, :, :vis] = np.arange(vis, dtype=np.int32)
    return assemble("dense_causal", seed, 64, Hkv, P, K, True, torch.bfloat16, torch.bfloat16,
                    [0, T], [L], bt, sel, NP, poison, all_pages=True)


MAKERS = {
    "tiny": make_tiny,
    "decode_gqa": make_decode_gqa,
    "prefill_shared": make_prefill_shared,
    "varlen_mqa": make_varlen_mqa,
    "decode_fp8": make_decode_fp8,
    "dense_causal": make_dense_causal,
    "decode_fp4": make_decode_fp4,
    "prefill_fp4": make_prefill_fp4,
    "decode_mqa": make_decode_mqa,
}


def make(name: str, seed: int | None = None, poison: bool = True, **kw) -> Workload:
    if seed is None:
        seed = CONFIGS[name]["seed"]
    return MAKERS[name](seed=seed, poison=poison, **kw)


# ----------------------------------------------------------------------------
# small custom workloads for edge cases
# ----------------------------------------------------------------------------
def make_custom(seed, tq_per_seq, kv_lens, Hq, Hkv, page_size, topk, causal=False,
                q_dtype=torch.bfloat16, kv_dtype=None, pick="random", pad_every=0,
                extra_pages=3, poison=True, max_pages=None, shared_chunk=0, shared_picks=0):
    """Small workloads with a chosen pick rule.

    pick: "random"  -- up to topk distinct uniform picks among the blocks a
                       token can see (all blocks when non-causal), -1 pads
          "all"     -- every visible block (topk must be large enough)
          "diag"    -- the token's own block plus random others
          "oob"     -- like random, plus ids >= nblk and negative ids
    pad_every: every n-th slot is forced to -1.
    shared_chunk/shared_picks: tokens in chunks of shared_chunk share that
                       many picks (drawn per chunk and kv head).
    """
    rng = np.random.default_rng(seed)
    kv_dtype = kv_dtype or q_dtype
    tq = np.asarray(tq_per_seq, dtype=np.int64)
    used = np.asarray(kv_lens, dtype=np.int32)
    bt, NP = _page_tables(rng, used, page_size, max_pages=max_pages, extra_pages=extra_pages)
    cu = np.concatenate([[0], np.cumsum(tq)]).astype(np.int64)
    Tq = int(cu[-1])
    sel = np.full((Tq, Hkv, topk), -1, dtype=np.int32)
    for s in range(len(tq)):
        L = int(used[s])
        nblk = (L + BLOCK - 1) // BLOCK
        shared = {}
        for i in range(int(tq[s])):
            t = int(cu[s]) + i
            pos = L - int(tq[s]) + i
            vis = nblk if not causal else max(0, min(nblk, pos // BLOCK + 1)) if pos >= 0 else 0
            for g in range(Hkv):
                if pick == "all":
                    picks = list(range(vis))[:topk]
                else:
                    base = []
                    if shared_chunk and vis > 0:
                        key = (i // shared_chunk, g)
                        if key not in shared:
                            shared[key] = list(rng.choice(vis, size=min(shared_picks, vis), replace=False))
                        base = [b for b in shared[key] if b < vis]
                    if pick == "diag" and vis > 0 and (vis - 1) not in base:
                        base = [vis - 1] + base
                    rest = np.setdiff1d(np.arange(vis), base)
                    n = min(topk - len(base), rest.size)
                    picks = base + (list(rng.choice(rest, size=n, replace=False)) if n > 0 else [])
                    if pick == "oob":
                        picks = picks[:max(0, topk - 2)] + [nblk + int(rng.integers(0, 5)), -int(rng.integers(1, 4))]
                    picks = list(rng.permutation(np.array(picks, dtype=np.int64)))
                row = np.full(topk, -1, dtype=np.int32)
                row[:len(picks)] = picks[:topk]
                if pad_every:
                    row[::pad_every] = -1
                sel[t, g] = row
    return assemble("custom", seed, Hq, Hkv, page_size, topk, causal, q_dtype, kv_dtype,
                    cu, used, bt, sel, NP, poison, all_pages=True)


# ----------------------------------------------------------------------------
# materialisation
# ----------------------------------------------------------------------------
def to_mxfp4(wl: Workload) -> Workload:
    """The same workload with MXFP4 caches: every drawn slice's K and V rows
    get fresh MXFP4 draws (seeded by the workload's seed)."""
    import dataclasses

    prow = _poison_rows(wl.slice_page, wl.block_tables, wl.used_kv_lens, wl.page_size) if wl.poison else None
    (kc, ks), (vc, vs) = _draw_mxfp4(wl.seed, len(wl.slice_page), wl.page_size, prow)
    return dataclasses.replace(wl, kv_dtype=torch.uint8, k_vals=kc, v_vals=vc, k_scales=ks, v_scales=vs)


def mxfp4_pool(wl: Workload, device="cpu", poison=None):
    """Full MXFP4 pools on ``device``: codes [num_pages, Hkv, P, 64] and
    scales [num_pages, Hkv, P, 4] of K, then of V. Slices nobody draws hold
    code and scale bytes 0xFF (poison) or zeros."""
    assert wl.mxfp4
    poison = wl.poison if poison is None else poison
    fill = MXFP4_POISON if poison else 0
    out = []
    for vals, sc in ((wl.k_vals, wl.k_scales), (wl.v_vals, wl.v_scales)):
        codes = torch.full((wl.num_pages, wl.Hkv, wl.page_size, HEAD_DIM // 2), fill, dtype=torch.uint8,
                           device=device)
        scales = torch.full((wl.num_pages, wl.Hkv, wl.page_size, 4), fill, dtype=torch.uint8, device=device)
        if len(wl.slice_page):
            pg = torch.from_numpy(wl.slice_page).to(device)
            hd = torch.from_numpy(wl.slice_head).to(device)
            codes[pg, hd] = vals.to(device)
            scales[pg, hd] = sc.to(device)
        out += [codes, scales]
    return tuple(out)


def kv_pool(wl: Workload, device="cpu", poison=None):
    """Full [num_pages, Hkv, P, 128] K and V pools on ``device``."""
    assert not wl.mxfp4, "MXFP4 workloads: mxfp4_pool"
    poison = wl.poison if poison is None else poison
    shape = (wl.num_pages, wl.Hkv, wl.page_size, HEAD_DIM)
    k = filled(shape, wl.kv_dtype, poison, device)
    v = filled(shape, wl.kv_dtype, poison, device)
    if len(wl.slice_page):
        pg = torch.from_numpy(wl.slice_page).to(device)
        hd = torch.from_numpy(wl.slice_head).to(device)
        _bits(k)[pg, hd] = _bits(wl.k_vals.to(device))
        _bits(v)[pg, hd] = _bits(wl.v_vals.to(device))
    return k, v


_BIT_VIEWS = {1: torch.uint8, 2: torch.int16, 4: torch.int32}


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(_BIT_VIEWS[x.element_size()])


def compact_cache(wl: Workload, heads=None):
    """CPU cache holding only the drawn slices of ``heads``, with a remapped table.

    Returns ``(k, v, block_tables)`` with ``k``/``v`` of shape
    [n_pages, len(heads), P, 128]; table entries of pages that hold no drawn
    slice become -1. Renumbering physical pages together with the table
    leaves every result unchanged.
    """
    heads = list(range(wl.Hkv)) if heads is None else list(heads)
    hsel = np.isin(wl.slice_head, heads)
    pages = np.unique(wl.slice_page[hsel])
    remap = np.full(wl.num_pages, -1, dtype=np.int64)
    remap[pages] = np.arange(pages.size)
    shape = (pages.size, len(heads), wl.page_size, HEAD_DIM)
    k = filled(shape, wl.kv_dtype, True)
    v = filled(shape, wl.kv_dtype, True)
    hpos = np.full(wl.Hkv, -1, dtype=np.int64)
    hpos[heads] = np.arange(len(heads))
    idx = np.nonzero(hsel)[0]
    pg = torch.from_numpy(remap[wl.slice_page[idx]])
    hd = torch.from_numpy(hpos[wl.slice_head[idx]])
    _bits(k)[pg, hd] = _bits(wl.k_vals[torch.from_numpy(idx)])
    _bits(v)[pg, hd] = _bits(wl.v_vals[torch.from_numpy(idx)])
    bt = wl.block_tables.astype(np.int64)
    bt_c = np.where(bt >= 0, remap[np.clip(bt, 0, None)], -1).astype(np.int32)
    return k, v, bt_c


# ----------------------------------------------------------------------------
# block selection inputs: index queries and a paged index K cache
# ----------------------------------------------------------------------------
@dataclass
class SelectionInputs:
    name: str
    seed: int
    page_size: int
    causal: bool
    topk: int
    cu_seqlens_q: np.ndarray     # [B+1] int64
    used_kv_lens: np.ndarray     # [B] int32
    block_tables: np.ndarray     # [B, max_pages] int32 (-1 = unused)
    q_idx: torch.Tensor          # [Tq, Hkv, 128] cpu, 16-bit
    k_idx: torch.Tensor          # [num_pages, Hkv, P, 128] cpu, q's dtype or e4m3fn

    @property
    def Tq(self):
        return int(self.cu_seqlens_q[-1])

    @property
    def Hkv(self):
        return int(self.q_idx.shape[1])


SELECT_CONFIGS = {
    "select_decode": dict(seed=1008),
    "select_prefill": dict(seed=1009),
}


def make_selection(seed, tq_per_seq, kv_lens, Hkv, page_size, topk, causal=True, q_dtype=torch.bfloat16,
                   key_dtype=None, poison=True, extra_pages=2, name="custom"):
    """Index queries and keys, N(0,1), for sequences of the given query and key counts.

    Every page a sequence needs is drawn (the selection reads all of its
    keys), one seeded stream per sequence; rows at or beyond a sequence's
    length, and the extra pages no table lists, hold NaN poison (zeros when
    ``poison`` is off).
    """
    key_dtype = key_dtype or q_dtype
    rng = np.random.default_rng([seed, 0])
    used = np.asarray(kv_lens, dtype=np.int32)
    tq = np.asarray(tq_per_seq, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(tq)]).astype(np.int64)
    bt, NP = _page_tables(rng, used, page_size, extra_pages=extra_pages)
    k_idx = filled((NP, Hkv, page_size, HEAD_DIM), key_dtype, poison)
    for s, L in enumerate(used):
        n = (int(L) + page_size - 1) // page_size
        if n == 0:
            continue
        gen = torch.Generator().manual_seed(int(seed) * 1_000_003 + 7919 * (s + 1))
        vals = torch.randn((int(L), Hkv, HEAD_DIM), generator=gen)
        rows = vals.clamp(-448, 448).to(key_dtype) if key_dtype == torch.float8_e4m3fn else vals.to(key_dtype)
        full = filled((n * page_size, Hkv, HEAD_DIM), key_dtype, poison)
        full[:L] = rows
        k_idx[torch.from_numpy(bt[s, :n].astype(np.int64))] = full.view(n, page_size, Hkv, HEAD_DIM).transpose(1, 2)
    q = np.random.default_rng([seed, 2]).standard_normal((int(cu[-1]), Hkv, HEAD_DIM), dtype=np.float32)
    return SelectionInputs(name, seed, page_size, causal, topk, cu, used, bt, to_dtype(q, q_dtype), k_idx)


def make_select_decode(seed=1008, poison=True, batch=64):
    """64 decode tokens (one per sequence), L ~ U{8192..32768}, Hkv 8, page 64,
    fp8 e4m3fn index keys, bf16 index queries, top-16, causal."""
    rng = np.random.default_rng([seed, 9])
    used = rng.integers(8192, 32769, size=batch)
    return make_selection(seed, np.ones(batch, np.int64), used, 8, 64, 16, True, torch.bfloat16,
                          torch.float8_e4m3fn, poison, name="select_decode")


def make_select_prefill(seed=1009, poison=True, seqlen=8192):
    """One sequence of seqlen tokens, all of them queries, Hkv 8, page 128, bf16
    index keys and queries, top-16, causal."""
    return make_selection(seed, [seqlen], [seqlen], 8, 128, 16, True, torch.bfloat16, torch.bfloat16,
                          poison, name="select_prefill")


SELECT_MAKERS = {"select_decode": make_select_decode, "select_prefill": make_select_prefill}
