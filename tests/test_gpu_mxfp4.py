"""GPU parity of the pass over MXFP4 caches against the fp64 oracle (MI355X only).

The oracle sees the caches through its own decoder (oracle/mxfp4.py) as
exact fp32 values; tolerances are those of the other parity tests. Rows
beyond each sequence's used length carry the scale byte 0xFF (the format's
NaN), and pages nobody selects hold 0xFF codes and scales.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W

from _helpers import all_pairs, compare, oracle_pairs, sample_pairs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_selection_amd as msa

    msa.load()
    yield


def _reference(wl, heads=None):
    """The workload with its MXFP4 slices (of ``heads``) decoded to fp32."""
    from oracle import mxfp4

    keep = np.ones(len(wl.slice_head), bool) if heads is None else np.isin(wl.slice_head, heads)
    idx = torch.from_numpy(np.nonzero(keep)[0])

    def dec(codes, scales):
        return torch.from_numpy(mxfp4.dequantize(codes[idx].numpy(), scales[idx].numpy())).float()

    return dataclasses.replace(wl, kv_dtype=torch.float32, slice_page=wl.slice_page[keep],
                               slice_head=wl.slice_head[keep], k_vals=dec(wl.k_vals, wl.k_scales),
                               v_vals=dec(wl.v_vals, wl.v_scales), k_scales=None, v_scales=None)


def _run(wl, poison=None, block_tables=None):
    import block_sparse_attention_selection_amd as msa

    kc, ks, vc, vs = W.mxfp4_pool(wl, "cuda", poison)
    dev = lambda a: torch.from_numpy(a).cuda()
    bt = wl.block_tables if block_tables is None else block_tables
    out, lse = msa.kvouter_attention_mxfp4(
        wl.q.cuda(), kc, ks, vc, vs, dev(wl.selected), dev(bt), cu_seqlens_q=dev(wl.cu_seqlens_q),
        used_kv_lens=dev(wl.used_kv_lens), page_size=wl.page_size, causal=wl.causal, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


CASES = {
    # name: (tokens per sequence, used lengths, Hq, Hkv, page, top-k, causal, pick, pad_every)
    "gqa_page64_causal": ([1] * 9, [900, 2000, 700, 1500, 64, 129, 1, 4100, 3000], 16, 2, 64, 6, True, "random", 0),
    "gqa_page128": ([1] * 5, [300, 1000, 2049, 128, 777], 32, 4, 128, 8, False, "random", 0),
    "mqa_g32": ([1] * 6, [5000, 260, 1024, 3333, 90, 2000], 32, 1, 128, 8, True, "random", 0),
    "mqa_g64": ([1] * 4, [4096, 700, 1500, 2222], 64, 1, 64, 12, True, "random", 0),
    "pads_and_out_of_range": ([1] * 6, [1000, 2500, 333, 4000, 50, 1800], 16, 2, 64, 8, True, "oob", 3),
    # Tq == B, but not one token per sequence: every token is still its own tile
    "uneven_tokens": ([2, 0, 1, 1, 2, 1, 0], [1200, 900, 2000, 640, 3000, 129, 700], 16, 2, 64, 6, True,
                      "random", 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_parity_mxfp4_decode(name):
    tq, lens, Hq, Hkv, P, K, causal, pick, pad = CASES[name]
    wl = W.to_mxfp4(W.make_custom(2024 + len(name), tq, lens, Hq, Hkv, P, K, causal=causal, pick=pick,
                                  pad_every=pad))
    out, lse = _run(wl)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(_reference(wl), pairs)
    compare(wl, out, lse, pairs, ref_o, ref_l)


def test_parity_mxfp4_full_size_sampled():
    # the 256-sequence batch the bench times, on sampled (token, KV head) pairs
    wl = W.make("decode_fp4")
    out, lse = _run(wl)
    pairs = sample_pairs(wl, 96, seed=3)
    ref_o = np.empty((len(pairs), wl.G, 128))
    ref_l = np.empty((len(pairs), wl.G))
    for g in np.unique(pairs % wl.Hkv):
        idx = np.nonzero(pairs % wl.Hkv == g)[0]
        o, l = oracle_pairs(_reference(wl, heads=[int(g)]), pairs[idx])
        ref_o[idx], ref_l[idx] = o, l
    compare(wl, out, lse, pairs, ref_o, ref_l)


def test_mxfp4_zero_pool_outside_the_drawn_slices():
    # timing runs fill the rest of the pool with zeros instead of poison
    wl = W.to_mxfp4(W.make_custom(77, [1] * 5, [700, 1900, 256, 3000, 40], 16, 2, 128, 6, causal=True))
    out, lse = _run(wl, poison=False)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(_reference(wl), pairs)
    compare(wl, out, lse, pairs, ref_o, ref_l)


PREFILL = {
    # name: make_custom arguments
    "shared_chunks_with_residuals": dict(tq=[40, 30], lens=[3000, 2000], Hq=16, Hkv=2, P=128, K=8, pick="diag",
                                         shared_chunk=8, shared_picks=4),
    "varlen_mqa_like": dict(tq=[37, 5, 60], lens=[2500, 700, 4000], Hq=32, Hkv=1, P=128, K=8, pick="diag"),
    "page64_non_causal": dict(tq=[20, 12], lens=[1500, 900], Hq=16, Hkv=2, P=64, K=6, pick="random", causal=False),
    "one_token_tiles_g128": dict(tq=[1, 1, 1], lens=[2000, 700, 3100], Hq=128, Hkv=1, P=64, K=6, pick="random"),
    "decode_shaped_with_residuals": dict(tq=[2] * 160, lens=[300 + 37 * i for i in range(160)], Hq=16, Hkv=2, P=64,
                                         K=6, pick="random"),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_parity_mxfp4_unit_and_tile_paths(name):
    a = dict(PREFILL[name])
    wl = W.to_mxfp4(W.make_custom(3030 + len(name), a.pop("tq"), a.pop("lens"), a.pop("Hq"), a.pop("Hkv"), a.pop("P"),
                                  a.pop("K"), causal=a.pop("causal", True), **a))
    out, lse = _run(wl)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(_reference(wl), pairs)
    compare(wl, out, lse, pairs, ref_o, ref_l)


# Page ids outside the pool (past its end, or negative) hold no keys: the
# same result as the oracle with the picks of those blocks removed.
PAGE_CASES = {
    "decode": dict(tq=[1] * 8, lens=[900, 2000, 700, 1500, 1300, 640, 2500, 1100], Hq=16, Hkv=2, P=128, K=6,
                   pick="random"),
    "tiles": dict(tq=[40, 30], lens=[3000, 2000], Hq=16, Hkv=2, P=64, K=8, pick="diag", shared_chunk=16,
                  shared_picks=4),
}


@pytest.mark.parametrize("name", list(PAGE_CASES))
def test_mxfp4_pages_outside_the_pool_hold_no_keys(name):
    a = dict(PAGE_CASES[name])
    wl = W.to_mxfp4(W.make_custom(690 + len(name), a.pop("tq"), a.pop("lens"), a.pop("Hq"), a.pop("Hkv"),
                                  a.pop("P"), a.pop("K"), causal=True, **a))
    bt = wl.block_tables.copy()
    sel_ref = wl.selected.copy()
    cu = wl.cu_seqlens_q
    ppb = 128 // wl.page_size
    for s in range(wl.B):
        picks = wl.selected[cu[s]:cu[s + 1]]
        nblk = -(-int(wl.used_kv_lens[s]) // 128)
        valid = picks[(picks >= 0) & (picks < nblk)]
        if valid.size == 0:
            continue
        b = int(np.bincount(valid).argmax())  # the block most tokens of s picked
        for lp in range(b * ppb, min((b + 1) * ppb, bt.shape[1])):
            bt[s, lp] = wl.num_pages + 3 if s % 2 == 0 else -2
        sel_ref[cu[s]:cu[s + 1]][picks == b] = -1
    out, lse = _run(wl, block_tables=bt)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(_reference(dataclasses.replace(wl, selected=sel_ref)), pairs)
    compare(wl, out, lse, pairs, ref_o, ref_l)


def test_mxfp4_refuses_fp16_queries():
    import block_sparse_attention_selection_amd as msa

    wl = W.to_mxfp4(W.make_custom(78, [1, 1], [700, 900], 16, 2, 64, 4, causal=True))
    wl.q = wl.q.to(torch.float16)
    with pytest.raises(msa.MsaError) as e:
        _run(wl)
    assert e.value.code == -2


@pytest.mark.parametrize("name", ["gqa_page64_causal", "shared_chunks_with_residuals"])
def test_mxfp4_deterministic_bits(name):
    if name in CASES:
        tq, lens, Hq, Hkv, P, K, causal, pick, pad = CASES[name]
        wl = W.to_mxfp4(W.make_custom(2024 + len(name), tq, lens, Hq, Hkv, P, K, causal=causal, pick=pick,
                                      pad_every=pad))
    else:
        a = dict(PREFILL[name])
        wl = W.to_mxfp4(W.make_custom(3030 + len(name), a.pop("tq"), a.pop("lens"), a.pop("Hq"), a.pop("Hkv"),
                                      a.pop("P"), a.pop("K"), causal=a.pop("causal", True), **a))
    o1, l1 = _run(wl)
    o2, l2 = _run(wl)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
