"""GPU parity of block selection (msa_select_blocks) against oracle/select_ref.

Three comparisons per case:
  * the kernel's fp32 block scores against the oracle's fp64 scores, within
    |d| <= 1e-3 + 1e-4 |s| (a 128-term fp32 dot product of bf16 / e4m3fn
    values carries a relative error near 2^-24 * 128 of the magnitudes);
    blocks without a visible key are -inf on both sides;
  * the kernel's selection against the oracle's top-k taken on the kernel's
    own fp32 scores: bit-exact (both decide in fp32);
  * the kernel's selection against the oracle's fp64 top-k: every pick valid
    and distinct, the local block first, and no unpicked visible block
    scoring above a picked one by more than the score tolerance.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import decode as odecode
from oracle import select_ref as R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_selection_amd as msa

    msa.load()
    yield


def _run(si: W.SelectionInputs, force_local=True, topk=None):
    import block_sparse_attention_selection_amd as msa

    dev = torch.device("cuda:0")
    sel, sc = msa.select_blocks(si.q_idx.to(dev), si.k_idx.to(dev), torch.from_numpy(si.block_tables).to(dev),
                                cu_seqlens_q=torch.from_numpy(si.cu_seqlens_q).to(dev),
                                used_kv_lens=torch.from_numpy(si.used_kv_lens).to(dev),
                                page_size=si.page_size, topk=topk or si.topk, causal=si.causal,
                                force_local=force_local, return_scores=True)
    # without a score output the library keeps the table in its workspace
    sel2 = msa.select_blocks(si.q_idx.to(dev), si.k_idx.to(dev), torch.from_numpy(si.block_tables).to(dev),
                             cu_seqlens_q=torch.from_numpy(si.cu_seqlens_q).to(dev),
                             used_kv_lens=torch.from_numpy(si.used_kv_lens).to(dev),
                             page_size=si.page_size, topk=topk or si.topk, causal=si.causal,
                             force_local=force_local)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    return sel.cpu().numpy(), sc.cpu().numpy()


def _tol(s):
    return 1e-3 + 1e-4 * np.abs(s)


def _check(si, sel, sc, ref_sc, topk, force_local, tokens=None):
    cu, used = si.cu_seqlens_q, si.used_kv_lens
    rows = np.arange(si.Tq) if tokens is None else np.asarray(tokens)
    g_sc, o_sc = sc[rows], ref_sc[rows]
    inf_g, inf_o = np.isneginf(g_sc), np.isneginf(o_sc)
    assert np.array_equal(inf_g, inf_o), "blocks without a visible key differ"
    fin = ~inf_o
    err = np.abs(g_sc[fin] - o_sc[fin])
    assert np.all(err <= _tol(o_sc[fin])), f"score error {err.max():.3e}"
    # the same decision in the same precision: bit-exact
    want = R.select_topk(sc.astype(np.float32), topk, cu, used, si.causal, force_local)
    assert np.array_equal(sel[rows], want[rows])
    # against the fp64 scores: valid, and the best within the tolerance
    seq, pos = R._positions(cu, used, si.Tq, si.causal)
    for t in rows:
        for g in range(si.Hkv):
            picks = [int(b) for b in sel[t, g] if b >= 0]
            assert all(b == -1 for b in sel[t, g, len(picks):])
            vis = np.nonzero(ref_sc[t, g] > -np.inf)[0]
            assert len(set(picks)) == len(picks) and set(picks) <= set(vis.tolist())
            assert len(picks) == min(topk, len(vis))
            if force_local and len(vis):
                assert picks[0] == pos[t] // 128
            rest = sorted(set(vis.tolist()) - set(picks))
            free = picks[1:] if force_local else picks
            if rest and free:
                lo = min(ref_sc[t, g, b] for b in free)
                hi = max(ref_sc[t, g, b] for b in rest)
                assert hi <= lo + 2 * _tol(max(abs(lo), abs(hi))), (t, g, lo, hi)


def _oracle_scores(si, tokens=None):
    q = odecode(si.q_idx)
    k = odecode(si.k_idx)
    return R.block_scores(q, k, si.block_tables, si.cu_seqlens_q, si.used_kv_lens, si.page_size, si.causal,
                          tokens=tokens)


CASES = [
    # (tq per seq, kv lens, Hkv, page, topk, causal, key dtype)
    ([1, 37, 70], [300, 2000, 5000], 2, 64, 8, True, torch.bfloat16),       # 16-token tiles, ragged
    ([1, 37, 70], [300, 2000, 5000], 2, 128, 8, False, torch.bfloat16),
    ([1, 37, 70], [300, 2000, 5000], 2, 64, 8, True, torch.float8_e4m3fn),
    ([200, 130], [1500, 4100], 1, 128, 12, True, torch.bfloat16),           # 64-token tiles (Tq > 4B)
    ([200, 130], [1500, 4100], 3, 64, 5, True, torch.float8_e4m3fn),
    ([3, 0, 5, 1], [129, 700, 0, 64], 2, 64, 40, True, torch.bfloat16),     # empty seqs, topk > blocks
    ([2, 3], [10000, 9000], 1, 64, 8, True, torch.float8_e4m3fn),          # 65..128 blocks a row
    ([1, 2], [100000, 20000], 1, 128, 16, True, torch.bfloat16),           # up to 782 blocks a row
    ([1, 1, 1, 1, 1], [3000, 200, 129, 128, 5000], 16, 128, 1, False, torch.float8_e4m3fn),  # 16 heads, top-1
    ([2], [128000], 1, 64, 16, True, torch.float8_e4m3fn),                 # 1000 blocks a row
    ([1, 1], [133120, 40000], 1, 128, 32, True, torch.bfloat16),           # 1040 blocks: varlen_mqa's longest
    ([1, 2], [256000, 3000], 1, 128, 16, False, torch.float8_e4m3fn),       # 2000 blocks, non-causal
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_select_matches_oracle(case):
    tq, lens, Hkv, P, topk, causal, kdt = CASES[case]
    si = W.make_selection(300 + case, tq, lens, Hkv, P, topk, causal, torch.bfloat16, kdt)
    sel, sc = _run(si)
    _check(si, sel, sc, _oracle_scores(si), topk, True)


@pytest.mark.parametrize("tq, lens", [([5, 90], [900, 3000]), ([2, 1], [4000, 700])])  # tiled, split
def test_select_without_forced_local_and_fp16(tq, lens):
    si = W.make_selection(320, tq, lens, 2, 64, 6, True, torch.float16, torch.float16)
    sel, sc = _run(si, force_local=False)
    _check(si, sel, sc, _oracle_scores(si), 6, False)


def test_select_feeds_the_attention_pass():
    # the selection's output is a valid `selected` for the pass: the pass over
    # it matches the attention oracle on the same selection
    import block_sparse_attention_selection_amd as msa
    import oracle

    dev = torch.device("cuda:0")
    si = W.make_selection(330, [4, 60], [1000, 2500], 2, 64, 6, True, torch.bfloat16, torch.bfloat16,
                          poison=False)
    sel, _ = _run(si)
    rng = np.random.default_rng(5)
    G = 4
    q = torch.from_numpy(rng.standard_normal((si.Tq, 2 * G, 128)).astype(np.float32)).to(torch.bfloat16)
    v = si.k_idx.flip(-1).contiguous()  # any cache of the same layout serves as V
    args = (q.to(dev), si.k_idx.to(dev), v.to(dev), torch.from_numpy(sel).to(dev),
            torch.from_numpy(si.block_tables).to(dev))
    out, lse = msa.kvouter_attention(*args, cu_seqlens_q=torch.from_numpy(si.cu_seqlens_q).to(dev),
                                     used_kv_lens=torch.from_numpy(si.used_kv_lens).to(dev),
                                     page_size=si.page_size, causal=True, return_lse=True)
    o_ref, l_ref = oracle.attention(q, si.k_idx, v, torch.from_numpy(sel), torch.from_numpy(si.block_tables),
                                    torch.from_numpy(si.cu_seqlens_q), torch.from_numpy(si.used_kv_lens), True)
    o = out.float().cpu().numpy()
    assert np.all(np.abs(o - o_ref) <= 1e-2 + 1e-2 * np.abs(o_ref))
    assert np.all(np.abs(lse.cpu().numpy() - l_ref) <= 1e-3)


@pytest.mark.parametrize("name", ["select_decode", "select_prefill"])
def test_select_full_size_sampled(name):
    # the benchmark's inputs and launch; the oracle scores a sample of rows
    si = W.SELECT_MAKERS[name]()
    sel, sc = _run(si)
    rng = np.random.default_rng(7)
    tokens = np.unique(rng.choice(si.Tq, size=min(si.Tq, 6), replace=False))
    seq, _ = R._positions(si.cu_seqlens_q, si.used_kv_lens, si.Tq, si.causal)
    ref = np.full(sc.shape, -np.inf)
    for t in tokens:  # one sequence at a time, de-paging only its pages
        s = int(seq[t])
        n = -(-int(si.used_kv_lens[s]) // si.page_size)
        pages = torch.from_numpy(si.block_tables[s, :n].astype(np.int64))
        sub_k = odecode(si.k_idx[pages])
        sub_bt = np.arange(n, dtype=np.int32)[None, :]
        a = int(si.cu_seqlens_q[s])
        sub_q = odecode(si.q_idx[a:int(si.cu_seqlens_q[s + 1])])
        r = R.block_scores(sub_q, sub_k, sub_bt, [0, sub_q.shape[0]], [si.used_kv_lens[s]], si.page_size,
                           si.causal, nb_cap=sc.shape[2], tokens=[int(t) - a])
        ref[t] = r[int(t) - a]
    _check(si, sel, sc, ref, si.topk, True, tokens=tokens)
    # every row, sampled or not: the list is the top-k of the kernel's own scores
    want = R.select_topk(sc, si.topk, si.cu_seqlens_q, si.used_kv_lens, si.causal, True)
    assert np.array_equal(sel, want)
