"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test fixes the oracle against something it does not compute itself:
an independent conversion routine, dense attention from library primitives,
a closed form, an exact invariance, or a second implementation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_oracle(oracle, wl, k=None, v=None, sel=None, bt=None, pairs=None):
    if k is None:
        k, v = W.kv_pool(wl)
    return oracle.attention(wl.q, k, v, wl.selected if sel is None else sel,
                            wl.block_tables if bt is None else bt, wl.cu_seqlens_q,
                            wl.used_kv_lens, wl.causal, pairs=pairs)


def run_dense(wl, k, v):
    from oracle import dense

    return dense.attention(wl.q, k, v, torch.from_numpy(wl.block_tables),
                           torch.from_numpy(wl.cu_seqlens_q), torch.from_numpy(wl.used_kv_lens),
                           wl.causal)


# ---------------------------------------------------------------------------
# exact decoding of the stored formats, against torch's own conversions
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,nbits", [(torch.bfloat16, 16), (torch.float16, 16),
                                         (torch.float8_e4m3fn, 8)])
def test_decode_every_code(oracle_lib, dtype, nbits):
    if nbits == 16:
        codes = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16).view(dtype)
    else:
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dtype)
    got = oracle_lib.decode(codes)
    want = codes.double().numpy()
    assert np.array_equal(got, want, equal_nan=True)


def test_e4m3fn_known_values(oracle_lib):
    # format facts: max finite 448 (0x7E), NaN 0x7F, smallest subnormal 2^-9,
    # smallest normal 2^-6, one 0x38
    codes = torch.tensor([0x7E, 0x7F, 0x01, 0x08, 0x38, 0xFE, 0x80], dtype=torch.uint8)
    got = oracle_lib.decode(codes.view(torch.float8_e4m3fn))
    assert got[0] == 448.0 and math.isnan(got[1])
    assert got[2] == 2.0 ** -9 and got[3] == 2.0 ** -6 and got[4] == 1.0
    assert got[5] == -448.0 and got[6] == 0.0 and math.copysign(1, got[6]) < 0


# ---------------------------------------------------------------------------
# the README quick-start call: every block selected == dense attention
# ---------------------------------------------------------------------------
def test_quickstart_example_matches_dense(oracle_lib):
    with open(os.path.join(GOLDEN, "quickstart_example.json")) as f:
        ex = json.load(f)
    g = torch.Generator().manual_seed(20260714)
    q = torch.randn(ex["Tq"], ex["Hq"], 128, generator=g).to(torch.bfloat16)
    k = torch.randn(ex["num_pages"], ex["Hkv"], ex["page_size"], 128, generator=g).to(torch.bfloat16)
    v = torch.randn(k.shape, generator=g).to(torch.bfloat16)
    bt = torch.tensor(ex["block_tables"], dtype=torch.int32)
    sel = torch.tensor(ex["selected"], dtype=torch.int32)
    cu = torch.tensor(ex["cu_seqlens_q"], dtype=torch.int64)
    used = torch.tensor(ex["used_kv_lens"], dtype=torch.int32)
    out, lse = oracle_lib.attention(q, k, v, sel, bt, cu, used, causal=False)
    assert list(out.shape) == ex["expected_out_shape"]
    assert list(lse.shape) == ex["expected_lse_shape"]
    # dense attention written with library primitives over the 256 keys
    K = k[:, 0].reshape(256, 128).double().numpy()
    V = v[:, 0].reshape(256, 128).double().numpy()
    Q = q[0].double().numpy()
    S = (Q @ K.T) / math.sqrt(128)
    m = S.max(axis=1, keepdims=True)
    Wt = np.exp(S - m)
    ref = (Wt @ V) / Wt.sum(axis=1, keepdims=True)
    ref_lse = m[:, 0] + np.log(Wt.sum(axis=1))
    assert np.abs(out[0] - ref).max() < 1e-12
    assert np.abs(lse[:, 0] - ref_lse).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,P", [(8, 2, 64), (4, 4, 128), (16, 1, 64), (12, 3, 128)])
def test_all_blocks_equals_dense(oracle_lib, causal, Hq, Hkv, P):
    wl = W.make_custom(11 + Hq + P, [3, 1, 5, 0, 2], [300, 129, 640, 77, 2],
                       Hq, Hkv, P, topk=6, causal=causal, pick="all", poison=True)
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    ref, ref_lse = run_dense(wl, k, v)
    assert np.abs(out - ref).max() < 1e-12
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12


@pytest.mark.parametrize("kv_dtype,q_dtype", [(torch.float16, torch.float16),
                                              (torch.float8_e4m3fn, torch.bfloat16),
                                              (torch.float8_e4m3fn, torch.float16)])
def test_all_blocks_equals_dense_dtypes(oracle_lib, kv_dtype, q_dtype):
    wl = W.make_custom(5, [4, 2], [257, 384], 8, 2, 64, topk=4, causal=True, pick="all",
                       q_dtype=q_dtype, kv_dtype=kv_dtype)
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    ref, ref_lse = run_dense(wl, k, v)
    assert np.abs(out - ref).max() < 1e-12
    assert np.nanmax(np.abs(lse - ref_lse)) < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def _gather_rows(cache, bt_row, js, g):
    P = cache.shape[2]
    js = np.asarray(js)
    pages = torch.from_numpy(np.asarray(bt_row, dtype=np.int64)[js // P])
    return cache[pages, g, torch.from_numpy(js % P)].double().numpy()


def test_equal_keys_give_uniform_mean(oracle_lib):
    wl = W.make_custom(21, [2], [500], 4, 1, 64, topk=3, causal=False, pick="random")
    k, v = W.kv_pool(wl)
    k.view(torch.int16)[:] = torch.tensor(0x3F80, dtype=torch.int16)  # every key is 1.0
    out, lse = run_oracle(oracle_lib, wl, k, v)
    for t in range(2):
        js = sorted({j for b in wl.selected[t, 0] if 0 <= b < 4
                     for j in range(128 * b, min(128 * b + 128, 500))})
        Vj = _gather_rows(v, wl.block_tables[0], js, 0)
        for h in range(4):
            x = wl.q[t, h].double().sum().item() / math.sqrt(128)
            assert abs(lse[h, t] - (x + math.log(len(js)))) < 1e-12
            assert np.abs(out[t, h] - Vj.mean(axis=0)).max() < 1e-12


def test_equal_value_rows_give_that_row(oracle_lib):
    wl = W.make_custom(22, [3, 2], [200, 640], 8, 2, 128, topk=4, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    row = torch.randn(128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    v[:] = row
    out, lse = run_oracle(oracle_lib, wl, k, v)
    fin = np.isfinite(lse.T)
    assert np.abs(out[fin] - row.double().numpy()[None, :]).max() < 1e-12


def test_single_key_returns_its_value_row(oracle_lib):
    wl = W.make_custom(23, [1, 1], [1, 1], 4, 2, 64, topk=2, causal=True, pick="all")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    for s in range(2):
        for h in range(4):
            g = h // 2
            page = wl.block_tables[s, 0]
            krow = k[page, g, 0].double().numpy()
            vrow = v[page, g, 0].double().numpy()
            assert np.array_equal(out[s, h], vrow)
            x = float(wl.q[s, h].double().numpy() @ krow) / math.sqrt(128)
            assert abs(lse[h, s] - x) < 1e-12


def test_weights_sum_to_one_via_constant_values(oracle_lib):
    # with every V row equal to 1.0 the output is the sum of the weights
    wl = W.make_custom(24, [5, 3], [700, 300], 8, 4, 64, topk=5, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    v.view(torch.int16)[:] = torch.tensor(0x3F80, dtype=torch.int16)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    fin = np.isfinite(lse.T)
    assert np.abs(out[fin] - 1.0).max() < 1e-13


# ---------------------------------------------------------------------------
# exact invariances
# ---------------------------------------------------------------------------
def test_pick_order_is_irrelevant(oracle_lib):
    wl = W.make_custom(31, [4, 3], [900, 400], 8, 2, 64, topk=5, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    sel2 = wl.selected[:, :, ::-1].copy()
    out2, lse2 = run_oracle(oracle_lib, wl, k, v, sel=sel2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_pads_and_out_of_range_ids_are_ignored(oracle_lib):
    wl = W.make_custom(32, [4, 3], [900, 400], 8, 2, 64, topk=4, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    extra = np.array([-1, 99, -7, 8], dtype=np.int32)  # 8 >= ceil(900/128)
    sel2 = np.concatenate([wl.selected, np.broadcast_to(extra, wl.selected.shape[:2] + (4,))], axis=2)
    out2, lse2 = run_oracle(oracle_lib, wl, k, v, sel=sel2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_physical_page_permutation_is_irrelevant(oracle_lib):
    wl = W.make_custom(33, [3, 2], [700, 260], 8, 2, 64, topk=4, causal=False, pick="random")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    perm = np.random.default_rng(0).permutation(wl.num_pages)
    k2 = torch.empty_like(k)
    v2 = torch.empty_like(v)
    k2[torch.from_numpy(perm)] = k
    v2[torch.from_numpy(perm)] = v
    bt2 = np.where(wl.block_tables >= 0, perm[np.clip(wl.block_tables, 0, None)], -1).astype(np.int32)
    out2, lse2 = run_oracle(oracle_lib, wl, k2, v2, bt=bt2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_gqa_equals_mha_with_replicated_kv_heads(oracle_lib):
    wl = W.make_custom(34, [3, 2], [520, 300], 8, 2, 64, topk=3, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    G = 4
    kr = k.repeat_interleave(G, dim=1).contiguous()
    vr = v.repeat_interleave(G, dim=1).contiguous()
    selr = np.repeat(wl.selected, G, axis=1)
    out2, lse2 = oracle_lib.attention(wl.q, kr, vr, selr, wl.block_tables, wl.cu_seqlens_q,
                                      wl.used_kv_lens, True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_merging_disjoint_selections_by_lse(oracle_lib):
    wl = W.make_custom(35, [4, 2], [1000, 600], 8, 2, 128, topk=6, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    a = wl.selected.copy()
    b = wl.selected.copy()
    a[:, :, 3:] = -1
    b[:, :, :3] = -1
    oa, la = run_oracle(oracle_lib, wl, k, v, sel=a)
    ob, lb = run_oracle(oracle_lib, wl, k, v, sel=b)
    M = np.maximum(la, lb)
    M = np.where(np.isfinite(M), M, 0.0)
    wa, wb = np.exp(la - M), np.exp(lb - M)
    tot = wa + wb
    merged_lse = np.where(tot > 0, M + np.log(np.where(tot > 0, tot, 1)), -np.inf)
    merged = (wa.T[:, :, None] * oa + wb.T[:, :, None] * ob) / np.where(tot > 0, tot, 1).T[:, :, None]
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(merged_lse), fin)
    assert np.abs(merged_lse[fin] - lse[fin]).max() < 1e-12
    assert np.abs(merged - out).max() < 1e-12


# ---------------------------------------------------------------------------
# degenerate cases and reported violations
# ---------------------------------------------------------------------------
def test_rows_without_keys(oracle_lib):
    # causal with Tq_s > L: the first queries see no key at all
    wl = W.make_custom(41, [5], [3], 4, 1, 64, topk=2, causal=True, pick="all")
    wl.selected[:, :, 0] = 0  # block 0 for everybody; invisible for pos < 0
    wl.selected[:, :, 1] = -1
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    # pos = 3 - 5 + i  -> tokens 0, 1 see nothing
    assert np.all(out[:2] == 0) and np.all(np.isneginf(lse[:, :2]))
    assert np.all(np.isfinite(lse[:, 2:]))
    # a row whose picks are all pads
    sel = wl.selected.copy()
    sel[4] = -1
    out2, lse2 = run_oracle(oracle_lib, wl, k, v, sel=sel)
    assert np.all(out2[4] == 0) and np.all(np.isneginf(lse2[:, 4]))


def test_repeated_pick_is_reported(oracle_lib):
    wl = W.make_custom(42, [2], [400], 4, 1, 64, topk=3, causal=False, pick="random")
    k, v = W.kv_pool(wl)
    sel = wl.selected.copy()
    sel[0, 0, :] = [1, 1, 2]
    with pytest.raises(oracle_lib.OracleError):
        run_oracle(oracle_lib, wl, k, v, sel=sel)


def test_page_out_of_range_is_reported(oracle_lib):
    wl = W.make_custom(43, [2], [400], 4, 1, 64, topk=3, causal=False, pick="all")
    k, v = W.kv_pool(wl)
    bt = wl.block_tables.copy()
    bt[0, 1] = wl.num_pages + 5
    with pytest.raises(oracle_lib.OracleError):
        run_oracle(oracle_lib, wl, k, v, bt=bt)


def test_poison_outside_selection_never_read(oracle_lib):
    # poison is NaN; if any unselected page or stale row were read, NaN would appear
    wl = W.make_custom(44, [3, 2], [333, 700], 8, 2, 64, topk=3, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    assert torch.isnan(k.float()).any()
    out, lse = run_oracle(oracle_lib, wl, k, v)
    assert not np.isnan(out).any() and not np.isnan(lse).any()


# ---------------------------------------------------------------------------
# second, independent implementation
# ---------------------------------------------------------------------------
def test_literal_oracle_agrees_on_tiny(oracle_lib):
    from oracle import literal

    wl = W.make("tiny")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    out2, lse2 = literal.attention(wl.q, k, v, torch.from_numpy(wl.selected),
                                   torch.from_numpy(wl.block_tables), torch.from_numpy(wl.cu_seqlens_q),
                                   torch.from_numpy(wl.used_kv_lens), wl.causal)
    assert np.abs(out - out2).max() < 1e-12
    assert np.abs(lse - lse2).max() < 1e-12


def test_literal_oracle_agrees_causal_gqa(oracle_lib):
    from oracle import literal

    wl = W.make_custom(45, [2, 1, 3], [260, 130, 200], 4, 2, 64, topk=4, causal=True, pick="oob")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    out2, lse2 = literal.attention(wl.q, k, v, torch.from_numpy(wl.selected),
                                   torch.from_numpy(wl.block_tables), torch.from_numpy(wl.cu_seqlens_q),
                                   torch.from_numpy(wl.used_kv_lens), wl.causal)
    assert np.abs(out - out2).max() < 1e-12
    fin = np.isfinite(lse2)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse2[fin]).max() < 1e-12


def test_pairs_subset_matches_full(oracle_lib):
    wl = W.make_custom(46, [3, 4], [500, 900], 8, 2, 64, topk=3, causal=True, pick="random")
    k, v = W.kv_pool(wl)
    out, lse = run_oracle(oracle_lib, wl, k, v)
    pairs = [0 * 2 + 1, 5 * 2 + 0, 6 * 2 + 1]
    o2, l2 = run_oracle(oracle_lib, wl, k, v, pairs=pairs)
    for i, p in enumerate(pairs):
        t, g = divmod(p, 2)
        assert np.array_equal(o2[i], out[t, g * 4:(g + 1) * 4])
        assert np.array_equal(l2[i], lse[g * 4:(g + 1) * 4, t])


# ---------------------------------------------------------------------------
# the generators' fp8 values follow the stated cast rule
# ---------------------------------------------------------------------------
def test_fp8_values_follow_the_cast_rule():
    x = np.random.default_rng(0).standard_normal(4096).astype(np.float32) * 300
    got = W.to_dtype(x, torch.float8_e4m3fn)
    want = torch.from_numpy(x).float().clamp(-448, 448).to(torch.float8_e4m3fn)
    assert torch.equal(got.view(torch.uint8), want.view(torch.uint8))
    assert got.float().abs().max().item() <= 448.0
