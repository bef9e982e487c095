"""Pins of the integer CPU reference of the index builder and work split (CPU only).

The reference (oracle/index_ref.py) is vectorised numpy; here it is checked
against a literal dictionary-and-loop construction on small inputs and
against structural invariants on the named workloads.
"""
import numpy as np
import pytest

import workloads as W
from oracle import index_ref


def literal_plan(selected, cu, used, causal, T, Tu, nb_max, Hkv, K, G=1, list_all=False):
    """Dictionary-and-loop restatement of the rules in index_ref's docstring.

    Returns the slot flags, the chains, the residual rows, and per (t, g) the
    chain length of t's tile and the number of residual slots, and the set
    of listed tiles (t_leader * Hkv + g)."""
    Tq = selected.shape[0]
    owner = {}
    for s in range(len(used)):
        for t in range(int(cu[s]), int(cu[s + 1])):
            owner.setdefault(t, s)
    valid = {}
    for t in range(Tq):
        for g in range(Hkv):
            for k in range(K):
                ok = False
                if t in owner:
                    s = owner[t]
                    L = int(used[s])
                    b = int(selected[t, g, k])
                    pos = L - (int(cu[s + 1]) - int(cu[s])) + (t - int(cu[s]))
                    ok = 0 <= b < min((L + 127) // 128, nb_max) and (not causal or 128 * b <= pos)
                valid[(t, g, k)] = ok
    picks = {(t, g): {int(selected[t, g, k]) for k in range(K) if valid[(t, g, k)]}
             for t in range(Tq) for g in range(Hkv)}
    flag = {key: (2 if v else 0) for key, v in valid.items()}
    chains = {}
    if T > 0:
        for s in range(len(used)):
            for t0 in range(int(cu[s]), int(cu[s + 1]), T):
                toks = range(t0, min(t0 + T, int(cu[s + 1])))
                for g in range(Hkv):
                    ch = []
                    for k in range(K):
                        b = int(selected[t0, g, k])
                        if valid[(t0, g, k)] and b not in ch and all(b in picks[(t, g)] for t in toks):
                            ch.append(b)
                    chains[(t0, g)] = ch
                    for t in toks:
                        for k in range(K):
                            if valid[(t, g, k)] and int(selected[t, g, k]) in ch:
                                flag[(t, g, k)] = 1
    rows = {}
    for (t, g, k), f in sorted(flag.items(), key=lambda kv: (kv[0][0] * Hkv + kv[0][1]) * K + kv[0][2]):
        if f == 2:
            r = int(selected[t, g, k]) * Hkv + g
            rows.setdefault(r, []).append((t * Hkv + g) * K + k)
    nres = {(t, g): sum(1 for k in range(K) if flag[(t, g, k)] == 2) for t in range(Tq) for g in range(Hkv)}
    chain_len = {(t, g): 0 for t in range(Tq) for g in range(Hkv)}
    listed = set()
    step = T if T > 0 else 1  # without chains every token is a tile of its own
    for s in range(len(used)):
        for t0 in range(int(cu[s]), int(cu[s + 1]), step):
            toks = list(range(t0, min(t0 + step, int(cu[s + 1]))))
            for g in range(Hkv):
                n = len(chains.get((t0, g), [])) if T > 0 else 0
                for t in toks:
                    chain_len[(t, g)] = n
                if list_all or len(toks) * G > 16 or any(nres[(t, g)] > 0 for t in toks):
                    listed.add(t0 * Hkv + g)
    return flag, chains, rows, chain_len, nres, listed


def check_against_literal(wl, T, Tu, nb_max, list_all=False):
    Tq, Hkv, K = wl.selected.shape
    plan = index_ref.build(wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, T, Tu, nb_max, wl.G,
                           list_all_tiles=list_all)
    flag, chains, rows, chain_len, nres, listed = literal_plan(
        wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, T, Tu, nb_max, Hkv, K, wl.G, list_all)
    for (t, g), n in chain_len.items():
        assert plan.tok_chain[t, g] == n, (t, g)
    for (t, g), n in nres.items():
        assert plan.tok_nres[t, g] == n, (t, g)
    assert plan.tile_items == listed
    for (t, g, k), f in flag.items():
        assert plan.slot_flag[t, g, k] == f, (t, g, k)
    for key, ch in chains.items():
        assert plan.chain_blk[key] == ch
    NR = nb_max * Hkv
    for r in range(NR):
        lst = rows.get(r, [])
        a, b = plan.row_off[r], plan.row_off[r + 1]
        assert list(plan.ent[a:b]) == lst
        assert plan.unit_off[r + 1] - plan.unit_off[r] == (len(lst) + Tu - 1) // Tu
    for i, slot in enumerate(plan.ent):
        assert plan.slot_pos.reshape(-1)[slot] == i
    assert (plan.slot_pos.reshape(-1) >= 0).sum() == plan.ent.size


@pytest.mark.parametrize("list_all", [False, True])
@pytest.mark.parametrize("T", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_matches_literal_rules(T, causal, list_all):
    wl = W.make_custom(100 + T, [3, 5, 1, 0, 4], [300, 700, 129, 50, 520], 4, 2, 64, topk=4,
                       causal=causal, pick="random", shared_chunk=2, shared_picks=2)
    nb_max = (wl.block_tables.shape[1] * 64 + 127) // 128
    check_against_literal(wl, T, 3, nb_max, list_all)


def test_reference_matches_literal_tile_listing_by_rows():
    # tiles of 2 tokens x G = 8 rows are listed only when they hold a
    # residual slot; tiles of 3 tokens x 8 = 24 rows always
    for T in (2, 3):
        wl = W.make_custom(150 + T, [6, 4, 1], [900, 400, 300], 16, 2, 64, topk=3, causal=True, pick="diag",
                           shared_chunk=T, shared_picks=2)
        nb_max = (wl.block_tables.shape[1] * 64 + 127) // 128
        check_against_literal(wl, T, 2, nb_max)


def test_reference_matches_literal_with_pads_and_oob():
    wl = W.make_custom(200, [4, 2], [900, 260], 8, 2, 128, topk=5, causal=True, pick="oob",
                       pad_every=3)
    nb_max = (wl.block_tables.shape[1] * 128 + 127) // 128
    check_against_literal(wl, 2, 2, nb_max)


def test_reference_matches_literal_on_tiny():
    wl = W.make("tiny")
    check_against_literal(wl, 8, 8, 4)


@pytest.mark.parametrize("name", ["tiny", "decode_gqa"])
def test_invariants_on_named_workloads(name):
    wl = W.make(name)
    Tq, Hkv, K = wl.selected.shape
    nb_max = (wl.block_tables.shape[1] * wl.page_size + 127) // 128
    T = max(1, 128 // wl.G)
    plan = index_ref.build(wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, T, T, nb_max, wl.G)
    _, valid = index_ref.slot_validity(wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, nb_max)
    # every valid slot is covered or residual, nothing else
    assert np.array_equal(plan.slot_flag > 0, valid)
    assert np.all(np.diff(plan.row_off) >= 0)
    assert plan.row_off[-1] == (plan.slot_flag == 2).sum() == plan.ent.size
    # within each row entries ascend
    for r in range(len(plan.row_off) - 1):
        seg = plan.ent[plan.row_off[r]:plan.row_off[r + 1]]
        assert np.all(np.diff(seg) > 0)
    if name == "decode_gqa":
        # one token per sequence: every tile is a single token, all slots covered
        assert plan.ent.size == 0
        assert not plan.tile_items


@pytest.mark.slow
def test_invariants_prefill_shared():
    wl = W.make("prefill_shared")
    nb_max = 128
    plan = index_ref.build(wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, True, 16, 16, nb_max, 8)
    # chunks of 64 tokens share at least 12 picks once the diagonal is >= 11
    for (t0, g), ch in plan.chain_blk.items():
        d = t0 // 128
        if d >= 11:
            assert len(ch) >= 12
    assert plan.row_off[-1] == (plan.slot_flag == 2).sum()
