"""GPU parity: the HIP library against the fp64 oracle (MI355X only).

Tolerances: |dO| <= 1e-2 + 1e-2*|O_ref| per element, |dLSE| <= 1e-3, rows
without keys must give O = 0 and LSE = -inf on both sides. Index arrays are
compared bit for bit with the integer CPU reference. Unselected pages and
rows beyond each sequence's used length hold NaN poison throughout.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W

from _helpers import all_pairs, compare, device_inputs, oracle_pairs, product_tiles, run_gpu, stratified_pairs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_selection_amd as msa

    msa.load()
    yield


def _full(wl):
    out, lse = run_gpu(wl)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(wl, pairs)
    return compare(wl, out, lse, pairs, ref_o, ref_l)


# ---------------------------------------------------------------------------
# fp8 widening: every e4m3fn code against the oracle's exact decoding
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_widen_fp8_every_code(out_dtype):
    import block_sparse_attention_selection_amd as msa
    import oracle

    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(4)
    x = codes.view(torch.float8_e4m3fn).cuda()
    got = msa.widen_fp8(x, out_dtype).cpu().double().numpy()
    want = oracle.decode(codes.view(torch.float8_e4m3fn))
    finite = ~np.isnan(want)
    assert np.array_equal(got[finite], want[finite])
    assert np.isnan(got[~finite]).all()


# ---------------------------------------------------------------------------
# index builder: bit-exact against the CPU reference
# ---------------------------------------------------------------------------
def _index_case(wl, T, Tu, list_all=False):
    import block_sparse_attention_selection_amd as msa
    from oracle import index_ref

    nb_max = (wl.block_tables.shape[1] * wl.page_size + 127) // 128
    ref = index_ref.build(wl.selected, wl.cu_seqlens_q, wl.used_kv_lens, wl.causal, T, Tu, nb_max, wl.G,
                          list_all_tiles=list_all)
    got = msa.build_index(torch.from_numpy(wl.selected).cuda(), torch.from_numpy(wl.cu_seqlens_q).cuda(),
                          torch.from_numpy(wl.used_kv_lens).cuda(), Hq=wl.Hq, nb_max=nb_max,
                          causal=wl.causal, tile_tokens=T, unit_tokens=Tu, list_all_tiles=list_all)
    got = {k: v.cpu().numpy() for k, v in got.items()}
    Tq, Hkv, K = wl.selected.shape
    assert np.array_equal(got["slot_flag"], ref.slot_flag.reshape(-1))
    assert np.array_equal(got["tok_chain"], ref.tok_chain.reshape(-1))
    assert np.array_equal(got["tok_nres"], ref.tok_nres.reshape(-1))
    assert np.array_equal(got["row_off"], ref.row_off)
    assert np.array_equal(got["unit_off"], ref.unit_off)
    n = ref.ent.size
    assert got["counters"][0] == n
    assert np.array_equal(got["ent"][:n], ref.ent)
    assert np.array_equal(got["slot_pos"], ref.slot_pos.reshape(-1))
    assert got["counters"][2] == ref.unit_off[-1]
    cb = got["chain_blk"].reshape(Tq, Hkv, K)
    for (t0, g), ch in ref.chain_blk.items():
        assert list(cb[t0, g, :len(ch)]) == ch, (t0, g)
    nt = got["counters"][1]
    assert sorted(got["tile_items"][:nt].tolist()) == sorted(ref.tile_items)


@pytest.mark.parametrize("list_all", [False, True])
@pytest.mark.parametrize("T,Tu", [(0, 3), (1, 2), (2, 2), (3, 4), (16, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_index_builder_bitexact_custom(T, Tu, causal, list_all):
    wl = W.make_custom(300 + T, [3, 5, 1, 0, 40, 7], [300, 700, 129, 50, 5200, 900], 16, 2, 64, topk=6,
                       causal=causal, pick="oob", shared_chunk=8, shared_picks=3, pad_every=5)
    _index_case(wl, T, Tu, list_all)


@pytest.mark.parametrize("list_all", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_index_builder_bitexact_whole_words(causal, list_all):
    # 32-token tiles that start at multiples of 32 are the only writers of
    # their bitmap words (tokens 0-31, 32-63) and store them whole; the last
    # tile (tokens 64-68) owns its word because no token follows it; a
    # second batch whose first sequence ends at 30 tokens leaves every word
    # shared (set bit by bit)
    for seed, tq, lens in ((41, [32, 37], [3000, 6000]), (42, [30, 7, 33], [2000, 900, 4100])):
        wl = W.make_custom(seed, tq, lens, 16, 2, 64, topk=6, causal=causal, pick="random",
                           shared_chunk=8, shared_picks=3)
        _index_case(wl, 32, 16, list_all)


@pytest.mark.parametrize("name", ["tiny", "decode_gqa", "varlen_mqa"])
def test_index_builder_bitexact_named(name):
    wl = W.make(name)
    T = max(1, 128 // wl.G)
    _index_case(wl, T, T, list_all=name == "varlen_mqa")


@pytest.mark.parametrize("name", ["prefill_shared", "varlen_mqa", "dense_causal"])
def test_index_builder_bitexact_product_tiles(name):
    # the tile and window sizes the attention call itself uses (32-token
    # tiles and 128-token windows at G = 8; 8 and 32 at G = 32)
    wl = W.make(name)
    T, Tu = product_tiles(wl)
    _index_case(wl, T, min(Tu, 128), list_all=True)


# ---------------------------------------------------------------------------
# attention parity
# ---------------------------------------------------------------------------
def test_parity_tiny():
    _full(W.make("tiny"))


def test_parity_quickstart_shape():
    # the README quick-start call: 1 query, 16 heads, 4 pages of 64, both blocks
    wl = W.make_custom(7, [1], [256], 16, 1, 64, topk=2, causal=False, pick="all", extra_pages=0)
    _full(wl)


EDGE = [
    # (tq_per_seq, kv_lens, Hq, Hkv, P, topk, causal, pick, dtypes)
    ([1, 1, 1], [1, 129, 640], 8, 1, 64, 4, True, "random", None),            # L=1, partial blocks
    ([3, 0, 5, 2], [300, 77, 900, 2], 8, 2, 64, 4, True, "diag", None),          # empty sequence
    ([6], [3], 4, 1, 64, 2, True, "all", None),                                  # Tq_s > L: keyless rows
    ([4, 4], [1000, 257], 16, 1, 128, 5, False, "oob", None),                    # pads and out-of-range ids
    ([33, 17], [2000, 700], 32, 1, 128, 8, True, "diag", None),                  # MQA G=32
    ([20, 9], [1500, 600], 4, 4, 64, 6, True, "random", None),                   # MHA G=1
    ([40], [4000], 8, 2, 128, 8, True, "random", None),                          # shared chunks below
    ([5, 3], [700, 350], 8, 2, 64, 4, True, "random", (torch.float16, torch.float16)),
    ([5, 3], [700, 350], 8, 2, 64, 4, True, "random", (torch.bfloat16, torch.float8_e4m3fn)),
    ([5, 3], [700, 350], 8, 2, 128, 4, False, "random", (torch.float16, torch.float8_e4m3fn)),
    ([2, 1], [64, 190], 64, 8, 64, 3, True, "all", None),                        # G=8, small
    ([2, 0, 1], [900, 300, 700], 16, 2, 64, 4, True, "random", None),            # Tq == B, one 2-token seq
    ([3, 0, 0, 1], [1200, 64, 64, 500], 8, 1, 128, 6, False, "all", None),       # Tq == B, non-causal
    ([77, 30], [3000, 1100], 4, 2, 64, 7, True, "random", None),                 # G=2: partial rows cross blocks
    ([12, 3], [2000, 900], 64, 1, 128, 5, False, "random", None),                # G=64: 4-token tiles
    ([9, 5], [1500, 700], 128, 1, 64, 6, True, "random", None),                  # G=128: 2-token tiles, 1-token pieces
]


def _edge(case, tile_path=False):
    tq, lens, Hq, Hkv, P, K, causal, pick, dt = EDGE[case]
    if tile_path:  # one more sequence of 40 tokens makes the batch too long for per-token streaming
        tq, lens = list(tq) + [40], list(lens) + [296]
    qd, kvd = dt if dt else (torch.bfloat16, None)
    return W.make_custom(500 + case, tq, lens, Hq, Hkv, P, topk=K, causal=causal, pick=pick,
                         q_dtype=qd, kv_dtype=kvd, shared_chunk=16 if case == 6 else 0,
                         shared_picks=5 if case == 6 else 0, pad_every=7 if pick == "oob" else 0)


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_parity_edge_cases(case):
    _full(_edge(case))


# Small decode-shaped batches (Tq <= 4B, G <= 16) stream every token in the
# front kernel; these cases again with a longer batch, so that the unit and
# tile kernels see the same shapes.
@pytest.mark.parametrize("case", [i for i, e in enumerate(EDGE)
                                  if sum(e[0]) <= 4 * len(e[0]) and e[2] // e[3] <= 16 and sum(e[0]) != len(e[0])])
def test_parity_edge_cases_tile_path(case):
    wl = _edge(case, tile_path=True)
    assert wl.Tq > 4 * len(wl.used_kv_lens)
    _full(wl)


# Tiles of 128 tokens (G <= 2) with wide selections: a tile's tokens x
# top-k exceed the 4096 residual positions the tile kernel keeps in LDS, so
# its epilogue reads each row's residual counts and positions from global
# memory. Chains of shared picks plus per-token residual picks.
LONG_TILES = [
    # (tq_per_seq, kv_lens, Hq, Hkv, P, topk, kv dtype)
    ([160, 130], [7000, 6400], 4, 4, 128, 48, None),                 # G = 1, 128-token tiles
    ([140, 9], [9000, 3000], 4, 2, 64, 64, None),                    # G = 2, top-64
    ([150], [8200], 8, 4, 64, 40, torch.float8_e4m3fn),              # G = 2, fp8 cache
]


@pytest.mark.parametrize("case", range(len(LONG_TILES)))
def test_parity_long_tiles_merge_from_global(case):
    tq, lens, Hq, Hkv, P, K, kvd = LONG_TILES[case]
    wl = W.make_custom(540 + case, tq, lens, Hq, Hkv, P, topk=K, causal=True, pick="diag",
                       kv_dtype=kvd, shared_chunk=32, shared_picks=K // 2)
    T, _ = product_tiles(wl)
    assert T == 128 and min(T, max(tq)) * K > 4096
    _full(wl)


# Decode with more than 16 query heads per KV head (MQA): one token per
# sequence, 32 or 64 rows per token.
MQA_DECODE = [
    (32, None), (64, None), (32, torch.float8_e4m3fn), (64, torch.float8_e4m3fn),
    (48, None),   # 3 row sets of 16 in the front kernel, the fourth empty
    (128, None),  # beyond the front kernel's 64 rows: one-token tiles of the tile kernel
    (24, torch.float8_e4m3fn),
]


@pytest.mark.parametrize("case", range(len(MQA_DECODE)))
def test_parity_mqa_decode(case):
    Hq, kvd = MQA_DECODE[case]
    rng = np.random.default_rng(560 + case)
    lens = [int(x) for x in rng.integers(300, 5000, size=24)]
    wl = W.make_custom(560 + case, [1] * 24, lens, Hq, 1, 64, topk=8, causal=True, pick="diag", kv_dtype=kvd)
    _full(wl)


# Decode-shaped batches too large for one round of front workgroups
# (Tq <= 4B, G <= 16, Tq != B, Tq * Hkv > 2 * CUs): the front kernel lists
# tiles with residual slots, and the unit kernel derives the residual order
# from the bitmaps itself.
@pytest.mark.parametrize("kvd", [None, torch.float8_e4m3fn])
def test_parity_decode_shaped_batch_with_residuals(kvd):
    rng = np.random.default_rng(580)
    lens = [int(x) for x in rng.integers(2100, 4000, size=160)]
    wl = W.make_custom(581 if kvd is None else 582, [2] * 160, lens, 64, 8, 64, topk=16, causal=True,
                       pick="random", kv_dtype=kvd)
    assert wl.Tq <= 4 * wl.B and wl.Tq * wl.Hkv > 2 * 256
    _full(wl)


# Page ids outside [0, num_pages) are a precondition violation; the pass
# still treats such a page as holding no keys, on every path. With every
# page of a block outside the pool the result equals the oracle's with that
# block's picks removed.
PAGE_CASES = {
    "decode": dict(tq=[1] * 8, lens=[900, 2000, 700, 1500, 1300, 640, 2500, 1100], Hq=16, Hkv=2, P=128, K=6,
                   pick="random", shared=0),
    "decode_fp8": dict(tq=[1] * 8, lens=[900, 2000, 700, 1500, 1300, 640, 2500, 1100], Hq=16, Hkv=2, P=128, K=6,
                       pick="random", shared=0, kvd=torch.float8_e4m3fn),
    "tiles": dict(tq=[40, 30], lens=[3000, 2000], Hq=16, Hkv=2, P=128, K=8, pick="diag", shared=4),
    "tiles_fp8": dict(tq=[40, 30], lens=[3000, 2000], Hq=16, Hkv=2, P=128, K=8, pick="diag", shared=4,
                      kvd=torch.float8_e4m3fn),
    "tiles_page64": dict(tq=[40, 30], lens=[3000, 2000], Hq=16, Hkv=2, P=64, K=8, pick="diag", shared=4),
}


@pytest.mark.parametrize("name", list(PAGE_CASES))
def test_pages_outside_the_pool_hold_no_keys(name):
    import dataclasses

    c = PAGE_CASES[name]
    wl = W.make_custom(590 + list(PAGE_CASES).index(name), c["tq"], c["lens"], c["Hq"], c["Hkv"], c["P"],
                       topk=c["K"], causal=True, pick=c["pick"], kv_dtype=c.get("kvd"),
                       shared_chunk=16 if c["shared"] else 0, shared_picks=c["shared"])
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
        b = int(np.bincount(valid).argmax())       # the block most tokens of s picked
        for lp in range(b * ppb, min((b + 1) * ppb, bt.shape[1])):
            bt[s, lp] = wl.num_pages + 3 if s % 2 == 0 else -2
        sel_ref[cu[s]:cu[s + 1]][picks == b] = -1
    d = device_inputs(wl)
    d["block_tables"] = torch.from_numpy(bt).cuda()
    out, lse = run_gpu(wl, d)
    ref_wl = dataclasses.replace(wl, selected=sel_ref)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(ref_wl, pairs)
    compare(wl, out, lse, pairs, ref_o, ref_l)


def test_parity_shared_chunks_with_residuals():
    # tiles with long chains plus residual picks (the prefill pattern at small size)
    wl = W.make_custom(611, [64, 48], [4096, 3000], 16, 2, 128, topk=10, causal=True, pick="diag",
                       shared_chunk=16, shared_picks=6)
    _full(wl)


def test_parity_decode_gqa():
    _full(W.make("decode_gqa"))


def test_parity_decode_mqa_full():
    # every pair of the 256-sequence MQA decode batch (32 query heads per KV head)
    _full(W.make("decode_mqa"))


def test_parity_decode_fp8_full():
    # every (token, KV head) pair of the 256-sequence fp8 decode batch
    _full(W.make("decode_fp8"))


def test_parity_varlen_mqa_full():
    # every (token, KV head) pair of the varlen MQA prefill (fp16)
    wl = W.make("varlen_mqa")
    _full(wl)


def _stratified(name):
    wl = W.make(name)
    out, lse = run_gpu(wl)
    assert not torch.isnan(out.float()).any()
    pairs = stratified_pairs(wl)
    ref_o, ref_l = oracle_pairs(wl, pairs)
    compare(wl, out, lse, pairs, ref_o, ref_l)
    return pairs


def test_parity_prefill_shared_every_tile_and_window():
    # every tile item (3 tokens each, all KV heads) and every unit window
    pairs = _stratified("prefill_shared")
    assert pairs.size >= 3 * 512 * 8


def test_parity_dense_causal_every_tile():
    # every visible block selected: dense causal attention through the sparse path
    _stratified("dense_causal")


FULL = pytest.mark.skipif(not os.environ.get("MSA_PARITY_FULL"),
                          reason="every pair at full size takes minutes of oracle time; set MSA_PARITY_FULL=1")


@FULL
@pytest.mark.parametrize("name", ["prefill_shared", "dense_causal"])
def test_parity_full_size_every_pair(name):
    _full(W.make(name))


@pytest.mark.parametrize("causal", [True, False])
def test_parity_dense_small(causal):
    # all blocks selected at a size the oracle checks in full, several tiles
    # and a ragged last block
    wl = W.make_custom(620 + int(causal), [200, 77], [900, 77 if causal else 333], 16, 2, 64, topk=8,
                       causal=causal, pick="all")
    _full(wl)


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------
def test_deterministic_bits():
    wl = W.make_custom(701, [24, 8, 1], [3000, 900, 5000], 16, 2, 64, topk=8, causal=True,
                       pick="diag", shared_chunk=8, shared_picks=4)
    inputs = device_inputs(wl)
    o1, l1 = run_gpu(wl, inputs)
    o2, l2 = run_gpu(wl, inputs)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_and_prefill_calls_interleaved():
    # Batches with one query token per sequence skip the index, unit and tile
    # kernels; the front kernel then resets the counter set of the next call.
    # Calls of both kinds, back to back on one stream, must each match the
    # oracle, whatever kind of call ran before them.
    dec = [W.make_custom(720 + i, [1] * 6, [900, 3000, 129, 4000, 640, 2000], 16, 2, 64, topk=6,
                         causal=True, pick="random") for i in range(2)]
    pre = [W.make_custom(730 + i, [40, 17], [2000, 700], 16, 2, 64, topk=8, causal=True, pick="diag",
                         shared_chunk=16, shared_picks=4) for i in range(2)]
    import block_sparse_attention_selection_amd as msa

    inputs = {id(w): device_inputs(w) for w in dec + pre}
    order = [pre[0], dec[0], dec[1], pre[1], dec[0], pre[0], pre[1], dec[1]]
    results = []
    for wl in order:  # enqueued back to back, one synchronisation at the end
        d = inputs[id(wl)]
        results.append(msa.kvouter_attention(
            d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"],
            cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"],
            page_size=wl.page_size, causal=wl.causal, return_lse=True))
    torch.cuda.synchronize()
    for wl, (out, lse) in zip(order, results):
        pairs = all_pairs(wl)
        ref_o, ref_l = oracle_pairs(wl, pairs)
        compare(wl, out, lse, pairs, ref_o, ref_l)


def test_tq_zero_is_a_no_op():
    import block_sparse_attention_selection_amd as msa

    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    out = msa.kvouter_attention(q, k, k, torch.empty((0, 1, 4), dtype=torch.int32, device="cuda"),
                                torch.zeros((1, 2), dtype=torch.int32, device="cuda"),
                                cu_seqlens_q=torch.zeros(2, dtype=torch.int64, device="cuda"),
                                used_kv_lens=torch.zeros(1, dtype=torch.int32, device="cuda"),
                                page_size=64)
    assert out.shape == (0, 8, 128)


def test_validate_inputs_reports_violations():
    import block_sparse_attention_selection_amd as msa

    wl = W.make_custom(801, [3, 2], [500, 300], 8, 2, 64, topk=3, causal=True, pick="random")
    d = device_inputs(wl)
    kw = dict(cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"], page_size=64, causal=True)
    msa.validate_inputs(d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"], **kw)
    bad = d["selected"].clone()
    bad[0, 0, 1] = bad[0, 0, 0] = 0
    with pytest.raises(msa.MsaError, match="twice"):
        msa.validate_inputs(d["q"], d["k_cache"], d["v_cache"], bad, d["block_tables"], **kw)
    bt = d["block_tables"].clone()
    bt[0, 0] = wl.num_pages + 3
    sel = d["selected"].clone()
    sel[0, 0, :] = torch.tensor([0, -1, -1], dtype=torch.int32)
    with pytest.raises(msa.MsaError, match="block_tables"):
        msa.validate_inputs(d["q"], d["k_cache"], d["v_cache"], sel, bt, **kw)
