"""The caller-owned workspace entry point, msa_kvouter_attention_ws, on the
GPU (MI355X only).

The call must give bit for bit what msa_kvouter_attention gives (the same
kernels run; only where their scratch lives differs), whatever the
workspace held before, and it must be capturable into a HIP graph: every
replay, with eager work and synchronisations between replays, must equal an
eager call on the same inputs. Results are also checked against the fp64
oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W

from _helpers import all_pairs, compare, device_inputs, oracle_pairs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_selection_amd as msa

    msa.load()
    yield


def _cases():
    rng = np.random.default_rng(31)
    return {
        # one token per sequence: front kernel only, no counters or bitmap
        "decode": lambda: W.make_custom(901, [1] * 12, [int(x) for x in rng.integers(200, 4000, 12)], 64, 8, 64,
                                        topk=8, causal=True, pick="diag"),
        # chains, residual units and the tile kernel's merges
        "prefill": lambda: W.make_custom(902, [64, 40, 3], [4000, 2500, 700], 16, 2, 128, topk=10, causal=True,
                                         pick="diag", shared_chunk=16, shared_picks=5),
        # MQA decode (G = 32): not decode-shaped for the front kernel
        "mqa_decode": lambda: W.make_custom(903, [1] * 10, [int(x) for x in rng.integers(300, 3000, 10)], 32, 1,
                                            64, topk=6, causal=True, pick="diag"),
        "prefill_fp8": lambda: W.make_custom(904, [50, 20], [3000, 1500], 16, 2, 64, topk=8, causal=True,
                                             pick="diag", kv_dtype=torch.float8_e4m3fn, shared_chunk=16,
                                             shared_picks=4),
    }


def _call(wl, d, workspace=None, out=None, lse=None):
    import block_sparse_attention_selection_amd as msa

    return msa.kvouter_attention(d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"],
                                 cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"],
                                 page_size=wl.page_size, causal=wl.causal, return_lse=True, out=out, lse=lse,
                                 workspace=workspace)


def _ws_for(wl, d, fill=0xAB):
    import block_sparse_attention_selection_amd as msa

    n = msa.workspace_bytes(d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"],
                            cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"],
                            page_size=wl.page_size, causal=wl.causal)
    assert n > 0
    return torch.full((n,), fill, dtype=torch.uint8, device="cuda")  # stale contents must not matter


def _same(a, b):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("name", list(_cases()))
def test_ws_call_equals_the_allocating_call_and_the_oracle(name):
    wl = _cases()[name]()
    d = device_inputs(wl)
    ref = _call(wl, d)
    ws = _ws_for(wl, d)
    got = _call(wl, d, workspace=ws)
    torch.cuda.synchronize()
    _same(ref, got)
    got2 = _call(wl, d, workspace=ws)  # the same workspace again, now holding the last call's leftovers
    torch.cuda.synchronize()
    _same(ref, got2)
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(wl, pairs)
    compare(wl, got[0], got[1], pairs, ref_o, ref_l)


def test_ws_too_small_is_refused():
    import block_sparse_attention_selection_amd as msa

    wl = _cases()["prefill"]()
    d = device_inputs(wl)
    ws = _ws_for(wl, d)
    with pytest.raises(msa.MsaError, match="workspace"):
        _call(wl, d, workspace=ws[: ws.numel() - 256])


@pytest.mark.parametrize("name", ["decode", "prefill", "prefill_fp8"])
def test_ws_call_captured_in_a_graph_replays_like_eager_calls(name):
    wl = _cases()[name]()
    d = device_inputs(wl)
    ws = _ws_for(wl, d)
    out = torch.empty_like(d["q"])
    lse = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(wl, d, workspace=ws, out=out, lse=lse)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(wl, d, workspace=ws, out=out, lse=lse)
    q0 = d["q"].clone()
    for i in range(4):
        # new query values in the captured input buffer, some eager work, then a replay
        gen = torch.Generator(device="cuda").manual_seed(100 + i)
        d["q"].copy_((torch.randn(q0.shape, generator=gen, device="cuda") * (1 + i)).to(q0.dtype))
        junk = torch.randn((1 << 20,), device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = _call(wl, d)  # the library-owned workspace, eager
        torch.cuda.synchronize()
        _same(eager, (out, lse))
        assert torch.isfinite(junk)
    del g


def test_workspace_limit_forces_out_of_memory_and_is_lifted():
    # the failure path of the library-owned workspace, forced from the host:
    # a cap below what a prefill call needs makes it fail cleanly with
    # MSA_ERR_OUT_OF_MEMORY (nothing enqueued), a decode call under the cap
    # still runs, and lifting the cap restores the prefill call
    import block_sparse_attention_selection_amd as msa

    pre = _cases()["prefill"]()
    dec = _cases()["decode"]()
    dp, dd = device_inputs(pre), device_inputs(dec)
    ref = _call(pre, dp)
    torch.cuda.synchronize()
    msa.set_workspace_limit(1 << 20)
    try:
        out = torch.full_like(dp["q"], 7.0)
        with pytest.raises(msa.MsaError, match="limit") as ei:
            _call(pre, dp, out=out)
        assert ei.value.code == -3
        torch.cuda.synchronize()
        assert torch.all(out == 7.0)  # refused before anything was enqueued
        got_dec = _call(dec, dd)      # a decode call needs far less than 1 MiB
        torch.cuda.synchronize()
        pairs = all_pairs(dec)
        ref_o, ref_l = oracle_pairs(dec, pairs)
        compare(dec, got_dec[0], got_dec[1], pairs, ref_o, ref_l)
    finally:
        msa.set_workspace_limit(0)
    _same(ref, _call(pre, dp))
