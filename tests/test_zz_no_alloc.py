"""The no-allocation entry point, msa_kvouter_attention_noalloc (MI355X only).

Called through the C ABI, it must give bit for bit what
msa_kvouter_attention gives on the same inputs (the same kernels run; only
their scratch differs), on two calls in a row, the second with a smaller
input, since every call on a device shares the one scratch array and must
clear what it needs itself. Calls whose scratch need exceeds the array are
refused. Results are also checked against the fp64 oracle.
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


def _both(wl):
    import block_sparse_attention_selection_amd as msa

    d = device_inputs(wl)
    args = (d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"])
    kw = dict(cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"], page_size=wl.page_size,
              causal=wl.causal)
    ref = msa.kvouter_attention(*args, return_lse=True, **kw)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.Hq, wl.Tq), float("nan"), dtype=torch.float32, device="cuda")
    got = msa.kvouter_attention_noalloc(*args, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return ref, got


def _check(wl, ref, got):
    (o1, l1), (o2, l2) = ref, got
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    pairs = all_pairs(wl)
    ref_o, ref_l = oracle_pairs(wl, pairs)
    compare(wl, o2, l2, pairs, ref_o, ref_l)


# (a larger call, then a smaller one) on the paths the entry point serves:
# the classifier alone (decode), and classifier, index, units and tiles
PAIRS = {
    "decode": (dict(tq=[1] * 48, Hq=64, Hkv=8, P=64, K=16, pick="diag", seed=951),
               dict(tq=[1] * 7, Hq=64, Hkv=8, P=64, K=16, pick="diag", seed=952)),
    "prefill": (dict(tq=[64, 40, 3], Hq=16, Hkv=2, P=128, K=10, pick="diag", seed=953, shared=5),
                dict(tq=[20, 5], Hq=16, Hkv=2, P=128, K=10, pick="diag", seed=954, shared=5)),
    "prefill_fp8": (dict(tq=[50, 20], Hq=16, Hkv=2, P=64, K=8, pick="diag", seed=955, shared=4,
                         kvd=torch.float8_e4m3fn),
                    dict(tq=[9], Hq=16, Hkv=2, P=64, K=8, pick="diag", seed=956, shared=4,
                         kvd=torch.float8_e4m3fn)),
}


def _make(c):
    rng = np.random.default_rng(c["seed"])
    lens = [int(x) for x in rng.integers(max(c["tq"]) + 200, 4000, size=len(c["tq"]))]
    return W.make_custom(c["seed"], c["tq"], lens, c["Hq"], c["Hkv"], c["P"], topk=c["K"], causal=True,
                         pick=c["pick"], kv_dtype=c.get("kvd"), shared_chunk=16 if c.get("shared") else 0,
                         shared_picks=c.get("shared", 0))


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_equals_the_allocating_call_twice_in_a_row(name):
    big, small = (_make(c) for c in PAIRS[name])
    assert small.Tq < big.Tq
    for wl in (big, small):
        ref, got = _both(wl)
        _check(wl, ref, got)


def test_noalloc_refuses_calls_beyond_its_scratch():
    import block_sparse_attention_selection_amd as msa

    wl = W.make_custom(957, [300, 200], [3000, 2500], 32, 1, 128, topk=32, causal=True, pick="diag")
    d = device_inputs(wl)
    need = msa.workspace_bytes(d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"],
                               cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"],
                               page_size=wl.page_size, causal=wl.causal)
    assert need > 32 << 20
    out = torch.zeros_like(d["q"])
    with pytest.raises(msa.MsaError, match="scratch"):
        msa.kvouter_attention_noalloc(d["q"], d["k_cache"], d["v_cache"], d["selected"], d["block_tables"],
                                      cu_seqlens_q=d["cu_seqlens_q"], used_kv_lens=d["used_kv_lens"],
                                      page_size=wl.page_size, causal=wl.causal, out=out)
    assert torch.count_nonzero(out) == 0  # refused before anything was enqueued
