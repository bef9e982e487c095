"""GPU parity of the paged K/V store (msa_store_kv) against oracle/store_ref.

Bit-exact: every byte of both caches, written slots and untouched ones.
The fp8 cast is exercised on every bf16 and every fp16 value.
"""
import numpy as np
import pytest
import torch

from oracle import store_ref as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_selection_amd as msa

    msa.load()
    yield


def _run(k_new, v_new, loc, cache_dtype, NP, P, fill):
    import block_sparse_attention_selection_amd as msa

    dev = torch.device("cuda:0")
    N, Hkv, _ = k_new.shape
    shape = (NP, Hkv, P, 128)
    if cache_dtype == torch.float8_e4m3fn:
        kc = torch.full(shape, fill, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
        vc = torch.full(shape, fill, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
    else:
        kc = torch.full(shape, fill, dtype=cache_dtype, device=dev)
        vc = torch.full(shape, fill, dtype=cache_dtype, device=dev)
    msa.store_kv(k_new.to(dev), v_new.to(dev), loc.to(dev), kc, vc, page_size=P)
    torch.cuda.synchronize()
    return kc.cpu(), vc.cpu()


def _expect(k_new, v_new, loc, cache_dtype, NP, P, fill):
    N, Hkv, _ = k_new.shape
    shape = (NP, Hkv, P, 128)
    if cache_dtype == torch.float8_e4m3fn:
        kc, vc = np.full(shape, fill, np.uint8), np.full(shape, fill, np.uint8)
    else:
        kc, vc = np.full(shape, float(fill)), np.full(shape, float(fill))
    S.store_kv(k_new.float().numpy(), v_new.float().numpy(), loc.numpy(), kc, vc, P)
    return kc, vc


def _bits(t):
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.float().numpy()


@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float16])
def test_fp8_store_every_16_bit_value(in_dtype):
    # 256 tokens x 2 KV heads x 128 dims hold each 16-bit code once (K) and in
    # another order (V); half of the 512 slots are written
    rng = np.random.default_rng(5)
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    k_new = codes[torch.from_numpy(rng.permutation(65536))].view(in_dtype).reshape(256, 2, 128).contiguous()
    v_new = codes[torch.from_numpy(rng.permutation(65536))].view(in_dtype).reshape(256, 2, 128).contiguous()
    NP, P = 8, 64
    loc = torch.from_numpy(rng.permutation(NP * P)[:256].astype(np.int64))
    kc, vc = _run(k_new, v_new, loc, torch.float8_e4m3fn, NP, P, 0x33)
    ek, ev = _expect(k_new, v_new, loc, torch.float8_e4m3fn, NP, P, 0x33)
    for got, want, name in ((_bits(kc), ek, "k"), (_bits(vc), ev, "v")):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name}: {bad.shape[0]} bytes differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("P", [64, 128])
@pytest.mark.parametrize("cache", ["same", "fp8"])
def test_store_slots_skips_and_layout(P, cache):
    rng = np.random.default_rng(17 + P)
    N, Hkv, NP = 300, 4, 7
    in_dtype = torch.bfloat16
    k_new = torch.from_numpy(rng.standard_normal((N, Hkv, 128)).astype(np.float32) * 40).to(in_dtype)
    v_new = torch.from_numpy(rng.standard_normal((N, Hkv, 128)).astype(np.float32) * 40).to(in_dtype)
    loc = rng.permutation(NP * P)[:N].astype(np.int64)
    loc[::17] = -1                    # skipped
    loc[5::23] = NP * P + 11          # beyond the caches: skipped
    loc = torch.from_numpy(loc)
    cdt = torch.float8_e4m3fn if cache == "fp8" else in_dtype
    fill = 0x44 if cache == "fp8" else 3.0
    kc, vc = _run(k_new, v_new, loc, cdt, NP, P, fill)
    ek, ev = _expect(k_new, v_new, loc, cdt, NP, P, fill)
    assert np.array_equal(_bits(kc), ek) and np.array_equal(_bits(vc), ev)


def test_store_then_attention_reads_the_stored_tokens():
    # a sequence whose cache is written by the store and read by the pass:
    # the result equals the pass over a cache written on the host
    import block_sparse_attention_selection_amd as msa

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(23)
    Hq, Hkv, P, L = 16, 2, 64, 320
    NP = 6
    k_rows = torch.from_numpy(rng.standard_normal((L, Hkv, 128)).astype(np.float32)).to(torch.bfloat16)
    v_rows = torch.from_numpy(rng.standard_normal((L, Hkv, 128)).astype(np.float32)).to(torch.bfloat16)
    pages = rng.permutation(NP)[:5].astype(np.int32)
    loc = torch.from_numpy((pages[np.arange(L) // P].astype(np.int64) * P + np.arange(L) % P))
    kc = torch.zeros((NP, Hkv, P, 128), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
    vc = torch.zeros_like(kc)
    msa.store_kv(k_rows.to(dev), v_rows.to(dev), loc.to(dev), kc, vc, page_size=P)
    kh = torch.zeros((NP, Hkv, P, 128), dtype=torch.float32)
    vh = torch.zeros_like(kh)
    for j in range(L):
        pg, off = int(pages[j // P]), j % P
        kh[pg, :, off] = k_rows[j].float().clamp(-448, 448)
        vh[pg, :, off] = v_rows[j].float().clamp(-448, 448)
    kh8 = kh.to(torch.float8_e4m3fn).to(dev)
    vh8 = vh.to(torch.float8_e4m3fn).to(dev)
    assert torch.equal(kc.view(torch.uint8), kh8.view(torch.uint8))
    q = torch.from_numpy(rng.standard_normal((3, Hq, 128)).astype(np.float32)).to(torch.bfloat16).to(dev)
    sel = torch.from_numpy(np.tile(np.array([2, 0, 1], dtype=np.int32), (3, Hkv, 1))).to(dev)
    bt = torch.from_numpy(pages[None, :]).to(dev)
    cu = torch.tensor([0, 3], dtype=torch.int64, device=dev)
    used = torch.tensor([L], dtype=torch.int32, device=dev)
    o1, l1 = msa.kvouter_attention(q, kc, vc, sel, bt, cu_seqlens_q=cu, used_kv_lens=used, page_size=P,
                                   causal=True, return_lse=True)
    o2, l2 = msa.kvouter_attention(q, kh8, vh8, sel, bt, cu_seqlens_q=cu, used_kv_lens=used, page_size=P,
                                   causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_store_keys_only_into_an_index_cache():
    # no V: only the K rows are written (the sparse index K cache), same bytes
    # as the oracle's K cache
    import block_sparse_attention_selection_amd as msa

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(31)
    N, Hkv, NP, P = 200, 2, 6, 64
    k_new = torch.from_numpy(rng.standard_normal((N, Hkv, 128)).astype(np.float32) * 30).to(torch.bfloat16)
    loc = torch.from_numpy(rng.permutation(NP * P)[:N].astype(np.int64))
    kc = torch.full((NP, Hkv, P, 128), 0x21, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
    msa.store_kv(k_new.to(dev), None, loc.to(dev), kc, None, page_size=P)
    torch.cuda.synchronize()
    ek = np.full((NP, Hkv, P, 128), 0x21, np.uint8)
    ev = np.full((NP, Hkv, P, 128), 0x21, np.uint8)
    S.store_kv(k_new.float().numpy(), k_new.float().numpy(), loc.numpy(), ek, ev, P)
    assert np.array_equal(kc.view(torch.uint8).cpu().numpy(), ek)
