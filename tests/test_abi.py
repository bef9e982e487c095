"""The C-ABI library loads, exports what its header declares, and rejects
bad descriptors on the host before touching any device memory (CPU only).

Descriptor data pointers here are fake aligned addresses: every case must be
refused by host validation, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_selection_amd as msa
from block_sparse_attention_selection_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa_kvouter.h")
FAKE = 1 << 20  # aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(msa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["msa_kvouter_attention", "msa_build_index", "msa_widen_fp8", "msa_validate_inputs",
              "msa_last_error", "msa_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(msa.lib_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_string():
    assert "gfx950" in msa.version()


def desc(shape, dtype, data=FAKE):
    d = _lib.MsaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    for i, n in enumerate(shape):
        d.shape[i] = n
    return d


def good(Tq=4, Hq=16, Hkv=2, NP=8, P=64, K=4, B=2, MP=4):
    return dict(
        q=desc([Tq, Hq, 128], msa.MSA_BF16),
        k=desc([NP, Hkv, P, 128], msa.MSA_BF16),
        v=desc([NP, Hkv, P, 128], msa.MSA_BF16),
        sel=desc([Tq, Hkv, K], msa.MSA_INT32),
        bt=desc([B, MP], msa.MSA_INT32),
        cu=desc([B + 1], msa.MSA_INT64),
        used=desc([B], msa.MSA_INT32),
        out=desc([Tq, Hq, 128], msa.MSA_BF16),
        lse=desc([Hq, Tq], msa.MSA_FP32),
        P=P,
        causal=1,
    )


def call(a):
    lib = msa.load()
    r = lambda x: ctypes.byref(x) if x is not None else None
    rc = lib.msa_kvouter_attention(r(a["q"]), r(a["k"]), r(a["v"]), r(a["sel"]), r(a["bt"]), r(a["cu"]),
                                   r(a["used"]), a["P"], a["causal"], r(a["out"]), r(a["lse"]), None)
    return rc, lib.msa_last_error().decode()


INV, UNS = -1, -2
BAD = [
    ("q rank", lambda a: a.update(q=desc([4, 16], msa.MSA_BF16)), INV),
    ("fp8 q", lambda a: a.update(q=desc([4, 16, 128], msa.MSA_FP8_E4M3FN)), UNS),
    ("fp32 q", lambda a: a.update(q=desc([4, 16, 128], msa.MSA_FP32)), INV),
    ("head dim 64", lambda a: a.update(q=desc([4, 16, 64], msa.MSA_BF16)), UNS),
    ("page size 32", lambda a: a.update(P=32, k=desc([8, 2, 32, 128], msa.MSA_BF16),
                                        v=desc([8, 2, 32, 128], msa.MSA_BF16)), UNS),
    ("page dim mismatch", lambda a: a.update(P=128), INV),
    ("kv dtype fp16 vs bf16 q", lambda a: a.update(k=desc([8, 2, 64, 128], msa.MSA_FP16),
                                                   v=desc([8, 2, 64, 128], msa.MSA_FP16)), UNS),
    ("v dtype differs", lambda a: a.update(v=desc([8, 2, 64, 128], msa.MSA_FP8_E4M3FN)), INV),
    ("v shape differs", lambda a: a.update(v=desc([9, 2, 64, 128], msa.MSA_BF16)), INV),
    ("Hq % Hkv", lambda a: a.update(k=desc([8, 3, 64, 128], msa.MSA_BF16), v=desc([8, 3, 64, 128], msa.MSA_BF16),
                                    sel=desc([4, 3, 4], msa.MSA_INT32)), INV),
    ("selected dtype", lambda a: a.update(sel=desc([4, 2, 4], msa.MSA_INT64)), INV),
    ("selected shape", lambda a: a.update(sel=desc([5, 2, 4], msa.MSA_INT32)), INV),
    ("topk 65", lambda a: a.update(sel=desc([4, 2, 65], msa.MSA_INT32)), UNS),
    ("cu dtype", lambda a: a.update(cu=desc([3], msa.MSA_INT32)), INV),
    ("cu length", lambda a: a.update(cu=desc([4], msa.MSA_INT64)), INV),
    ("used length", lambda a: a.update(used=desc([3], msa.MSA_INT32)), INV),
    ("out dtype", lambda a: a.update(out=desc([4, 16, 128], msa.MSA_FP16)), INV),
    ("out shape", lambda a: a.update(out=desc([4, 8, 128], msa.MSA_BF16)), INV),
    ("lse shape", lambda a: a.update(lse=desc([4, 16], msa.MSA_FP32)), INV),
    ("lse dtype", lambda a: a.update(lse=desc([16, 4], msa.MSA_BF16)), INV),
    ("null q data", lambda a: a.update(q=desc([4, 16, 128], msa.MSA_BF16, data=0)), INV),
    ("misaligned k", lambda a: a.update(k=desc([8, 2, 64, 128], msa.MSA_BF16, data=FAKE + 8)), INV),
    ("causal 2", lambda a: a.update(causal=2), INV),
    ("null q descriptor", lambda a: a.update(q=None), INV),
    ("null out descriptor", lambda a: a.update(out=None), INV),
]


@pytest.mark.parametrize("name,mutate,code", BAD, ids=[b[0] for b in BAD])
def test_invalid_descriptors_are_refused_on_the_host(name, mutate, code):
    a = good()
    mutate(a)
    rc, msg = call(a)
    assert rc == code, (rc, msg)
    assert msg


# ---------------------------------------------------------------------------
# msa_kvouter_attention_mxfp4: host refusals
# ---------------------------------------------------------------------------
def good_fp4(Tq=2, Hq=16, Hkv=2, NP=8, P=64, K=4, B=2, MP=4):
    a = good(Tq=Tq, Hq=Hq, Hkv=Hkv, NP=NP, P=P, K=K, B=B, MP=MP)
    del a["k"], a["v"]
    a.update(kc=desc([NP, Hkv, P, 64], msa.MSA_UINT8), ks=desc([NP, Hkv, P, 4], msa.MSA_UINT8),
             vc=desc([NP, Hkv, P, 64], msa.MSA_UINT8), vs=desc([NP, Hkv, P, 4], msa.MSA_UINT8))
    return a


def call_fp4(a):
    lib = msa.load()
    r = lambda x: ctypes.byref(x) if x is not None else None
    rc = lib.msa_kvouter_attention_mxfp4(r(a["q"]), r(a["kc"]), r(a["ks"]), r(a["vc"]), r(a["vs"]), r(a["sel"]),
                                         r(a["bt"]), r(a["cu"]), r(a["used"]), a["P"], a["causal"], r(a["out"]),
                                         r(a["lse"]), None)
    return rc, lib.msa_last_error().decode()


BAD_FP4 = [
    ("codes dtype", lambda a: a.update(kc=desc([8, 2, 64, 64], msa.MSA_FP8_E4M3FN)), INV),
    ("codes row bytes", lambda a: a.update(kc=desc([8, 2, 64, 32], msa.MSA_UINT8),
                                           vc=desc([8, 2, 64, 32], msa.MSA_UINT8)), UNS),
    ("v codes shape", lambda a: a.update(vc=desc([9, 2, 64, 64], msa.MSA_UINT8)), INV),
    ("scales per row", lambda a: a.update(ks=desc([8, 2, 64, 8], msa.MSA_UINT8)), INV),
    ("scales pages", lambda a: a.update(vs=desc([7, 2, 64, 4], msa.MSA_UINT8)), INV),
    ("misaligned codes", lambda a: a.update(kc=desc([8, 2, 64, 64], msa.MSA_UINT8, data=FAKE + 8)), INV),
    ("misaligned scales", lambda a: a.update(ks=desc([8, 2, 64, 4], msa.MSA_UINT8, data=FAKE + 4)), INV),
    ("fp16 q", lambda a: a.update(q=desc([2, 16, 128], msa.MSA_FP16), out=desc([2, 16, 128], msa.MSA_FP16)), UNS),
    ("page size 32", lambda a: a.update(P=32), UNS),
    ("selected shape", lambda a: a.update(sel=desc([2, 3, 4], msa.MSA_INT32)), INV),
    ("null scales", lambda a: a.update(vs=None), INV),
    ("null out", lambda a: a.update(out=None), INV),
]


@pytest.mark.parametrize("name,mutate,code", BAD_FP4, ids=[b[0] for b in BAD_FP4])
def test_mxfp4_descriptors_are_refused_on_the_host(name, mutate, code):
    a = good_fp4()
    mutate(a)
    rc, msg = call_fp4(a)
    assert rc == code, (rc, msg)
    assert msg


def test_mxfp4_empty_batch_enqueues_nothing():
    rc, msg = call_fp4(good_fp4(Tq=0, B=0))
    assert rc == 0, msg


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_mxfp4_no_device_is_an_error_not_a_crash():
    rc, msg = call_fp4(good_fp4())
    assert rc == -4 and msg


def test_empty_batch_enqueues_nothing():
    a = good(Tq=0)
    rc, msg = call(a)
    assert rc == 0, msg


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_no_device_is_an_error_not_a_crash():
    rc, msg = call(good())
    assert rc == -4 and msg


def test_widen_argument_checks():
    lib = msa.load()
    assert lib.msa_widen_fp8(None, 16, msa.MSA_BF16, FAKE, None) == INV
    assert lib.msa_widen_fp8(FAKE, 15, msa.MSA_BF16, FAKE, None) == INV
    assert lib.msa_widen_fp8(FAKE, 16, msa.MSA_FP32, FAKE, None) == INV
    assert lib.msa_widen_fp8(FAKE + 4, 16, msa.MSA_BF16, FAKE, None) == INV


def test_build_index_argument_checks():
    lib = msa.load()
    o = _lib.MsaIndexOut(*([FAKE] * 10))
    sel = desc([4, 2, 4], msa.MSA_INT32)
    cu = desc([3], msa.MSA_INT64)
    used = desc([2], msa.MSA_INT32)
    r = ctypes.byref
    assert lib.msa_build_index(r(sel), r(cu), r(used), 15, 4, 0, 8, 8, 0, r(o), None) == INV   # Hq % Hkv
    assert lib.msa_build_index(r(sel), r(cu), r(used), 16, 4, 0, 129, 8, 0, r(o), None) == INV  # tile too big
    assert lib.msa_build_index(r(sel), r(cu), r(used), 16, 4, 0, 8, 0, 0, r(o), None) == INV    # unit 0
    assert lib.msa_build_index(r(sel), r(cu), r(used), 16, 0, 0, 8, 8, 0, r(o), None) == INV    # nb_max 0
    assert lib.msa_build_index(r(sel), r(cu), r(used), 16, 4, 0, 8, 8, 2, r(o), None) == INV    # flag
    assert lib.msa_build_index(r(sel), r(cu), r(used), 16, 4, 0, 8, 8, 0, None, None) == INV


def test_store_kv_argument_checks():
    lib = msa.load()
    r = ctypes.byref

    def args(N=8, Hkv=2, NP=4, P=64, in_dt=msa.MSA_BF16, cache_dt=msa.MSA_FP8_E4M3FN, nloc=None, vshape=None):
        k = desc([N, Hkv, 128], in_dt)
        v = desc(vshape or [N, Hkv, 128], in_dt)
        loc = desc([N if nloc is None else nloc], msa.MSA_INT64)
        kc = desc([NP, Hkv, P, 128], cache_dt)
        vc = desc([NP, Hkv, P, 128], cache_dt)
        return k, v, loc, kc, vc

    def call_store(a, P=64):
        k, v, loc, kc, vc = a
        return lib.msa_store_kv(r(k), r(v), r(loc), r(kc), r(vc), P, None)

    assert call_store(args(in_dt=msa.MSA_FP32)) == INV                          # input dtype
    assert call_store(args(cache_dt=msa.MSA_FP16)) == INV                       # bf16 into fp16 cache
    assert call_store(args(nloc=7)) == INV                                      # one slot per token
    assert call_store(args(vshape=[8, 2, 64])) != 0                             # K and V differ
    assert call_store(args(P=128)) == INV                                       # page dim != page_size
    assert call_store(args(), P=32) != 0                                        # unsupported page size
    k, v, loc, kc, vc = args()
    assert lib.msa_store_kv(None, r(v), r(loc), r(kc), r(vc), 64, None) == INV
    assert call_store(args(N=0)) == 0                                           # nothing to store
    assert lib.msa_store_kv(r(k), None, r(loc), r(kc), r(vc), 64, None) == INV   # V half given
    assert lib.msa_store_kv(r(k), None, r(loc), r(kc), None, 128, None) == INV   # K only: checks still run


def test_select_blocks_argument_checks():
    lib = msa.load()
    r = ctypes.byref

    def args(Tq=4, Hkv=2, NP=8, P=64, B=2, MP=4, topk=4, q_dt=msa.MSA_BF16, k_dt=msa.MSA_FP8_E4M3FN, sel=None,
             sc=None):
        return [desc([Tq, Hkv, 128], q_dt), desc([NP, Hkv, P, 128], k_dt), desc([B, MP], msa.MSA_INT32),
                desc([B + 1], msa.MSA_INT64), desc([B], msa.MSA_INT32), desc(sel or [Tq, Hkv, topk], msa.MSA_INT32),
                None if sc is None else desc(sc, msa.MSA_FP32)]

    def call_sel(a, P=64, causal=1, topk=4, force=1):
        q, k, bt, cu, used, sel, sc = a
        return lib.msa_select_blocks(r(q), r(k), r(bt), r(cu), r(used), P, causal, topk, force, r(sel),
                                     r(sc) if sc is not None else None, None)

    assert call_sel(args(q_dt=msa.MSA_FP8_E4M3FN)) == INV                  # fp8 index queries
    assert call_sel(args(k_dt=msa.MSA_FP16)) == INV                        # keys of another 16-bit type
    assert call_sel(args(), topk=0) == INV                                 # topk outside [1, 1024]
    assert call_sel(args(topk=5)) == INV                                   # selected width != topk
    assert call_sel(args(sc=[4, 2, 3])) == INV                             # scores: nb = 4*64/128 = 2
    assert call_sel(args(MP=4200)) == UNS                                  # beyond 2048 blocks
    assert call_sel(args(P=128)) == INV                                    # page dim != page_size
    assert call_sel(args(), causal=2) == INV
    assert call_sel(args(Tq=0)) == 0                                       # nothing to select
    assert call_sel(args(sc=[4, 2, 2]), P=32) == UNS                       # page size


# ---------------------------------------------------------------------------
# caller-owned workspace: the size query (shapes only) and host-side refusals
# ---------------------------------------------------------------------------
def ws_bytes(a, null_data=False):
    lib = msa.load()
    r = lambda x: ctypes.byref(x) if x is not None else None
    if null_data:
        for key in ("q", "k", "v", "sel", "bt", "cu", "used"):
            a[key].data = 0
    n = ctypes.c_size_t(123)
    rc = lib.msa_kvouter_workspace_bytes(r(a["q"]), r(a["k"]), r(a["v"]), r(a["sel"]), r(a["bt"]), r(a["cu"]),
                                         r(a["used"]), a["P"], a["causal"], ctypes.byref(n))
    return rc, int(n.value)


def _align(n):
    return (n + 255) // 256 * 256


def expected_ws(Tq, Hq, Hkv, K, B, MP, P):
    """The documented size: counters, then (non-decode calls) the bitmap, then
    the planning arrays and partials, each array 256-byte aligned."""
    G, nb = Hq // Hkv, -(-MP * P // 128)
    NR, W, ns, TG = nb * Hkv, -(-Tq // 32), Tq * Hkv * K, Tq * Hkv
    decode = Tq == B and G <= 64
    head = _align(256 + (0 if decode else NR * W * 4))
    sizes = [0 if decode else NR * W * 4] * 2 + [ns, TG * 4, TG * 4, ns * 4, TG * 4, NR * 4, (NR + 1) * 4,
                                                 (NR + 1) * 4, 0 if decode else ns * 4, 0 if decode else ns * 4]
    if not decode:
        T = min(128, max(1, 256 // G))
        items = ((Tq + T - 1) // T + B) * Hkv
        sizes += [8192, ns * 4, ns, ns * 16, 2 * items * 16, items * 4 * K * 16,
                  (ns * G + 31) // 32 * 32 * 128 * 2, ns * G * 4]
    off = 0
    for n in sizes:
        off = _align(off) + n
    return head + off + 256


@pytest.mark.parametrize("shape", [
    dict(Tq=64, Hq=64, Hkv=8, K=16, B=64, MP=512, P=64),    # decode: planning arrays only
    dict(Tq=4, Hq=16, Hkv=2, K=4, B=2, MP=4, P=64),         # small prefill-shaped batch
    dict(Tq=300, Hq=32, Hkv=1, K=32, B=3, MP=40, P=128),    # MQA prefill
    dict(Tq=64, Hq=64, Hkv=2, K=8, B=64, MP=16, P=64),      # decode with G = 32: front kernel only
    dict(Tq=64, Hq=128, Hkv=1, K=8, B=64, MP=16, P=64),     # decode with G = 128: the prefill path
])
def test_workspace_bytes_matches_the_documented_layout(shape):
    a = good(Tq=shape["Tq"], Hq=shape["Hq"], Hkv=shape["Hkv"], NP=16, P=shape["P"], K=shape["K"], B=shape["B"],
             MP=shape["MP"])
    rc, n = ws_bytes(a, null_data=True)   # shapes only: data pointers may be NULL
    assert rc == 0
    assert n == expected_ws(**shape)


def test_workspace_bytes_of_a_decode_batch_is_small_and_of_a_prefill_holds_every_partial():
    dec = ws_bytes(good(Tq=64, Hq=64, Hkv=8, K=16, B=64, MP=512, P=64))[1]
    assert dec < 100_000
    Tq, Hq, Hkv, K = 16384, 64, 8, 16
    pre = ws_bytes(good(Tq=Tq, Hq=Hq, Hkv=Hkv, K=K, B=1, MP=128, P=128))[1]
    assert pre >= Tq * Hkv * K * (Hq // Hkv) * (256 + 4)          # every slot's partial rows
    assert pre < 1.05 * Tq * Hkv * K * (Hq // Hkv) * (256 + 4) + 100e6


def test_workspace_bytes_refuses_what_the_call_refuses():
    a = good(Tq=0)
    assert ws_bytes(a) == (0, 0)
    a = good()
    a["q"] = desc([4, 16, 64], msa.MSA_BF16)
    assert ws_bytes(a)[0] == UNS
    lib = msa.load()
    b = good()
    r = ctypes.byref
    assert lib.msa_kvouter_workspace_bytes(r(b["q"]), r(b["k"]), r(b["v"]), r(b["sel"]), r(b["bt"]), r(b["cu"]),
                                           r(b["used"]), 64, 1, None) == INV


def call_ws(a, ws, nbytes):
    lib = msa.load()
    r = lambda x: ctypes.byref(x) if x is not None else None
    rc = lib.msa_kvouter_attention_ws(r(a["q"]), r(a["k"]), r(a["v"]), r(a["sel"]), r(a["bt"]), r(a["cu"]),
                                      r(a["used"]), a["P"], a["causal"], r(a["out"]), r(a["lse"]), ws, nbytes, None)
    return rc, lib.msa_last_error().decode()


@pytest.mark.parametrize("name,mutate,code", BAD, ids=[b[0] for b in BAD])
def test_ws_call_refuses_bad_descriptors_like_the_allocating_call(name, mutate, code):
    a = good()
    mutate(a)
    rc, msg = call_ws(a, FAKE, 1 << 30)
    assert rc == code, (rc, msg)


def test_ws_call_refuses_a_missing_or_misaligned_workspace():
    assert call_ws(good(), None, 1 << 20)[0] == INV
    rc, msg = call_ws(good(), FAKE + 64, 1 << 20)
    assert rc == INV and "aligned" in msg
    assert call_ws(good(Tq=0), None, 0)[0] == 0   # nothing to do, nothing needed
