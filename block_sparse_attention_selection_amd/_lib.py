"""ctypes binding of libmsa_kvouter.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "lib", "libmsa_kvouter.so")

MSA_BF16, MSA_FP16, MSA_FP8_E4M3FN, MSA_FP32, MSA_INT32, MSA_INT64, MSA_UINT8 = range(7)
_DTYPES = {
    torch.bfloat16: MSA_BF16,
    torch.float16: MSA_FP16,
    torch.float8_e4m3fn: MSA_FP8_E4M3FN,
    torch.float32: MSA_FP32,
    torch.int32: MSA_INT32,
    torch.int64: MSA_INT64,
    torch.uint8: MSA_UINT8,
}
ERRORS = {
    -1: "invalid argument",
    -2: "unsupported",
    -3: "out of memory",
    -4: "HIP error",
    -5: "precondition violated",
}


class MsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class MsaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
    ]


class MsaIndexOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "slot_flag", "tok_chain", "tok_nres", "chain_blk", "row_off", "unit_off",
        "ent", "slot_pos", "tile_items", "counters")]


_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing; build it with "
                "`python -m block_sparse_attention_selection_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(_LIB_PATH)
        T = ctypes.POINTER(MsaTensor)
        i32, vp = ctypes.c_int32, ctypes.c_void_p
        lib.msa_kvouter_attention.restype = i32
        lib.msa_kvouter_attention.argtypes = [T, T, T, T, T, T, T, i32, i32, T, T, vp]
        lib.msa_kvouter_workspace_bytes.restype = i32
        lib.msa_kvouter_attention_mxfp4.restype = i32
        lib.msa_kvouter_attention_mxfp4.argtypes = [T, T, T, T, T, T, T, T, T, i32, i32, T, T, vp]
        lib.msa_kvouter_workspace_bytes.argtypes = [T, T, T, T, T, T, T, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
        lib.msa_kvouter_attention_noalloc.restype = i32
        lib.msa_kvouter_attention_noalloc.argtypes = [T, T, T, T, T, T, T, i32, i32, T, T, vp]
        lib.msa_kvouter_attention_ws.restype = i32
        lib.msa_kvouter_attention_ws.argtypes = [T, T, T, T, T, T, T, i32, i32, T, T, vp, ctypes.c_size_t, vp]
        lib.msa_build_index.restype = i32
        lib.msa_build_index.argtypes = [T, T, T, i32, i32, i32, i32, i32, i32, ctypes.POINTER(MsaIndexOut), vp]
        lib.msa_widen_fp8.restype = i32
        lib.msa_widen_fp8.argtypes = [vp, ctypes.c_int64, i32, vp, vp]
        lib.msa_store_kv.restype = i32
        lib.msa_store_kv.argtypes = [T, T, T, T, T, i32, vp]
        lib.msa_select_blocks.restype = i32
        lib.msa_select_blocks.argtypes = [T, T, T, T, T, i32, i32, i32, i32, T, T, vp]
        lib.msa_validate_inputs.restype = i32
        lib.msa_validate_inputs.argtypes = [T, T, T, T, T, T, T, i32, i32, vp]
        lib.msa_profile_enable.restype = i32
        lib.msa_profile_enable.argtypes = [ctypes.c_uint32]
        lib.msa_profile_collect.restype = i32
        lib.msa_profile_collect.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        lib.msa_set_workspace_limit.restype = i32
        lib.msa_set_workspace_limit.argtypes = [ctypes.c_size_t]
        lib.msa_last_error.restype = ctypes.c_char_p
        lib.msa_last_error.argtypes = []
        lib.msa_version.restype = ctypes.c_char_p
        lib.msa_version.argtypes = []
        _lib = lib
        return lib


def version() -> str:
    return load().msa_version().decode()


def _check(rc: int):
    if rc != 0:
        raise MsaError(rc, load().msa_last_error().decode())


def describe(t: torch.Tensor | None):
    """msa_tensor descriptor of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    d = MsaTensor()
    d.data = t.data_ptr() if t.numel() else 0
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i, n in enumerate(t.shape):
        d.shape[i] = n
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _device_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("kvouter_attention takes device (HIP) tensors only")


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def kvouter_attention(q, k_cache, v_cache, selected, block_tables, *, cu_seqlens_q, used_kv_lens,
                      page_size: int, causal: bool = False, return_lse: bool = False,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """Block-sparse attention forward; see include/msa_kvouter.h for the contract.

    Returns ``out`` ``[Tq, Hq, 128]`` (q's dtype), or ``(out, lse)`` with
    ``lse`` fp32 ``[Hq, Tq]`` when ``return_lse`` is set. With ``workspace``
    (a contiguous device tensor of at least :func:`workspace_bytes` bytes) the
    call uses it as scratch (msa_kvouter_attention_ws) and allocates nothing;
    otherwise the library's own per-device workspace is used.
    """
    lib = load()
    _device_check(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, out, lse, workspace)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    ds = [describe(x) for x in (q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens)]
    do, dl = describe(out), describe(lse if return_lse or lse is not None else None)
    with torch.cuda.device(q.device):
        if workspace is None:
            rc = lib.msa_kvouter_attention(*[_ref(d) for d in ds], int(page_size), int(bool(causal)),
                                           _ref(do), _ref(dl), _stream(q.device))
        else:
            if not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
            nbytes = workspace.numel() * workspace.element_size()
            rc = lib.msa_kvouter_attention_ws(*[_ref(d) for d in ds], int(page_size), int(bool(causal)),
                                              _ref(do), _ref(dl), workspace.data_ptr() if nbytes else None,
                                              nbytes, _stream(q.device))
    _check(rc)
    return (out, lse) if return_lse else out


def kvouter_attention_mxfp4(q, k_codes, k_scales, v_codes, v_scales, selected, block_tables, *, cu_seqlens_q,
                            used_kv_lens, page_size: int, causal: bool = False, return_lse: bool = False,
                            out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """msa_kvouter_attention_mxfp4: the pass over MXFP4 caches (uint8 codes
    ``[NP, Hkv, P, 64]`` and e8m0 scales ``[NP, Hkv, P, 4]``, for K and for
    V), decode-shaped batches of bf16 queries. Returns ``out`` or
    ``(out, lse)`` as :func:`kvouter_attention`."""
    lib = load()
    _device_check(q, k_codes, k_scales, v_codes, v_scales, selected, block_tables, cu_seqlens_q, used_kv_lens,
                  out, lse)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    ds = [describe(x) for x in (q, k_codes, k_scales, v_codes, v_scales, selected, block_tables, cu_seqlens_q,
                                used_kv_lens)]
    do, dl = describe(out), describe(lse if return_lse or lse is not None else None)
    with torch.cuda.device(q.device):
        rc = lib.msa_kvouter_attention_mxfp4(*[_ref(d) for d in ds], int(page_size), int(bool(causal)),
                                             _ref(do), _ref(dl), _stream(q.device))
    _check(rc)
    return (out, lse) if return_lse else out


def kvouter_attention_noalloc(q, k_cache, v_cache, selected, block_tables, *, cu_seqlens_q, used_kv_lens,
                              page_size: int, causal: bool = False, out: torch.Tensor, lse: torch.Tensor | None = None):
    """msa_kvouter_attention_noalloc: the pass with the library's fixed
    per-device scratch array; ``out`` (and ``lse`` when wanted) must be
    given, so nothing is allocated. Returns ``out`` or ``(out, lse)``."""
    lib = load()
    _device_check(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, out, lse)
    ds = [describe(x) for x in (q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens)]
    with torch.cuda.device(q.device):
        rc = lib.msa_kvouter_attention_noalloc(*[_ref(d) for d in ds], int(page_size), int(bool(causal)),
                                               _ref(describe(out)), _ref(describe(lse)), _stream(q.device))
    _check(rc)
    return out if lse is None else (out, lse)


def workspace_bytes(q, k_cache, v_cache, selected, block_tables, *, cu_seqlens_q, used_kv_lens,
                    page_size: int, causal: bool = False) -> int:
    """Bytes of the caller-owned workspace a call with these shapes needs
    (msa_kvouter_workspace_bytes). Reads shapes and dtypes only; the tensors
    may live on any device."""
    lib = load()
    ds = [describe(x) for x in (q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens)]
    n = ctypes.c_size_t()
    _check(lib.msa_kvouter_workspace_bytes(*[_ref(d) for d in ds], int(page_size), int(bool(causal)),
                                           ctypes.byref(n)))
    return int(n.value)


def store_kv(k_new, v_new, loc, k_cache, v_cache, *, page_size: int):
    """Store new tokens' K and V rows into the paged caches (in place); see
    include/msa_kvouter.h (msa_store_kv) for the contract. v_new and v_cache
    may both be None (K rows only, e.g. an index key cache)."""
    lib = load()
    _device_check(*[x for x in (k_new, v_new, loc, k_cache, v_cache) if x is not None])
    ds = [describe(x) for x in (k_new, v_new, loc, k_cache, v_cache)]
    with torch.cuda.device(k_new.device):
        rc = lib.msa_store_kv(*[_ref(d) for d in ds], int(page_size), _stream(k_new.device))
    _check(rc)
    return k_cache, v_cache


def select_blocks(q_idx, k_idx_cache, block_tables, *, cu_seqlens_q, used_kv_lens, page_size: int,
                  topk: int, causal: bool = False, force_local: bool = True, selected=None,
                  return_scores: bool = False, scores=None):
    """Top-k block selection from index queries and the paged index K cache.

    Returns ``selected [Tq, Hkv, topk]`` int32, or ``(selected, scores)`` with
    ``scores [Tq, Hkv, ceil(max_pages * page_size / 128)]`` fp32. The scoring
    rule and the order of the list are in include/msa_kvouter.h
    (msa_select_blocks)."""
    lib = load()
    _device_check(q_idx, k_idx_cache, block_tables, cu_seqlens_q, used_kv_lens)
    Tq, Hkv = q_idx.shape[0], q_idx.shape[1]
    if selected is None:
        selected = torch.empty((Tq, Hkv, int(topk)), dtype=torch.int32, device=q_idx.device)
    if return_scores and scores is None:
        nb = -(-block_tables.shape[1] * int(page_size) // 128)
        scores = torch.empty((Tq, Hkv, nb), dtype=torch.float32, device=q_idx.device)
    ds = [describe(x) for x in (q_idx, k_idx_cache, block_tables, cu_seqlens_q, used_kv_lens)]
    dsel, dsc = describe(selected), describe(scores)
    with torch.cuda.device(q_idx.device):
        rc = lib.msa_select_blocks(*[_ref(d) for d in ds], int(page_size), int(bool(causal)), int(topk),
                                   int(bool(force_local)), _ref(dsel), _ref(dsc), _stream(q_idx.device))
    _check(rc)
    return (selected, scores) if return_scores else selected


def validate_inputs(q, k_cache, v_cache, selected, block_tables, *, cu_seqlens_q, used_kv_lens,
                    page_size: int, causal: bool = False):
    """Synchronous check of the data-dependent preconditions; raises MsaError."""
    lib = load()
    _device_check(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens)
    ds = [describe(x) for x in (q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens)]
    with torch.cuda.device(q.device):
        rc = lib.msa_validate_inputs(*[_ref(d) for d in ds], int(page_size), int(bool(causal)),
                                     _stream(q.device))
    _check(rc)


def build_index(selected, cu_seqlens_q, used_kv_lens, *, Hq: int, nb_max: int, causal: bool,
                tile_tokens: int, unit_tokens: int, list_all_tiles: bool = False):
    """Run the index builder alone; returns its device arrays as a dict."""
    lib = load()
    _device_check(selected, cu_seqlens_q, used_kv_lens)
    Tq, Hkv, K = selected.shape
    dev = selected.device
    NR = nb_max * Hkv
    i32 = dict(dtype=torch.int32, device=dev)
    res = dict(
        slot_flag=torch.zeros(Tq * Hkv * K, dtype=torch.uint8, device=dev),
        tok_chain=torch.zeros(Tq * Hkv, **i32),
        tok_nres=torch.zeros(Tq * Hkv, **i32),
        chain_blk=torch.full((Tq * Hkv * K,), -1, **i32),
        row_off=torch.zeros(NR + 1, **i32),
        unit_off=torch.zeros(NR + 1, **i32),
        ent=torch.full((max(1, Tq * Hkv * K),), -1, **i32),
        slot_pos=torch.zeros(Tq * Hkv * K, **i32),
        tile_items=torch.full((max(1, Tq * Hkv),), -1, **i32),
        counters=torch.zeros(8, **i32),
    )
    o = MsaIndexOut(**{k: v.data_ptr() for k, v in res.items()})
    ds = [describe(x) for x in (selected, cu_seqlens_q, used_kv_lens)]
    with torch.cuda.device(dev):
        rc = lib.msa_build_index(*[_ref(d) for d in ds], int(Hq), int(nb_max), int(bool(causal)),
                                 int(tile_tokens), int(unit_tokens), int(bool(list_all_tiles)),
                                 ctypes.byref(o), _stream(dev))
    _check(rc)
    return res


def set_workspace_limit(nbytes: int):
    """Cap the library-owned workspace (0: no cap); msa_set_workspace_limit."""
    _check(load().msa_set_workspace_limit(int(nbytes)))


KERNELS = {"index": 0, "front": 1, "units": 2, "tiles": 3, "store": 4, "select": 5}


def profile_enable(kernels=()):
    """Record HIP events around launches of the named kernels (empty: off)."""
    mask = 0
    for k in kernels:
        mask |= 1 << KERNELS[k]
    _check(load().msa_profile_enable(mask))


def profile_collect(kernel: str):
    """(total ms, launches) of the recorded launches of one kernel."""
    tot = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load().msa_profile_collect(KERNELS[kernel], ctypes.byref(tot), ctypes.byref(n)))
    return tot.value, n.value


def widen_fp8(x: torch.Tensor, out_dtype=torch.bfloat16) -> torch.Tensor:
    """Widen e4m3fn values with the kernels' conversion (numel % 16 == 0)."""
    lib = load()
    _device_check(x)
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    with torch.cuda.device(x.device):
        rc = lib.msa_widen_fp8(x.data_ptr(), x.numel(), _DTYPES[out_dtype], out.data_ptr(), _stream(x.device))
    _check(rc)
    return out
