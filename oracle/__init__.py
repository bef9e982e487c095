"""Oracle for MiniMax-M3 block-sparse attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library under
``block_sparse_attention_selection_amd`` never imports, links or runs it, and
it shares no code with that library.

Contents
  * ``attention``      -- ctypes front end of the fp64 C oracle in
                          ``msa_oracle.c`` (the plain definition of the pass;
                          fw-ai/minimax-kernels README, intro and "Quick start").
  * ``decode``         -- the oracle's exact decoders of bf16 / fp16 / e4m3fn.
  * ``literal``        -- a second, pure-Python-loop oracle for tiny inputs.
  * ``dense``          -- brute-force dense attention over de-paged K/V, the
                          special case "every block selected".
  * ``index_ref``      -- integer CPU reference of the selection inversion and
                          the work split that the GPU index builder must match
                          bit for bit.
  * ``mxfp4``          -- exact decoder of MXFP4 caches (e2m1 codes, e8m0
                          scales per 32 values), the reading of the pages'
                          FP4; parity unpinned against the pages.
  * ``store_ref``      -- reference of the paged K/V store with its fp8 e4m3fn
                          cast (the step before the pass).
  * ``select_ref``     -- reference of block selection (index-key block scores,
                          then top-k), the step that produces ``selected``; its
                          scoring rule is a reading, parity unpinned against
                          the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmsa_oracle.so")
_lock = threading.Lock()
_lib = None

# dtype codes of msa_oracle.c
ORC_BF16, ORC_FP16, ORC_FP8_E4M3FN, ORC_FP32 = 0, 1, 2, 3
_DTYPE_CODE = {
    torch.bfloat16: ORC_BF16,
    torch.float16: ORC_FP16,
    torch.float8_e4m3fn: ORC_FP8_E4M3FN,
    torch.float32: ORC_FP32,
}
ERRORS = {
    -1: "bad argument",
    -2: "repeated block id within one (token, kv-head) selection",
    -3: "page id outside [0, num_pages) for a selected key",
    -4: "out of memory",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile msa_oracle.c with gcc (fp64, OpenMP) into libmsa_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.msa_oracle_attention.restype = i32
            lib.msa_oracle_attention.argtypes = [
                vp, i32, i64, i32,  # q, q_dtype, Tq, Hq
                vp, vp, i32,  # k, v, kv_dtype
                i64, i32, i32,  # num_pages, Hkv, page_size
                vp, i32,  # selected, topk
                vp, i32, i64,  # block_tables, B, max_pages
                vp, vp,  # cu_seqlens_q, used_kv_lens
                i32, dbl,  # causal, scale
                vp, i64,  # pairs, n_pairs
                vp, vp, i32,  # out, lse, threads
            ]
            lib.msa_oracle_decode.restype = i32
            lib.msa_oracle_decode.argtypes = [i32, vp, i64, vp]
            lib.msa_oracle_max_threads.restype = i32
            lib.msa_oracle_max_threads.argtypes = []
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().msa_oracle_max_threads())


def _cpu(x, dtype=None):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    x = x.detach().to("cpu")
    if dtype is not None:
        x = x.to(dtype)
    return x.contiguous()


def decode(x: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a bf16 / fp16 / e4m3fn / fp32 tensor, decoded by the oracle."""
    x = _cpu(x)
    code = _DTYPE_CODE[x.dtype]
    out = np.empty(x.numel(), dtype=np.float64)
    rc = _load().msa_oracle_decode(code, x.data_ptr(), x.numel(), out.ctypes.data)
    if rc != 0:
        raise OracleError(ERRORS.get(rc, rc))
    return out.reshape(tuple(x.shape))


def attention(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens,
              causal: bool, pairs=None, threads: int = 0, scale: float | None = None):
    """Run the fp64 oracle.

    Returns ``(out, lse)``: with ``pairs=None`` they are ``[Tq, Hq, 128]`` and
    ``[Hq, Tq]`` (the layouts of the pass); with ``pairs`` (ids ``t*Hkv + g``)
    they are ``[n_pairs, G, 128]`` and ``[n_pairs, G]``.
    """
    q = _cpu(q)
    k_cache = _cpu(k_cache)
    v_cache = _cpu(v_cache)
    selected = _cpu(selected, torch.int32)
    block_tables = _cpu(block_tables, torch.int32)
    cu = _cpu(cu_seqlens_q, torch.int64)
    used = _cpu(used_kv_lens, torch.int32)
    Tq, Hq, D = q.shape
    NP, Hkv, P, D2 = k_cache.shape
    assert D == 128 and D2 == 128 and v_cache.shape == k_cache.shape
    assert v_cache.dtype == k_cache.dtype
    topk = selected.shape[2]
    B = block_tables.shape[0]
    MP = block_tables.shape[1] if block_tables.dim() == 2 else 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(128.0)
    if pairs is None:
        n_pairs = Tq * Hkv
        pairs_t = None
    else:
        pairs_t = _cpu(torch.as_tensor(np.asarray(pairs, dtype=np.int64)), torch.int64)
        n_pairs = pairs_t.numel()
    out = np.empty((n_pairs, G, 128), dtype=np.float64)
    lse = np.empty((n_pairs, G), dtype=np.float64)
    rc = _load().msa_oracle_attention(
        q.data_ptr(), _DTYPE_CODE[q.dtype], Tq, Hq,
        k_cache.data_ptr(), v_cache.data_ptr(), _DTYPE_CODE[k_cache.dtype],
        NP, Hkv, P,
        selected.data_ptr(), topk,
        block_tables.data_ptr(), B, MP,
        cu.data_ptr(), used.data_ptr(),
        1 if causal else 0, float(scale),
        pairs_t.data_ptr() if pairs_t is not None else None, n_pairs,
        out.ctypes.data, lse.ctypes.data, int(threads),
    )
    if rc != 0:
        raise OracleError(ERRORS.get(rc, rc))
    if pairs is None:
        return out.reshape(Tq, Hq, 128), lse.reshape(Tq, Hq).T.copy()
    return out, lse
