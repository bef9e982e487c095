"""MI355X (gfx950) MiniMax-M3 block-sparse attention forward.

Python surface mirroring the ``kvouter_attention`` call of the
fw-ai/minimax-kernels README ("Quick start"): token-major queries, a paged
KV cache, per-(token, KV head) block selections and the page table in;
``out [Tq, Hq, 128]`` and optionally the fp32 ``lse [Hq, Tq]`` back.

This module only marshals arguments into the C ABI of
``include/msa_kvouter.h`` (``lib/libmsa_kvouter.so``); every step of the
computation runs in the library's HIP kernels. There is no other path: if
the library is missing or a request is unsupported, the call raises.
"""
from __future__ import annotations

from ._lib import (
    MSA_BF16,
    MSA_FP16,
    MSA_FP8_E4M3FN,
    MSA_FP32,
    MSA_INT32,
    MSA_INT64,
    MSA_UINT8,
    MsaError,
    build_index,
    kvouter_attention,
    kvouter_attention_mxfp4,
    kvouter_attention_noalloc,
    lib_path,
    load,
    profile_collect,
    profile_enable,
    store_kv,
    select_blocks,
    set_workspace_limit,
    validate_inputs,
    version,
    widen_fp8,
    workspace_bytes,
)

__all__ = [
    "kvouter_attention",
    "kvouter_attention_mxfp4",
    "kvouter_attention_noalloc",
    "workspace_bytes",
    "build_index",
    "widen_fp8",
    "store_kv",
    "select_blocks",
    "set_workspace_limit",
    "validate_inputs",
    "version",
    "load",
    "profile_enable",
    "profile_collect",
    "lib_path",
    "MsaError",
    "MSA_BF16",
    "MSA_FP16",
    "MSA_FP8_E4M3FN",
    "MSA_FP32",
    "MSA_INT32",
    "MSA_INT64",
    "MSA_UINT8",
]
