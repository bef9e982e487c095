"""Reference of the paged K/V store with an fp8 cast -- TEST INFRASTRUCTURE.

Only the test suite may import this module; the product library never
imports, links or runs it and shares no code with it.

The step before the attention pass writes the keys and values of new tokens
into the slots of the paged caches. The sglang pull request "Speed up
MiniMax-M3 sparse attention on Hopper" (summary and "Verification") fuses
that store with an unscaled cast of 16-bit values to fp8 e4m3fn and states
its result: bit-exact with ``x.float().clamp(-448, 448).to(float8_e4m3fn)``.

Readings (the pages give the cast, not the store's interface):
  * A new token i has a flat cache slot ``loc[i] = page * page_size + offset``
    (the usual paged-cache location); its K and V rows for KV head g go to
    ``cache[page, g, offset, :]`` of the ``[num_pages, Hkv, page_size, 128]``
    caches the attention pass reads. A negative slot, or one at or beyond
    ``num_pages * page_size``, stores nothing.
  * A cache of the new values' own dtype receives them unchanged; an fp8
    e4m3fn cache receives the cast above.

``e4m3fn_encode`` writes out that cast from the format's definition: sign,
4 exponent bits with bias 7, 3 mantissa bits; subnormals step by 2^-9; the
largest finite value is 448 (exponent field 15, mantissa 6); exponent field
15 with mantissa 7 is NaN. The value is clamped to [-448, 448] and rounded
to the nearest representable value, ties to the even mantissa; NaN keeps
its sign bit and becomes the NaN code.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUB_STEP = 2.0 ** -9


def e4m3fn_encode(x) -> np.ndarray:
    """uint8 e4m3fn codes of the float values x (any float dtype, exact in float64)."""
    with np.errstate(invalid="ignore"):  # signalling NaN inputs become quiet NaNs
        x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)  # the clamp (|inf| -> 448)
    # quantisation step of the binade holding a: 2^(e - 3) for normals
    # (e = floor(log2 a) >= -6), 2^-9 below the smallest normal
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.where(a >= _MIN_NORMAL, np.exp2(e - 3), _SUB_STEP)
    n = np.rint(a / step)  # round half to even: the quotient's halves are exact
    v = n * step           # the rounded magnitude (may step up into the next binade)
    # code of v
    code = np.zeros(a.shape, dtype=np.int64)
    sub = v < _MIN_NORMAL
    code[sub] = np.rint(v[sub] / _SUB_STEP).astype(np.int64)
    nv = ~sub
    with np.errstate(divide="ignore"):
        ev = np.floor(np.log2(np.where(nv, v, 1.0)))
    mant = np.rint(v / np.exp2(ev) * 8.0 - 8.0).astype(np.int64)
    code[nv] = ((ev[nv].astype(np.int64) + 7) << 3) | mant[nv]
    out = (code.astype(np.uint8) | sign).astype(np.uint8)
    out[nan] = (0x7F | sign[nan]).astype(np.uint8)
    return out


def e4m3fn_decode(codes) -> np.ndarray:
    """float64 values of uint8 e4m3fn codes (NaN codes give NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * _SUB_STEP, (1.0 + m / 8.0) * np.exp2(e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def store_kv(k_new, v_new, loc, k_cache, v_cache, page_size: int):
    """The store on numpy arrays, in place on k_cache / v_cache.

    k_new, v_new: [N, Hkv, 128] float arrays (the 16-bit inputs' exact
    values); loc: [N] integer slots; caches: [NP, Hkv, P, 128] float
    arrays (16-bit caches: same values) or uint8 arrays (fp8 caches: codes).
    """
    NP = k_cache.shape[0]
    fp8 = k_cache.dtype == np.uint8
    for i, slot in enumerate(np.asarray(loc, dtype=np.int64)):
        if slot < 0 or slot >= NP * page_size:
            continue
        page, off = divmod(int(slot), page_size)
        for cache, src in ((k_cache, k_new), (v_cache, v_new)):
            rows = np.asarray(src[i], dtype=np.float64)
            cache[page, :, off, :] = e4m3fn_encode(rows) if fp8 else rows
    return k_cache, v_cache
