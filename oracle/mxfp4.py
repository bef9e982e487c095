"""MXFP4 decoding -- TEST INFRASTRUCTURE (part of the oracle).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this module; the product library never imports it.

The MSA summary page ("Highlighted Details") lists FP4 and NVFP4 among the
kernels' formats but defines no scale format. The reading taken here is the
OCP microscaling format MXFP4, written out from its definition:

  * a row of 128 values is 32-value blocks j = 0..3 (dims 32 j .. 32 j + 31),
    each with one e8m0 scale byte s: the value 2^(s - 127), s = 255 is NaN;
  * each value is an e2m1 code: bit 3 the sign, bits 2..1 the exponent e
    (bias 1), bit 0 the mantissa m: (m / 2) for e = 0, else
    2^(e - 1) * (1 + m / 2);
  * codes are packed two a byte, value 2 i in the low nibble of byte i and
    value 2 i + 1 in the high nibble;
  * the stored value is code value x scale, exactly.

Parity of this reading against the pages is unpinned (they give no format);
the decoder is pinned to the definition above by ``tests/test_mxfp4_ref.py``.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Value of one e2m1 code (0..15)."""
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


def e8m0_value(b: int) -> float:
    """Value of one e8m0 scale byte (0..255)."""
    return float("nan") if b == 255 else 2.0 ** (int(b) - 127)


_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E8M0 = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def dequantize(codes, scales) -> np.ndarray:
    """float64 values [..., 128] of MXFP4 rows: ``codes`` [..., 64] and
    ``scales`` [..., 4] uint8 arrays (numpy or torch)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert codes.shape[-1] == 64 and scales.shape[-1] == 4 and codes.shape[:-1] == scales.shape[:-1]
    vals = np.empty(codes.shape[:-1] + (128,), dtype=np.float64)
    vals[..., 0::2] = _E2M1[codes & 15]
    vals[..., 1::2] = _E2M1[codes >> 4]
    return vals * np.repeat(_E8M0[scales], 32, axis=-1)
