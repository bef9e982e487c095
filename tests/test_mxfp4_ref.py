"""Pins of the oracle's MXFP4 decoder (CPU only).

The decoder (oracle/mxfp4.py) follows the reading of the pages' FP4 stated
there: OCP MXFP4, e2m1 codes with one e8m0 scale per 32 values. These pins
tie it to that definition from outside its own formulas: the e2m1 value
table as the format lists it, the scale at its anchor points, the nibble
order and the 32-value blocks on hand-made rows, and exactness in float32
(the oracle's attention takes the decoded caches as fp32).
"""
import numpy as np
import pytest

from oracle import mxfp4

# The e2m1 values as the format lists them: codes 0..7 positive, 8..15 the
# same magnitudes negative.
E2M1_LISTED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_every_e2m1_code():
    got = [mxfp4.e2m1_value(c) for c in range(16)]
    assert got[:8] == E2M1_LISTED
    assert got[8:] == [-x for x in E2M1_LISTED]
    assert np.signbit(got[8])  # code 8 is -0


def test_e8m0_anchor_points():
    assert mxfp4.e8m0_value(127) == 1.0
    assert mxfp4.e8m0_value(128) == 2.0
    assert mxfp4.e8m0_value(126) == 0.5
    assert mxfp4.e8m0_value(0) == 2.0 ** -127
    assert mxfp4.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(mxfp4.e8m0_value(255))


def test_low_nibble_is_the_first_value():
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 0] = 0x21  # value 0: code 1 (0.5), value 1: code 2 (1.0)
    codes[0, 1] = 0xF7  # value 2: code 7 (6.0), value 3: code 15 (-6.0)
    v = mxfp4.dequantize(codes, np.full((1, 4), 127, np.uint8))
    assert v[0, :4].tolist() == [0.5, 1.0, 6.0, -6.0]
    assert not v[0, 4:].any()


def test_one_scale_per_32_values():
    codes = np.full((1, 64), 0x22, np.uint8)  # every value 1.0
    scales = np.array([[127, 128, 126, 130]], np.uint8)
    v = mxfp4.dequantize(codes, scales)[0]
    assert (v[0:32] == 1.0).all() and (v[32:64] == 2.0).all()
    assert (v[64:96] == 0.5).all() and (v[96:128] == 8.0).all()


def test_batch_shapes_and_every_byte():
    # every code byte once per row position, scales varying by row
    rng = np.random.default_rng(7)
    codes = np.tile(np.arange(256, dtype=np.uint8).reshape(4, 64), (3, 1, 1))  # [3, 4, 64]
    scales = rng.integers(120, 135, size=(3, 4, 4)).astype(np.uint8)
    v = mxfp4.dequantize(codes, scales)
    assert v.shape == (3, 4, 128)
    for i in range(3):
        for r in range(4):
            for d in range(128):
                byte = int(codes[i, r, d // 2])
                code = byte & 15 if d % 2 == 0 else byte >> 4
                want = E2M1_LISTED[code & 7] * (-1 if code & 8 else 1) * 2.0 ** (int(scales[i, r, d // 32]) - 127)
                assert v[i, r, d] == want


@pytest.mark.parametrize("s", [1, 60, 127, 200, 252])
def test_values_are_exact_in_float32(s):
    codes = np.arange(256, dtype=np.uint8).reshape(4, 64)
    v = mxfp4.dequantize(codes, np.full((4, 4), s, np.uint8))
    assert np.array_equal(v.astype(np.float32).astype(np.float64), v)
