"""Pins of the paged K/V store reference and its e4m3fn cast (CPU).

The cast is pinned to what the pages state it must equal bit for bit,
``x.float().clamp(-448, 448).to(float8_e4m3fn)`` (sglang pull request
"Speed up MiniMax-M3 sparse attention on Hopper", "Verification"), on every
bf16 and every fp16 value, and to hand-worked values of the format.
"""
import numpy as np
import pytest
import torch

from oracle import store_ref as S


def _torch_cast(x32: torch.Tensor) -> np.ndarray:
    return x32.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_cast_matches_the_stated_rule_on_every_16_bit_value(dtype):
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(dtype)
    x32 = x.float()
    got = S.e4m3fn_encode(x32.numpy())
    want = _torch_cast(x32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(b)), float(x32[b]), hex(got[b]), hex(want[b])) for b in bad[:8]]


def test_cast_matches_on_random_fp32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 50.0, 400.0)]).astype(np.float32)
    got = S.e4m3fn_encode(x)
    assert np.array_equal(got, _torch_cast(torch.from_numpy(x)))


@pytest.mark.parametrize("value, code", [
    (0.0, 0x00), (-0.0, 0x80), (-1e-10, 0x80),
    (2.0 ** -9, 0x01),           # smallest subnormal
    (2.0 ** -10, 0x00),          # half of it: tie, to the even code 0
    (3 * 2.0 ** -11, 0x01),      # three quarters of it: rounds up
    (2.0 ** -6, 0x08),           # smallest normal
    (1.0, 0x38), (-1.0, 0xB8),
    (17.0, 0x58),                # 17 lies halfway between 16 and 18: to the even mantissa (16)
    (19.0, 0x5A),                # halfway between 18 and 20: to 20
    (448.0, 0x7E), (1e6, 0x7E), (float("inf"), 0x7E), (float("-inf"), 0xFE),
    (float("nan"), 0x7F),
])
def test_cast_hand_values(value, code):
    assert int(S.e4m3fn_encode(np.array([value]))[0]) == code


def test_decode_then_encode_is_the_identity_on_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(S.e4m3fn_encode(S.e4m3fn_decode(codes)), codes)


def test_cast_is_the_nearest_code():
    # the decoded code is never further from the clamped value than any other code
    rng = np.random.default_rng(11)
    x = rng.uniform(-500, 500, size=4000)
    grid = S.e4m3fn_decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8))
    xc = np.clip(x, -448, 448)
    got = S.e4m3fn_decode(S.e4m3fn_encode(x))
    best = np.min(np.abs(grid[None, :] - xc[:, None]), axis=1)
    assert np.all(np.abs(got - xc) <= best)


def test_store_writes_the_slots_and_nothing_else():
    rng = np.random.default_rng(3)
    NP, Hkv, P, N = 5, 2, 64, 9
    k_new = rng.standard_normal((N, Hkv, 128)) * 30
    v_new = rng.standard_normal((N, Hkv, 128)) * 30
    loc = rng.permutation(NP * P)[:N].astype(np.int64)
    loc[2] = -1          # skipped
    loc[5] = NP * P + 3  # beyond the cache: skipped
    k16, v16 = np.full((NP, Hkv, P, 128), 7.0), np.full((NP, Hkv, P, 128), 7.0)
    k8, v8 = np.full((NP, Hkv, P, 128), 0x11, np.uint8), np.full((NP, Hkv, P, 128), 0x11, np.uint8)
    S.store_kv(k_new, v_new, loc, k16, v16, P)
    S.store_kv(k_new, v_new, loc, k8, v8, P)
    written = np.zeros((NP, P), dtype=bool)
    for i, slot in enumerate(loc):
        if 0 <= slot < NP * P:
            pg, off = slot // P, slot % P
            written[pg, off] = True
            assert np.array_equal(k16[pg, :, off], k_new[i]) and np.array_equal(v16[pg, :, off], v_new[i])
            assert np.array_equal(k8[pg, :, off], _torch_cast(torch.from_numpy(k_new[i]).float()))
            assert np.array_equal(v8[pg, :, off], _torch_cast(torch.from_numpy(v_new[i]).float()))
    untouched = ~written
    assert np.all(k16.transpose(0, 2, 1, 3)[untouched] == 7.0)
    assert np.all(v8.transpose(0, 2, 1, 3)[untouched] == 0x11)
