"""Error budget of an e4m3 probability operand for P.V (CPU only).

gfx950's f8f6f4 MFMA would multiply the probabilities P by an fp8 V if P
were rounded to e4m3fn. This test emulates exactly that rounding (torch's
RNE cast of the fp32 probabilities exp2(s - m), with the row sum taken, as
in the kernels, over the unrounded fp32 values) and measures the output
error against the fp64 oracle, on decode-shaped fp8 inputs and on rows
whose attention is peaked on two or three keys.

The measured facts the design rests on: the error stays far inside
|dO| <= 1e-2 + 1e-2 |O_ref| on near-uniform rows (thousands of keys of
N(0,1) data), but exceeds it on peaked rows, where one probability carries
a relative rounding error of up to 2^-4 onto a value row of magnitude ~1.
So the fp8 P.V path cannot meet the pass's tolerance for every input.
"""
import numpy as np
import torch

import oracle
import workloads as W

TOL_A, TOL_R = 1e-2, 1e-2


def _emulate_fp8_pv(wl, k_cache, v_cache, t):
    """O[t] for every head, with P rounded to e4m3fn and V fp8, fp64 sums."""
    s = int(np.searchsorted(wl.cu_seqlens_q, t, side="right") - 1)
    L = int(wl.used_kv_lens[s])
    pos = L - int(wl.cu_seqlens_q[s + 1] - wl.cu_seqlens_q[s]) + (t - int(wl.cu_seqlens_q[s]))
    q = oracle.decode(wl.q[t])                         # [Hq, 128]
    out = np.zeros((wl.Hq, 128))
    for g in range(wl.Hkv):
        keys = sorted({j for b in wl.selected[t, g] if 0 <= b < -(-L // 128)
                       for j in range(128 * b, min(128 * b + 128, L)) if not wl.causal or j <= pos})
        pages = wl.block_tables[s, [j // wl.page_size for j in keys]]
        offs = [j % wl.page_size for j in keys]
        K = oracle.decode(k_cache[pages, g, offs])        # [n, 128]
        V = oracle.decode(v_cache[pages, g, offs])
        for r in range(wl.G):
            h = g * wl.G + r
            x = (K @ q[h]) / np.sqrt(128.0) * np.log2(np.e)   # log2 units
            p = np.exp2(np.float32(x - x.max())).astype(np.float32)
            l = np.float64(p.sum(dtype=np.float32))
            p8 = torch.from_numpy(p).to(torch.float8_e4m3fn).to(torch.float64).numpy()
            out[h] = (p8 @ V) / l
    return out


def _max_excess(wl, tokens):
    k, v = W.kv_pool(wl)
    ref_o, _ = oracle.attention(wl.q, k, v, wl.selected, wl.block_tables, wl.cu_seqlens_q, wl.used_kv_lens,
                                wl.causal)
    worst = 0.0
    for t in tokens:
        o = _emulate_fp8_pv(wl, k, v, t)
        err = np.abs(o - ref_o[t])
        worst = max(worst, float((err / (TOL_A + TOL_R * np.abs(ref_o[t]))).max()))
    return worst


def test_fp8_p_meets_the_tolerance_on_decode_shaped_rows():
    # decode_fp8's shape at a smaller batch: one token per sequence, 16
    # uniform picks of 128-key blocks, fp8 K/V, bf16 q
    wl = W.make_custom(1205, [1] * 6, [65536] * 6, 64, 8, 64, topk=16, causal=True, pick="random",
                       kv_dtype=torch.float8_e4m3fn)
    ratio = _max_excess(wl, range(wl.Tq))
    assert ratio < 1.0, ratio  # measured: the worst element uses about half of its tolerance


def test_fp8_p_breaks_the_tolerance_on_a_two_key_row():
    # One block of 128 keys in a 64-key page pair; q = sqrt(128) e_0, so a
    # key's score is its first component. Key 5 scores 2, key 77 scores
    # 1.375, every other key -16 (probability ~1e-8 relative): the row's
    # probabilities are 1 and e^-0.625 = 0.535, which e4m3fn rounds to 0.5625
    # (error 0.0275). All values are exact in bf16 and e4m3fn.
    wl = W.make_custom(1206, [1], [128], 1, 1, 64, topk=1, causal=False, pick="all", kv_dtype=torch.float8_e4m3fn)
    k, v = W.kv_pool(wl)
    kk = torch.zeros((128, 128))
    kk[:, 0] = -16.0
    kk[5, 0], kk[77, 0] = 2.0, 1.375
    vv = torch.from_numpy(np.random.default_rng(5).standard_normal((128, 128)).astype(np.float32) * 2)
    for j in range(128):
        page = wl.block_tables[0, j // 64]
        k[page, 0, j % 64] = kk[j].to(torch.float8_e4m3fn)
        v[page, 0, j % 64] = vv[j].clamp(-448, 448).to(torch.float8_e4m3fn)
    wl.q = torch.zeros((1, 1, 128)).to(torch.bfloat16)
    wl.q[0, 0, 0] = float(np.sqrt(128.0))
    ref_o, _ = oracle.attention(wl.q, k, v, wl.selected, wl.block_tables, wl.cu_seqlens_q, wl.used_kv_lens, False)
    o = _emulate_fp8_pv(wl, k, v, 0)
    ratio = float((np.abs(o - ref_o[0]) / (TOL_A + TOL_R * np.abs(ref_o[0]))).max())
    assert ratio > 1.0, ratio  # the rounding of one probability alone misses the tolerance
