"""Integer CPU reference of the selection inversion and work split -- TEST INFRASTRUCTURE.

The GPU index builder must reproduce these arrays bit for bit. The rules are
the library's own (the pages name an index builder and a load-balancing
scheduler -- fw-ai/minimax-kernels README, "Tests" -- but do not define
them); they are restated here plainly:

Slot (t, g, k) holds block b = selected[t, g, k]. Token t belongs to the
sequence s with cu[s] <= t < cu[s+1]; with L = used_kv_lens[s] and
Tq_s = cu[s+1] - cu[s], its position is pos = L - Tq_s + (t - cu[s]).
The slot is VALID when 0 <= b < min(ceil(L/128), nb_max) and, if causal,
128*b <= pos (the block holds at least one visible key).

Tiles: the tokens of each sequence are cut into runs of ``tile_tokens``
consecutive tokens (the last run may be shorter); the first token of a run
is its leader. For a tile and KV head g, the CHAIN is the list of blocks
that every token of the tile selected validly, in the order of the leader's
picks. ``tile_tokens == 0`` disables chains (tiles are then single tokens
with empty chains).

A valid slot whose block is in its tile's chain is COVERED (flag 1); any
other valid slot is RESIDUAL (flag 2); invalid slots have flag 0.

Residual slots are inverted into rows r = b*Hkv + g (nb_max*Hkv rows):
``row_off`` is the exclusive scan of the per-row counts, ``ent`` lists the
residual slot ids of each row in ascending slot id, and ``slot_pos[slot]``
is the slot's index in ``ent`` (-1 for non-residual slots). Each row is cut
into units of at most ``unit_tokens`` entries; ``unit_off`` is the
exclusive scan of ceil(count/unit_tokens).

Per (t, g): ``tok_chain`` is the chain length of t's tile and ``tok_nres``
the number of residual slots of (t, g). Tiles (t_leader, g) form the tile
work list, except -- unless ``list_all_tiles`` is set -- tiles of at most 16
query rows (tile tokens x G) none of whose slots is residual: the
classifier finishes those itself.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Plan:
    tile_tokens: int
    unit_tokens: int
    nb_max: int
    slot_flag: np.ndarray      # [Tq, Hkv, K] uint8
    tok_chain: np.ndarray      # [Tq, Hkv] int32
    tok_nres: np.ndarray       # [Tq, Hkv] int32
    chain_blk: dict            # (leader t, g) -> list of blocks
    row_off: np.ndarray        # [nb_max*Hkv + 1] int32
    ent: np.ndarray            # [nres] int32
    slot_pos: np.ndarray       # [Tq, Hkv, K] int32
    unit_off: np.ndarray       # [nb_max*Hkv + 1] int32
    tile_items: set            # {t0*Hkv + g} tiles left to the tile kernel


def token_sequence(cu: np.ndarray, Tq: int) -> np.ndarray:
    """Owner sequence of each token (-1 outside every sequence)."""
    seq = np.full(Tq, -1, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        a, b = max(a, 0), min(b, Tq)
        if b > a:
            seq[a:b] = np.where(seq[a:b] < 0, s, seq[a:b])
    return seq


def slot_validity(selected, cu, used, causal, nb_max):
    Tq, Hkv, K = selected.shape
    cu = np.asarray(cu, dtype=np.int64)
    used = np.asarray(used, dtype=np.int64)
    seq = token_sequence(cu, Tq)
    has = seq >= 0
    s = np.where(has, seq, 0)
    L = np.where(has, used[s], 0)
    Tq_s = np.where(has, cu[s + 1] - cu[s], 0)
    pos = L - Tq_s + (np.arange(Tq) - np.where(has, cu[s], 0))
    nblk = np.minimum((L + 127) // 128, nb_max)
    b = selected.astype(np.int64)
    valid = has[:, None, None] & (b >= 0) & (b < nblk[:, None, None])
    if causal:
        valid &= (128 * b) <= pos[:, None, None]
    return seq, valid


def build(selected, cu, used, causal: bool, tile_tokens: int, unit_tokens: int,
          nb_max: int, G: int, list_all_tiles: bool = False) -> Plan:
    selected = np.asarray(selected, dtype=np.int32)
    Tq, Hkv, K = selected.shape
    cu = np.asarray(cu, dtype=np.int64)
    seq, valid = slot_validity(selected, cu, used, causal, nb_max)
    b64 = selected.astype(np.int64)

    # membership of (t, g, b) among valid picks
    tgb = (np.arange(Tq)[:, None, None] * Hkv + np.arange(Hkv)[None, :, None]) * nb_max + b64
    member = np.unique(tgb[valid])

    def has_pick(t, g, b):
        key = (t * Hkv + g) * nb_max + b
        i = np.searchsorted(member, key)
        return (i < member.size) & (member[np.minimum(i, member.size - 1)] == key)

    slot_flag = np.where(valid, 2, 0).astype(np.uint8)
    tok_chain = np.zeros((Tq, Hkv), dtype=np.int32)
    chain_blk = {}
    tiles = set()
    T = max(tile_tokens, 1)
    for s in range(len(cu) - 1):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        for t0 in range(q0, q1, T):
            t1 = min(t0 + T, q1)
            toks = np.arange(t0, t1)
            for g in range(Hkv):
                chain = []
                for k in range(K if tile_tokens > 0 else 0):
                    if not valid[t0, g, k]:
                        continue
                    bb = int(b64[t0, g, k])
                    if bb in chain:
                        continue
                    if np.all(has_pick(toks, g, bb)):
                        chain.append(bb)
                chain_blk[(t0, g)] = chain
                tok_chain[t0:t1, g] = len(chain)
                if chain:
                    cover = valid[t0:t1, g, :] & np.isin(b64[t0:t1, g, :], chain)
                    slot_flag[t0:t1, g, :][cover] = 1
                has_res = bool(np.any(slot_flag[t0:t1, g, :] == 2))
                if list_all_tiles or (t1 - t0) * G > 16 or has_res:
                    tiles.add(t0 * Hkv + g)
    tok_nres = (slot_flag == 2).sum(axis=2).astype(np.int32)

    NR = nb_max * Hkv
    slot_ids = np.arange(Tq * Hkv * K, dtype=np.int64).reshape(Tq, Hkv, K)
    res = slot_flag == 2
    rows = (b64 * Hkv + np.arange(Hkv)[None, :, None])[res]
    ids = slot_ids[res]
    order = np.lexsort((ids, rows))
    rows, ids = rows[order], ids[order]
    cnt = np.bincount(rows, minlength=NR).astype(np.int64)
    row_off = np.zeros(NR + 1, dtype=np.int64)
    row_off[1:] = np.cumsum(cnt)
    slot_pos = np.full(Tq * Hkv * K, -1, dtype=np.int64)
    slot_pos[ids] = np.arange(ids.size)
    units = (cnt + unit_tokens - 1) // unit_tokens
    unit_off = np.zeros(NR + 1, dtype=np.int64)
    unit_off[1:] = np.cumsum(units)
    return Plan(
        tile_tokens=tile_tokens, unit_tokens=unit_tokens, nb_max=nb_max,
        slot_flag=slot_flag, tok_chain=tok_chain, tok_nres=tok_nres, chain_blk=chain_blk,
        row_off=row_off.astype(np.int32), ent=ids.astype(np.int32),
        slot_pos=slot_pos.reshape(Tq, Hkv, K).astype(np.int32),
        unit_off=unit_off.astype(np.int32), tile_items=tiles,
    )
