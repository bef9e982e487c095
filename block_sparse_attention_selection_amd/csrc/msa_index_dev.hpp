// msa_index_dev.hpp -- device functions of the residual inversion and of the
// tile descriptors, shared by the classifiers (msa_forward.hip), the index
// kernels (msa_index.hip) and the unit and tile kernels (msa_tiles.hip).
#pragma once

#include "msa_device.hpp"
#include <limits.h>

#include "msa_internal.hpp"

namespace msa {

// exclusive scan across a workgroup of NT threads (NT a multiple of 64)
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int* total, int* smem) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) smem[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int v = (lane < NW) ? smem[lane] : 0;
    int vi = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(vi, off, 64);
      if (lane >= off) vi += y;
    }
    if (lane < NW) smem[lane] = vi - v;
    if (lane == NW - 1) smem[NW] = vi;
  }
  __syncthreads();
  const int res = smem[wid] + incl - x;
  *total = smem[NW];
  __syncthreads();
  return res;
}

// Row r (block b, KV head g): popcount prefix of its token bitmap, by one
// wave (the words are split over the 64 lanes and scanned with cross-lane
// shuffles, so a workgroup's rows are processed side by side, one per wave);
// the words are copied to wordbits and cleared. Returns the row's count to
// every lane.
__device__ __forceinline__ int rowcount_row_wave(const Params& p, int r) {
  const int lane = threadIdx.x & 63;
  uint32_t* bm = p.bitmap + (size_t)r * p.W;
  uint32_t* pre = p.wordpre + (size_t)r * p.W;
  uint32_t* bits = p.wordbits + (size_t)r * p.W;
  const int per = (p.W + 63) / 64;
  const int w0 = min(lane * per, p.W);
  const int w1 = min(w0 + per, p.W);
  int sum = 0;
  for (int w = w0; w < w1; ++w) sum += __popc(bm[w]);
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  int run = incl - sum;
  const int total = __shfl(incl, 63, 64);
  for (int w = w0; w < w1; ++w) {
    const uint32_t x = bm[w];
    pre[w] = (uint32_t)run;
    bits[w] = x;
    bm[w] = 0u;  // leave the bitmap clear for the next call
    run += __popc(x);
  }
  return total;
}

// Exclusive scans of the row counts (row_off) and of the units per row
// (unit_off); the unit total goes to counters[kCntUnits]. The row counts are
// read with agent-scope atomic loads: they were published by other
// workgroups of the same kernel through atomic stores.
template <int NT>
__device__ __forceinline__ void rowscan_all(const Params& p, int* smem) {
  const int NR = p.NR;
  const int per = (NR + NT - 1) / NT;
  const int r0 = min((int)threadIdx.x * per, NR);
  const int r1 = min(r0 + per, NR);
  int cnt = 0, units = 0;
  for (int r = r0; r < r1; ++r) {
    const int c = __hip_atomic_load(&p.row_cnt[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cnt += c;
    units += (c + p.Tu - 1) / p.Tu;
  }
  int tot_cnt, tot_units;
  int run_c = block_excl_scan<NT>(cnt, &tot_cnt, smem);
  int run_u = block_excl_scan<NT>(units, &tot_units, smem);
  for (int r = r0; r < r1; ++r) {
    const int c = __hip_atomic_load(&p.row_cnt[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p.row_off[r] = run_c;
    p.unit_off[r] = run_u;
    const int nu = (c + p.Tu - 1) / p.Tu;
    if (p.win_desc) {  // (row, first rank, first entry, entries) of each of the row's windows
      for (int i = 0; i < nu; ++i) {
        const int rank0 = i * p.Tu;
        p.win_desc[run_u + i] = int4{r, rank0, run_c + rank0, min(p.Tu, c - rank0)};
      }
    }
    run_c += c;
    run_u += nu;
  }
  if (threadIdx.x == 0) {
    p.row_off[NR] = tot_cnt;
    p.unit_off[NR] = tot_units;
    p.counters[kCntUnits] = tot_units;
    p.counters[kCntResidual] = tot_cnt;  // every workgroup of this kernel has read the flag by now
  }
}

// element offset of the 32-key chunk starting at key0 of sequence s, KV head
// g, or -1 when the chunk lies beyond the keys the page table can reach or
// its page is out of range (its keys are then treated as absent)
__device__ __forceinline__ int64_t chunk_offset(const Params& p, int s, int g, int key0, int Leff) {
  if (key0 >= Leff) return -1;
  const int page = p.block_tables[(size_t)s * p.MP + key0 / p.P];
  if (page < 0 || page >= p.NP) return -1;
  return (((int64_t)page * p.Hkv + g) * p.P + (key0 % p.P)) * 128;
}

// Descriptor and chunk table of tile item `item` (tile leader t0 of sequence
// s, nt tokens, KV head g, chain of n_ch blocks): tdesc[2 item] = (t0, s, nt,
// chunks in the table), tdesc[2 item + 1] = (reachable keys Leff, base
// position: pos = base + token, g, nfull), and the table ctab[item * 4 topk
// + ...] of (element offset low, high, first key, keys present) per chunk.
// Chunks that start after the tile's last position are left out (no row
// sees a key of them); a chunk whose page id lies outside the pool, or that
// starts at or beyond Leff, has offset -1 and no keys present. The table
// lists first the nfull chunks every row of the tile sees whole (32 keys
// present, all at or before the first row's position), then the others,
// each class in chain order, so that the tile kernel runs its unmasked
// loop up to nfull and masks the rest against their first key + keys
// present. One wave calls this (lane 0..63).
__device__ __forceinline__ void write_tile_desc(const Params& p, int item, int t0, int s, int nt, int n_ch, int L,
                                                int Tq_s, int64_t q0, int g, const int* chain, int lane) {
  const int Leff = min(L, p.MP * p.P);
  const int base = (int)(L - Tq_s - q0);
  const int pmax = p.causal ? base + t0 + nt - 1 : INT_MAX;
  const int pmin = p.causal ? base + t0 : INT_MAX;
  const size_t K4 = 4 * (size_t)p.K;
  const int n = 4 * n_ch;  // at most 4 * 64: four batches of 64 chunks
  auto key_of = [&](int ci) { return 128 * chain[ci >> 2] + 32 * (ci & 3); };
  int64_t offs[4];
  bool used[4];  // the chunk has a key at or before the tile's last position
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = 64 * i + lane;
    const int key0 = ci < n ? key_of(ci) : 0;
    used[i] = ci < n && key0 <= pmax;
    offs[i] = used[i] ? chunk_offset(p, s, g, key0, Leff) : (int64_t)-1;
  }
  auto whole = [&](int ci, int64_t off) {
    const int k0 = key_of(ci);
    return off >= 0 && k0 + 31 < Leff && k0 + 31 <= pmin;
  };
  int nfull = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = 64 * i + lane;
    nfull += __popcll(__ballot(used[i] && whole(ci, offs[i])));
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int fb = 0, pb = 0;  // whole / other chunks of earlier batches
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = 64 * i + lane;
    const bool in = used[i];
    const int64_t off = offs[i];
    const bool f = in && whole(ci, off);
    const uint64_t bf = __ballot(f), bo = __ballot(in && !f);
    if (in) {
      const int at = f ? fb + __popcll(bf & below) : nfull + pb + __popcll(bo & below);
      const int key0 = key_of(ci);
      const int present = off >= 0 ? min(32, Leff - key0) : 0;
      p.ctab[(size_t)item * K4 + at] = int4{(int)(uint32_t)(uint64_t)off, (int)(off >> 32), key0, present};
    }
    fb += __popcll(bf);
    pb += __popcll(bo);
  }
  if (lane == 0) {
    p.tdesc[2 * (size_t)item] = int4{t0, s, nt, fb + pb};
    p.tdesc[2 * (size_t)item + 1] = int4{Leff, base, g, nfull};
  }
}

// Index of residual slot (t, g) -> block b in the residual order: the row's
// offset plus the token's rank among the row's set bits. The row data were
// written by an earlier kernel.
__device__ __forceinline__ int residual_pos(const Params& p, int t, int g, int b) {
  const size_t r = (size_t)b * p.Hkv + g;
  const size_t w = r * p.W + (t >> 5);
  const uint32_t below = p.wordbits[w] & ((1u << (t & 31)) - 1u);
  return p.row_off[r] + (int)p.wordpre[w] + __popc(below);
}

// Materialises the residual order for one slot: ent[pos] = slot, and, when
// present, slot_pos[slot] = pos (staged index entry point) and the slot's
// entry in its (t, g) residual list, res_list[tg * K + rank] = pos (attention;
// rank from res_rank). Flags of tokens this call did not classify (only with
// malformed cu_seqlens) are ignored: their bit is not set.
__device__ __forceinline__ void emit_slot(const Params& p, int64_t slot) {
  if (p.slot_flag[slot] != 2) return;
  // slot = (t * Hkv + g) * K + k; in 32 bits while the slot numbers fit
  int t, g;
  if (slot <= 0xFFFFFFFFll) {
    const uint32_t tg = (uint32_t)slot / (uint32_t)p.K;
    t = (int)(tg / (uint32_t)p.Hkv);
    g = (int)(tg - (uint32_t)t * (uint32_t)p.Hkv);
  } else {
    t = (int)(slot / ((int64_t)p.Hkv * p.K));
    g = (int)((slot / p.K) % p.Hkv);
  }
  const int b = p.selected[slot];
  if (b < 0 || b >= p.nb_max) return;
  const size_t w = ((size_t)b * p.Hkv + g) * p.W + (t >> 5);
  if (!((p.wordbits[w] >> (t & 31)) & 1u)) return;
  const int pos = residual_pos(p, t, g, b);
  p.ent[pos] = (int)slot;
  if (p.slot_pos) p.slot_pos[slot] = pos;
  if (p.res_list) {
    const int64_t k = slot - ((int64_t)t * p.Hkv + g) * p.K;
    p.res_list[slot - k + p.res_rank[slot]] = pos;
  }
}

}  // namespace msa
