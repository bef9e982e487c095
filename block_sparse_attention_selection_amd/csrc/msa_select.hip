// msa_select.hip -- block selection, the step that produces `selected`:
// every (query token, KV head) scores the 128-token blocks of its sequence
// with index keys and keeps the top-k.
//
// The MSA README ("How It Works", "Highlighted Details") lists sparse top-k
// selection beside its attention kernels, and the sglang pull request "Speed
// up MiniMax-M3 sparse attention on Hopper" ("Changes to existing code")
// keeps a sparse index K cache next to the K/V caches (fp8 with fp8 KV). The
// scoring is not given there; the rule implemented is:
//   score(t, g, b) = max over the visible tokens j of block b of
//                    q_idx[t, g, :] . k_idx(s, g, j, :)
// (visible: j < L_s and, when causal, j <= pos(t), the attention pass's
// bottom-right position), and selected[t, g, :] lists the token's own block
// first (when force_local), then the other blocks by descending score, equal
// scores by ascending block id, padded with -1. Blocks without a visible
// token, and NaN scores, are never selected.
//
// Work: S^T = K . Q^T with 16x16x32 MFMA for 16 keys at a time, max-pooled
// per (query row, block) into an fp32 score table [Tq, Hkv, nb]; a second
// launch lists every row from the table (one wave per row).
// Prefill-shaped batches: one workgroup of 4 waves per (256-token tile of
// one sequence, KV head, slice of 8 blocks); each block's keys are brought
// into LDS once and shared by the four waves (64 query rows each).
// Decode-shaped batches (a few tokens per long sequence): 16-token tiles,
// each sequence's blocks split over several workgroups whose waves read the
// keys straight from the paged cache into operand registers (a lane reads 32
// contiguous dims of one key row).
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {


// 32 consecutive index-key dims of one row, as four 8-value MFMA fragments
template <typename QT, typename KT>
struct KeyRow;

template <typename QT>
struct KeyRow<QT, QT> {  // 16-bit keys: 64 bytes
  u32x4 w[4];
  __device__ __forceinline__ void load(const void* row, int h) {
    const u32x4* p = (const u32x4*)((const uint16_t*)row + 32 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = p[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // from a block staged in LDS (row r's 16-byte piece c at r * 16 + (c ^ sw))
  __device__ __forceinline__ void load_lds(const u32x4* blk, int row, int sw, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = blk[row * 16 + ((4 * h + i) ^ sw)];
  }
  __device__ __forceinline__ u32x4 frag(int st) const { return w[st]; }
};

template <typename QT>
struct KeyRow<QT, fp8_e4m3_t> {  // e4m3fn keys: 32 bytes, widened exactly when used
  u32x4 w[2];
  __device__ __forceinline__ void load(const void* row, int h) {
    const u32x4* p = (const u32x4*)((const uint8_t*)row + 32 * h);
    w[0] = p[0];
    w[1] = p[1];
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = u32x4{0u, 0u, 0u, 0u}; }
  // from a block staged in LDS (row r's 16-byte piece c at r * 8 + (c ^ sw))
  __device__ __forceinline__ void load_lds(const u32x4* blk, int row, int sw, int h) {
    w[0] = blk[row * 8 + ((2 * h) ^ sw)];
    w[1] = blk[row * 8 + ((2 * h + 1) ^ sw)];
  }
  __device__ __forceinline__ u32x4 frag(int st) const {
    const u32x4 x = w[st >> 1];
    return (st & 1) ? widen8<QT>(u32x2{x[2], x[3]}) : widen8<QT>(u32x2{x[0], x[1]});
  }
};

template <typename KT>
struct KeyBytes {
  static constexpr int kRow = 256;  // 128 16-bit values
};
template <>
struct KeyBytes<fp8_e4m3_t> {
  static constexpr int kRow = 128;
};

// (value, block) order of the selection: larger value first, then lower block
__device__ __forceinline__ bool sel_better(float v, int b, float v2, int b2) {
  return v > v2 || (v == v2 && b < b2);
}

// The tile of workgroup-level work: token rows [t0, t0 + ntok) of sequence s
// for KV head g, with the sequence's clamped length and the block range
// [0, nscan) that some row of the tile sees.
struct SelTile {
  int s, g, ntok, L, nb, nscan;
  int64_t t0, c0, tq_s;
  bool causal;
  // position of tile row r (bottom-right causal alignment); L - 1 when not causal
  __device__ __forceinline__ int64_t pos(int r) const { return causal ? (int64_t)L - tq_s + (t0 + r - c0) : (int64_t)L - 1; }
};

__device__ __forceinline__ bool sel_tile(const SelectParams& p, int tile, int g, int T, SelTile* st) {
  int64_t t0 = 0;
  const int s = wave_tile_of(p.cu, p.B, p.Tq, T, tile, &t0);
  if (s < 0) return false;
  SelTile& x = *st;
  x.s = s;
  x.g = g;
  x.t0 = t0;
  x.c0 = p.cu[s];
  const int64_t c1 = p.cu[s + 1];
  x.tq_s = c1 - x.c0;
  x.ntok = (int)min((int64_t)T, min(c1, (int64_t)p.Tq) - t0);
  // a sequence reaches no further than its page table (and nowhere without a cache)
  x.L = p.num_pages > 0 ? min(p.used[s], p.MP * p.P) : 0;
  x.causal = p.causal != 0;
  x.nb = min((x.L + 127) / 128, p.nb_cap);
  const int64_t pos_max = x.pos(x.ntok - 1);
  x.nscan = (x.L <= 0 || pos_max < 0) ? 0 : (int)min((int64_t)x.nb, pos_max / 128 + 1);
  return true;
}

// Block scores of the tile's rows for blocks [b0, b1) (b1 <= nscan): wave w
// takes blocks b0 + w, b0 + w + NW, ...; row r's score of block b goes to
// dst[r * row_stride + b].
template <typename QT, typename KT, int NRB, int NW>
__device__ __forceinline__ void score_blocks(const SelectParams& p, const SelTile& x, int b0, int b1, float* dst,
                                             int64_t row_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = x.g, L = x.L;
  // index queries of the tile as MFMA B operands: lane holds token row
  // (lane & 15) of row block rb, dims 32 (lane >> 4) + 8 st + [0, 8)
  const int h = lane >> 4, col = lane & 15;
  u32x4 qf[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = rb * 16 + col;
    if (r < x.ntok) {
      const u32x4* q = (const u32x4*)((const uint16_t*)p.q + ((x.t0 + r) * p.Hkv + g) * (int64_t)kD + 32 * h);
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[rb][st] = q[st];
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[rb][st] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // positions as int32 (below L < 2^31; -1 stands for "sees nothing")
  int posr[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) posr[rb] = (int)max(x.pos(rb * 16 + col), (int64_t)-1);
  const int pos_lo = (int)max(x.pos(0), (int64_t)-1);  // the tile's first row sees the fewest keys
  const int32_t* bt = p.bt + (int64_t)x.s * p.MP;
  // physical pages of block b's two 64-token halves (the same page when P
  // is 128); wave-uniform, -1 where the half holds no token below L
  auto pages_of = [&](int b, int& pa, int& pb) {
    const int j0 = 128 * b;
    pa = j0 < L ? bt[j0 / p.P] : -1;
    pb = p.P == 64 ? (j0 + 64 < L ? bt[(j0 + 64) / p.P] : -1) : pa;
  };
  // group kg of block b: keys 128 b + 16 kg + [0, 16); a lane reads key
  // (lane & 15), dims 32 (lane >> 4) + [0, 32)
  // Every fetch loads: a half without a page (beyond L) or with a page id
  // outside the cache reads page 0 instead (num_pages >= 1 here), and the
  // mask removes keys at or beyond L, so no branch zeroes registers.
  auto fetch = [&](KeyRow<QT, KT>& kr, int b, int kg, int pa, int pb) {
    int page = kg >= 4 ? pb : pa;
    page = (page >= 0 && page < p.num_pages) ? page : 0;
    const int64_t row = ((int64_t)page * p.Hkv + g) * p.P + ((16 * kg + col) & (p.P - 1));
    kr.load((const uint8_t*)p.k + row * KeyBytes<KT>::kRow, h);
  };
  const int first = b0 + wave;
  const int nblk_w = b1 > first ? (b1 - first + NW - 1) / NW : 0;
  // a ring of four key groups, two in flight ahead of the one in use; with
  // the group loop unrolled by 8 every slot index is a constant
  KeyRow<QT, KT> kr[4];
  int pa = -1, pb = -1, na = -1, nb2 = -1;
  if (nblk_w > 0) {
    pages_of(first, pa, pb);
    fetch(kr[0], first, 0, pa, pb);
    fetch(kr[1], first, 1, pa, pb);
  }
  for (int bi = 0, b = first; bi < nblk_w; ++bi, b += NW) {
    const bool has_next = bi + 1 < nblk_w;
    if (has_next) pages_of(b + NW, na, nb2);
    // a block every key of which every row of the tile sees needs no mask
    const bool full = 128 * b + 127 < L && 128 * b + 127 <= pos_lo;
    float m[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) m[rb] = -INFINITY;
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      if (kg < 6)
        fetch(kr[(kg + 2) & 3], b, kg + 2, pa, pb);
      else if (has_next)
        fetch(kr[(kg + 2) & 3], b + NW, kg - 6, na, nb2);
      const int jbase = 128 * b + 16 * kg + 4 * h;  // keys of this lane's accumulator rows
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = Mma<QT>::run(kr[kg & 3].frag(st), qf[rb][st], acc);
        float v;
        if (full) {
          v = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
        } else {
          v = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = jbase + i;
            v = fmaxf(v, (j < L && j <= posr[rb]) ? acc[i] : -INFINITY);
          }
        }
        m[rb] = fmaxf(m[rb], v);  // this lane's keys; the lane groups are combined once per block
      }
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mb = max_over_groups(m[rb]);
      if (h == 0 && rb * 16 + col < x.ntok) dst[(rb * 16 + col) * row_stride + b] = mb;
    }
    pa = na;
    pb = nb2;
  }
}

// One 16-byte direct-to-LDS buffer load per lane with the non-temporal hint
// (lane i's bytes land at LDS byte address lds + 16 i): key rows that are
// read once, each load instruction covering whole 128-byte lines.
__device__ __forceinline__ void dma16_nt(i32x4v rsrc, uint32_t lds, int voff) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"{m0}"(a), "v"(voff), "s"(rsrc) : "memory");
}

// score_blocks with the key groups staged through LDS: each wave streams its
// blocks' groups of 16 key rows into a ring of four LDS slots of its own
// (two groups in flight ahead of the one in use) by direct-to-LDS loads that
// cover whole lines (one instruction: 64 / kPc complete rows, their pieces
// swizzled as in k_select_tiles), then reads them in the MFMA layout. Rows
// are read once a call: the loads carry the non-temporal hint, which the
// register-loading score_blocks cannot use (there two loads share each
// line). Page lookups are scalar loads, so no compiler-tracked load waits
// behind the ring's loads.
template <typename QT, typename KT, int NRB, int NW>
__device__ __forceinline__ void score_blocks_staged(const SelectParams& p, const SelTile& x, int b0, int b1,
                                                    float* dst, int64_t row_stride, u32x4* ring) {
  constexpr int kPc = KeyBytes<KT>::kRow / 16;  // 16-byte pieces per key row
  constexpr int kGrpU4 = 16 * kPc;              // pieces per group of 16 rows
  constexpr int kLd = kGrpU4 / 64;              // load instructions per group
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = x.g, L = x.L;
  const int h = lane >> 4, col = lane & 15;
  u32x4 qf[NRB][4];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = rb * 16 + col;
    if (r < x.ntok) {
      const u32x4* q = (const u32x4*)((const uint16_t*)p.q + ((x.t0 + r) * p.Hkv + g) * (int64_t)kD + 32 * h);
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[rb][st] = q[st];
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[rb][st] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  int posr[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) posr[rb] = (int)max(x.pos(rb * 16 + col), (int64_t)-1);
  const int pos_lo = (int)max(x.pos(0), (int64_t)-1);
  const int32_t* bt = p.bt + (int64_t)x.s * p.MP;
  auto swz = [&](int row) { return kPc == 16 ? (row & 15) : ((row >> 1) & 7); };
  // group kg of block b into ring slot sl: LDS piece i of the slot holds row
  // i / kPc of the group, its piece (i % kPc) ^ swz(row). A half without a
  // page (beyond L) or with a page id outside the cache reads page 0
  // (num_pages >= 1 here); the mask removes keys at or beyond L.
  auto issue = [&](int b, int kg, int sl) {
    const int j0 = 128 * b + (kg >= 4 ? 64 : 0);
    int pg = j0 < L ? sload32(bt + j0 / p.P) : -1;
    pg = (pg >= 0 && pg < p.num_pages) ? pg : 0;
    const int rowb = KeyBytes<KT>::kRow;
    const i32x4v rs = make_rsrc((const uint8_t*)p.k + ((int64_t)pg * p.Hkv + g) * p.P * rowb, p.P * rowb);
    const uint32_t base = lds_addr(ring + kGrpU4 * sl);
    const int row0 = (16 * kg) & (p.P - 1);  // the group's first row within its page
#pragma unroll
    for (int j = 0; j < kLd; ++j) {
      const int i = 64 * j + lane, r = i / kPc, pc = i % kPc;
      dma16_nt(rs, base + 1024 * j, (row0 + r) * rowb + 16 * (pc ^ swz(r)));
    }
  };
  const int first = b0 + wave;
  const int nblk_w = b1 > first ? (b1 - first + NW - 1) / NW : 0;
  if (nblk_w == 0) return;
  issue(first, 0, 0);
  issue(first, 1, 1);
  for (int bi = 0, b = first; bi < nblk_w; ++bi, b += NW) {
    const bool has_next = bi + 1 < nblk_w;
    const bool full = 128 * b + 127 < L && 128 * b + 127 <= pos_lo;
    float m[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) m[rb] = -INFINITY;
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      const int gi = 8 * bi + kg;  // this group's number in the wave's stream
      // the group two ahead (this block's, or the next block's first two)
      if (kg < 6) {
        issue(b, kg + 2, (gi + 2) & 3);
        wait_vmcnt<2 * kLd>();  // group gi has landed (gi + 1 and gi + 2 may be in flight)
      } else if (has_next) {
        issue(b + NW, kg - 6, (gi + 2) & 3);
        wait_vmcnt<2 * kLd>();
      } else if (kg == 6) {
        wait_vmcnt<kLd>();  // the last two groups: gi + 1 may be in flight
      } else {
        wait_vmcnt<0>();
      }
      asm volatile("" ::: "memory");  // the slot's reads below follow the wait
      KeyRow<QT, KT> kr;
      kr.load_lds(ring + kGrpU4 * (gi & 3), col, swz(col), h);
      const int jbase = 128 * b + 16 * kg + 4 * h;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = Mma<QT>::run(kr.frag(st), qf[rb][st], acc);
        float v;
        if (full) {
          v = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
        } else {
          v = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = jbase + i;
            v = fmaxf(v, (j < L && j <= posr[rb]) ? acc[i] : -INFINITY);
          }
        }
        m[rb] = fmaxf(m[rb], v);
      }
      // every lane's reads of this slot are done before a later issue
      // overwrites it (two groups on)
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mb = max_over_groups(m[rb]);
      if (h == 0 && rb * 16 + col < x.ntok) dst[(rb * 16 + col) * row_stride + b] = mb;
    }
  }
}

// The list of one (token t, KV head g) row whose token sits at position pos
// and sees blocks [0, nr), from its scores row[0, nr) (LDS or global). One
// wave. Also writes the row to p.scores when requested (unless the row is
// already there: in_place).
template <int NPL>
__device__ __forceinline__ void topk_row(const SelectParams& p, int64_t t, int g, int64_t pos, int nr,
                                         const float* row, bool in_place) {
  const int lane = threadIdx.x & 63;
  int32_t* out = p.selected + (t * p.Hkv + g) * (int64_t)p.topk;
  float* srow = p.scores ? p.scores + (t * p.Hkv + g) * (int64_t)p.nb_cap : nullptr;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int b = lane + 64 * i;
    float x = b < nr ? row[b] : -INFINITY;
    if (srow && b < p.nb_cap && !(in_place && b < nr)) srow[b] = x;
    v[i] = (x != x) ? -INFINITY : x;  // a NaN score is never selected
  }
  int k = 0;
  if (p.force_local && nr > 0 && p.topk > 0) {
    const int lb = (int)(pos / 128);  // the token's own block (the last one when not causal)
    float own = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i == lb) own = v[i];
    if (__shfl(own, lb & 63, 64) > -INFINITY) {  // it holds the token itself: only a NaN score fails
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (lane + 64 * i == lb) v[i] = -INFINITY;
      if (lane == 0) out[0] = lb;
      k = 1;
    }
  }
  if constexpr (NPL == 1) {
    // At most 64 blocks, one per lane: the wave's (value, block) pairs are
    // sorted by a bitonic network (value descending, equal values by
    // ascending block; values map to order-preserving integers, blocks that
    // cannot be chosen to 0, below every valid one), all on the vector ALU
    // with cross-lane shuffles. Lane i then holds the i-th best block.
    const float x0 = v[0] == 0.f ? 0.f : v[0];  // -0 and +0 are one value
    const uint32_t bits = __float_as_uint(x0);
    const bool valid = x0 > -INFINITY;
    uint32_t key = valid ? ((bits & 0x80000000u) ? ~bits : (bits | 0x80000000u)) : 0u;
    int blk = lane;
    const int need = min(__popcll(__ballot(valid)), p.topk - k);
#pragma unroll
    for (int w = 2; w <= 64; w <<= 1) {
#pragma unroll
      for (int j = w >> 1; j > 0; j >>= 1) {
        const uint32_t pk = (uint32_t)__shfl_xor((int)key, j, 64);
        const int pb = __shfl_xor(blk, j, 64);
        const bool p_better = pk > key || (pk == key && pb < blk);
        // the lower lane of a pair keeps the better of the two where the
        // w-run is ordered best-first, the worse one elsewhere
        const bool keep_better = ((lane & j) == 0) == ((lane & w) == 0);
        if (keep_better == p_better) {
          key = pk;
          blk = pb;
        }
      }
    }
    if (lane < need) out[k + lane] = blk;
    k += max(need, 0);
  } else {
    // each lane keeps its own best (value, block); a round reduces them over
    // the wave and only the winning lane rescans its registers
    auto lane_best = [&](float& bv, int& bb) {
      bv = -INFINITY;
      bb = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (sel_better(v[i], lane + 64 * i, bv, bb)) {
          bv = v[i];
          bb = lane + 64 * i;
        }
    };
    float lv;
    int lbk;
    lane_best(lv, lbk);
    for (; k < p.topk; ++k) {
      float bv = lv;
      int bb = lbk;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int ob = __shfl_xor(bb, off, 64);
        if (sel_better(ov, ob, bv, bb)) {
          bv = ov;
          bb = ob;
        }
      }
      if (bv == -INFINITY) break;  // every lane agrees: nothing left to select
      if (lane == 0) out[k] = bb;
      if ((bb & 63) == lane) {
#pragma unroll
        for (int i = 0; i < NPL; ++i)
          if (lane + 64 * i == bb) v[i] = -INFINITY;
        lane_best(lv, lbk);
      }
    }
  }
  for (int i = k + lane; i < p.topk; i += 64) out[i] = -1;
}

// Tiled path (prefill-shaped batches), first pass: one workgroup of 4 waves
// per (256-token tile of one sequence, KV head, slice of kSelTileBlocks
// blocks). The slice's blocks pass through two LDS slots by direct-to-LDS
// loads (the next block lands while the current one is multiplied), and each
// wave multiplies every block against its own 64 query rows (four 16-row
// blocks, S^T = K Q^T with 16x16x32 MFMA as in score_blocks), so a key row
// is read from L2 once per 256 queries. A row's block scores stay in
// registers until the slice is done and then go to the table sc [Tq, Hkv,
// nb_cap]; k_select_lists lists the rows.
constexpr int kSelTileTokens = 256;
constexpr int kSelTileBlocks = 8;

template <typename QT, typename KT>
__global__ __launch_bounds__(256, 2) void k_select_tiles(SelectParams p, float* sc, int nsplit) {
  constexpr int kPc = KeyBytes<KT>::kRow / 16;  // 16-byte pieces per key row: 16 (16-bit) or 8 (e4m3fn)
  constexpr int kBlkU4 = 128 * kPc;             // pieces per block
  __shared__ u32x4 s_key[2][kBlkU4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 4, col = lane & 15;
  const int g = (int)(blockIdx.x % (unsigned)p.Hkv);
  const int rest = (int)(blockIdx.x / (unsigned)p.Hkv);
  const int split = rest % nsplit;
  const int tile = (int)(gridDim.x / (unsigned)(p.Hkv * nsplit)) - 1 - rest / nsplit;
  SelTile x;
  if (!sel_tile(p, tile, g, kSelTileTokens, &x)) return;
  const int b0 = split * kSelTileBlocks;
  const int nb = min(kSelTileBlocks, x.nscan - b0);  // blocks of this slice
  if (nb <= 0) return;
  const int L = x.L;
  // the wave's query rows 64 wave + 16 rb + col as MFMA B operands (dims
  // 32 h + 8 st + [0, 8)), and their positions
  u32x4 qf[4][4];
  int posr[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int r = 64 * wave + 16 * rb + col;
    if (r < x.ntok) {
      const u32x4* q = (const u32x4*)((const uint16_t*)p.q + ((x.t0 + r) * p.Hkv + g) * (int64_t)kD + 32 * h);
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[rb][st] = q[st];
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) qf[rb][st] = u32x4{0u, 0u, 0u, 0u};
    }
    posr[rb] = (int)max(x.pos(r), (int64_t)-1);
  }
  const int pos_lo = (int)max(x.pos(64 * wave), (int64_t)-1);  // the wave's first row sees the fewest keys
  const int32_t* bt = p.bt + (int64_t)x.s * p.MP;
  // Block b into slot sl. LDS piece i of the slot holds key row i / kPc, its
  // 16-byte piece (i % kPc) ^ swz(row): sixteen lanes reading one piece of
  // sixteen consecutive rows then hit distinct banks. A half without a page
  // (beyond L) or with a page id outside the cache reads page 0 (num_pages
  // >= 1 here); the mask removes keys at or beyond L.
  auto swz = [&](int row) { return kPc == 16 ? (row & 15) : ((row >> 1) & 7); };
  auto issue_block = [&](int b, int sl) {
    const int j0 = 128 * b;
    int pa = j0 < L ? sload32(bt + j0 / p.P) : -1;
    int pb = p.P == 64 ? (j0 + 64 < L ? sload32(bt + (j0 + 64) / p.P) : -1) : pa;
    pa = (pa >= 0 && pa < p.num_pages) ? pa : 0;
    pb = (pb >= 0 && pb < p.num_pages) ? pb : 0;
    const int rowb = KeyBytes<KT>::kRow, nrec = p.P * rowb;  // one page of one KV head
    const i32x4v ra = make_rsrc((const uint8_t*)p.k + ((int64_t)pa * p.Hkv + g) * p.P * rowb, nrec);
    const i32x4v rh = make_rsrc((const uint8_t*)p.k + ((int64_t)pb * p.Hkv + g) * p.P * rowb, nrec);
    const uint32_t base = lds_addr(s_key[sl]);
#pragma unroll
    for (int j = 0; j < kBlkU4 / 256; ++j) {
      const int i = 256 * j + tid, row = i / kPc, pc = i % kPc;
      // this load's rows (256 / kPc of them) lie in one 64-row half
      const bool upper = p.P == 64 && j * (256 / kPc) >= 64;
      const int rip = p.P == 64 ? (row & 63) : row;  // row within its page (j0 is a multiple of 128)
      dma16(upper ? rh : ra, base + 4096 * j + 1024 * wave, rip * rowb + 16 * (pc ^ swz(row)));
    }
  };
  float mreg[kSelTileBlocks][4];
  issue_block(b0, 0);
#pragma unroll
  for (int i = 0; i < kSelTileBlocks; ++i) {
    if (i >= nb) break;
    const int b = b0 + i;
    wait_vmcnt<0>();  // block b has landed (this wave's part) ...
    __syncthreads();  // ... every wave's part; and every wave is done with block b - 1
    if (i + 1 < nb) issue_block(b + 1, (i + 1) & 1);
    const u32x4* blk = s_key[i & 1];
    // a block every key of which every row of the wave sees needs no mask
    const bool full = 128 * b + 127 < L && 128 * b + 127 <= pos_lo;
    float m[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) m[rb] = -INFINITY;
    KeyRow<QT, KT> kr[2];
    kr[0].load_lds(blk, col, swz(col), h);
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      if (kg + 1 < 8) {
        const int rn = 16 * (kg + 1) + col;
        kr[(kg + 1) & 1].load_lds(blk, rn, swz(rn), h);
      }
      f32x4 acc[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[rb] = Mma<QT>::run(kr[kg & 1].frag(st), qf[rb][st], acc[rb]);
      const int jbase = 128 * b + 16 * kg + 4 * h;  // keys of this lane's accumulator rows
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        float v;
        if (full) {
          v = fmaxf(fmaxf(acc[rb][0], acc[rb][1]), fmaxf(acc[rb][2], acc[rb][3]));
        } else {
          v = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = jbase + e;
            v = fmaxf(v, (j < L && j <= posr[rb]) ? acc[rb][e] : -INFINITY);
          }
        }
        m[rb] = fmaxf(m[rb], v);
      }
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) mreg[i][rb] = max_over_groups(m[rb]);
  }
  // the slice's scores of the wave's rows (lanes of group 0 hold them)
  if (h == 0) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 64 * wave + 16 * rb + col;
      if (r >= x.ntok) continue;
      float* dst = sc + ((x.t0 + r) * p.Hkv + g) * (int64_t)p.nb_cap + b0;
#pragma unroll
      for (int i = 0; i < kSelTileBlocks; ++i)
        if (i < nb) dst[i] = mreg[i][rb];
    }
  }
}

// Split path (decode-shaped batches), first pass: one workgroup per (16-token
// tile, KV head, slice of kSelSplitBlocks blocks) writes its blocks' scores
// to the global table sc [Tq, Hkv, nb_cap]; the slices of a long sequence run
// side by side.
template <typename QT, typename KT>
__global__ __launch_bounds__(64 * kSelSplitWaves) void k_select_scores(SelectParams p, float* sc, int nsplit) {
  const int g = (int)(blockIdx.x % (unsigned)p.Hkv);
  const int rest = (int)(blockIdx.x / (unsigned)p.Hkv);
  const int split = rest % nsplit;
  const int tile = (int)(gridDim.x / (unsigned)(p.Hkv * nsplit)) - 1 - rest / nsplit;
  SelTile x;
  if (!sel_tile(p, tile, g, 16, &x)) return;
  const int b0 = split * kSelSplitBlocks, b1 = min(b0 + kSelSplitBlocks, x.nscan);
  if (b0 >= b1) return;
  float* dst = sc + (x.t0 * p.Hkv + g) * (int64_t)p.nb_cap;
  if constexpr (sizeof(KT) == 1) {
    // e4m3fn keys through LDS (8 KB a wave); 16-bit keys would need twice
    // that and halve the waves a CU holds, so they load straight to registers
    __shared__ u32x4 s_ring[kSelSplitWaves][4 * 16 * (KeyBytes<KT>::kRow / 16)];
    score_blocks_staged<QT, KT, 1, kSelSplitWaves>(p, x, b0, b1, dst, (int64_t)p.Hkv * p.nb_cap,
                                                   s_ring[threadIdx.x >> 6]);
  } else {
    score_blocks<QT, KT, 1, kSelSplitWaves>(p, x, b0, b1, dst, (int64_t)p.Hkv * p.nb_cap);
  }
}

// Split path, second pass: one wave per (token, KV head) row lists it from
// the global table.
template <int NPL>
__global__ __launch_bounds__(256) void k_select_lists(SelectParams p, const float* sc) {
  const int64_t rid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * Hkv + g
  if (rid >= (int64_t)p.Tq * p.Hkv) return;
  const int64_t t = rid / p.Hkv;
  const int g = (int)(rid - t * p.Hkv);
  const int s = wave_seq_of(p.cu, p.B, t);
  int nr = 0;
  int64_t pos = -1;
  if (s >= 0) {
    const int L = p.num_pages > 0 ? min(p.used[s], p.MP * p.P) : 0;
    const int64_t c0 = p.cu[s], tq_s = p.cu[s + 1] - c0;
    pos = p.causal ? (int64_t)L - tq_s + (t - c0) : (int64_t)L - 1;
    const int nb = min((L + 127) / 128, p.nb_cap);
    nr = (L <= 0 || pos < 0) ? 0 : (int)min((int64_t)nb, pos / 128 + 1);
  }
  topk_row<NPL>(p, t, g, pos, nr, sc + rid * p.nb_cap, sc == p.scores);
}

static hipError_t launch_lists(const ProfSpan& sp, const SelectParams& p, const float* sc, hipStream_t st) {
  const dim3 grid((unsigned)(((int64_t)p.Tq * p.Hkv + 3) / 4)), block(256);
  if (p.nb_cap <= 64) return launch_k(sp, false, true, k_select_lists<1>, grid, block, 0, st, p, sc);
  if (p.nb_cap <= 128) return launch_k(sp, false, true, k_select_lists<2>, grid, block, 0, st, p, sc);
  if (p.nb_cap <= 256) return launch_k(sp, false, true, k_select_lists<4>, grid, block, 0, st, p, sc);
  if (p.nb_cap <= 512) return launch_k(sp, false, true, k_select_lists<8>, grid, block, 0, st, p, sc);
  if (p.nb_cap <= 1024) return launch_k(sp, false, true, k_select_lists<16>, grid, block, 0, st, p, sc);
  return launch_k(sp, false, true, k_select_lists<kSelMaxBlocks / 64>, grid, block, 0, st, p, sc);
}

template <typename QT, typename KT>
static hipError_t launch_select_t(const ProfSpan& sp, const SelectParams& p, float* table, bool tiled,
                                  hipStream_t st) {
  if (tiled) {
    // 256-token tiles sharing each block through LDS, then the lists
    const int64_t tiles = ((int64_t)p.Tq + kSelTileTokens - 1) / kSelTileTokens + p.B;
    const int nsplit = (p.nb_cap + kSelTileBlocks - 1) / kSelTileBlocks;
    hipError_t e = launch_k(sp, true, false, k_select_tiles<QT, KT>, dim3((unsigned)(tiles * p.Hkv * nsplit)),
                            dim3(256), 0, st, p, table, nsplit);
    if (e == hipSuccess) e = launch_lists(sp, p, table, st);
    return e;
  }
  const int64_t tiles = ((int64_t)p.Tq + 15) / 16 + p.B;
  const int nsplit = (p.nb_cap + kSelSplitBlocks - 1) / kSelSplitBlocks;
  hipError_t e = launch_k(sp, true, false, k_select_scores<QT, KT>, dim3((unsigned)(tiles * p.Hkv * nsplit)),
                          dim3(64 * kSelSplitWaves), 0, st, p, table, nsplit);
  if (e == hipSuccess) e = launch_lists(sp, p, table, st);
  return e;
}

hipError_t launch_select(const SelectParams& p, int q_elem, bool fp8_keys, float* table, bool tiled, hipStream_t st) {
  if (p.Tq == 0 || p.Hkv == 0) return hipSuccess;
  const ProfSpan sp = profile_begin(kKSelect);
  hipError_t e;
  if (q_elem == kElemBF16)
    e = fp8_keys ? launch_select_t<bf16_t, fp8_e4m3_t>(sp, p, table, tiled, st)
                 : launch_select_t<bf16_t, bf16_t>(sp, p, table, tiled, st);
  else
    e = fp8_keys ? launch_select_t<f16_t, fp8_e4m3_t>(sp, p, table, tiled, st)
                 : launch_select_t<f16_t, f16_t>(sp, p, table, tiled, st);
  profile_end(sp, e == hipSuccess);
  return e;
}

}  // namespace msa
