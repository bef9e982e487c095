// msa_forward.hip -- the front kernel: classification of every tile, and
// the decode-shaped tiles finished in place, on gfx950 MFMA (16x16x32).
//
// fw-ai/minimax-kernels README, intro: a selected KV block is loaded once
// and every query that selected it is processed against it. Queries are cut
// into tiles of consecutive tokens of one sequence (x the G query heads of
// KV head g); a tile's CHAIN is the blocks every token of the tile selected.
// The front kernel runs one workgroup per tile leader: it finds the chain,
// flags each slot covered (its block is in the chain) or residual, sets the
// residual bits of the per-(block, KV head) token bitmaps, and either
//   finishes the tile itself (decode-shaped batches: at most 16 query rows
//   and no residual slot -- one decode token x G heads is the common case),
//   streaming the chain's blocks with the rows held in registers, or
//   lists the tile for the tile kernel (msa_tiles.hip), which also merges
//   the KV-outer partials of the residual slots.
// Each wave of the streaming path owns 16 query rows. Scores are computed
// transposed, S^T = K * Q^T, so that a lane's D fragment holds one query
// row; the probabilities are then already laid out as the B operand of
// O^T = V^T * P^T and the online-softmax rescale stays lane-local.
// Rows whose keys are masked (beyond the used length, causally invisible,
// or from another sequence) are removed by select, never by arithmetic, and
// value rows beyond the used length are zero-filled, so stale or poisoned
// cache contents cannot reach the result.
//
// fp8 (e4m3fn) caches are widened exactly to the query's 16-bit type before
// the MFMA; the sglang pull request "Speed up MiniMax-M3 sparse attention on
// Hopper", section "Summary", widens its fp8 decode operands the same way.
#include <limits.h>

#include <type_traits>

#include "msa_device.hpp"
#include "msa_index_dev.hpp"
#include "msa_internal.hpp"

namespace msa {

// marks a residual slot in the classifiers' LDS pick lists (block ids are < 2^30)
constexpr int kResidualMark = 1 << 30;

// query rows of one tile the front kernel streams when every tile is one
// token (4 row sets of 16; a token with Hq/Hkv <= 64)
constexpr int kStreamRowsMax = 64;
constexpr int kFrontBitWords = 2048;  // block masks of a classification-only workgroup (8 KB)

// element offset of k-step s (0..3, 32 dims each) for lane group q: pairs of
// k-steps share one 64-dim slab, so an fp8 lane reads 16 contiguous bytes
__device__ __forceinline__ int kmap(int s, int q) { return 64 * (s >> 1) + 16 * q + 8 * (s & 1); }

// key (0..31 within a chunk) of element e (0..7) of lane group q
__device__ __forceinline__ int key_of(int q, int e) { return (e < 4) ? (4 * q + e) : (16 + 4 * q + (e - 4)); }

template <typename CT>
struct RowTile {
  u32x4 qb[4];  // Q^T B-operand fragments for the four k-steps
  f32x4 o[8];   // O^T accumulators: d-tile t, element r -> d = 32q + 8r + t
  float m;      // running max of the lane's row (log2 units)
  float l;      // this lane's share of the row sum
  int pos;      // causal position of the row (INT_MAX when not causal)
  int seq;      // owning sequence (-1: padding row)
};

template <typename CT>
__device__ __forceinline__ void tile_reset(RowTile<CT>& rt) {
#pragma unroll
  for (int t = 0; t < 8; ++t) rt.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  rt.m = -INFINITY;
  rt.l = 0.f;
}

// Q fragments of one row (token tok, head h); zero for padding rows.
template <typename CT>
__device__ __forceinline__ void tile_load_q(RowTile<CT>& rt, const Params& p, int tok, int h, int q) {
  if (tok < 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) rt.qb[s] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const uint16_t* base = (const uint16_t*)p.q + ((size_t)tok * p.Hq + h) * kD;
#pragma unroll
  for (int s = 0; s < 4; ++s) rt.qb[s] = *(const u32x4*)(base + kmap(s, q));
}

// A row's reference maximum is only raised when a chunk's scores exceed it
// by more than this many powers of two, so the accumulators are rescaled
// rarely; the probabilities stay below 2^kRescale.
constexpr float kRescale = 8.0f;

// One 32-key chunk, split in two stages so that several row tiles can share
// one chunk's fragments: tile_probs computes the scores and the masked
// online-softmax step of one row tile and returns its probabilities as the
// B operand; tile_pv builds each V^T operand once and accumulates it into
// every row tile.
//   ka[j][s]  K fragment: key 16j + c, dims of k-step s
//   va[e]     V fragment: key key_of(q, e), dims 8c .. 8c+7
//   key0      token index of key 0 of the chunk; keys at or beyond lim are absent
//   run_seq   sequence the chunk belongs to (rows of other sequences skip it)
template <typename CT>
__device__ __forceinline__ u32x4 tile_probs(RowTile<CT>& rt, const u32x4 (&ka)[2][4], int key0, int lim,
                                            int run_seq, int q, float scale_log2) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    s0 = Mma<CT>::run(ka[0][s], rt.qb[s], s0);
    s1 = Mma<CT>::run(ka[1][s], rt.qb[s], s1);
  }
  const bool live = rt.seq == run_seq;
  float x[8];
  float cmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tok = key0 + key_of(q, e);
    const bool ok = live && tok < lim && tok <= rt.pos;
    const float sv = (e < 4) ? s0[e] : s1[e - 4];
    x[e] = ok ? sv * scale_log2 : -INFINITY;
    cmax = fmaxf(cmax, x[e]);
  }
  cmax = max_over_groups(cmax);
  if (__any(cmax > rt.m + kRescale)) {
    const float m_new = fmaxf(rt.m, cmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(rt.m - m_new);
    rt.l *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) rt.o[t] *= alpha;
    rt.m = m_new;
  }
  const float m_use = (rt.m == -INFINITY) ? 0.f : rt.m;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
    rt.l += p[e];
  }
  u32x4 pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = pack2<CT>(p[2 * i], p[2 * i + 1]);
  return pb;
}

template <typename CT, int RS>
__device__ __forceinline__ void tile_pv(RowTile<CT> (&rt)[RS], const u32x4 (&va)[8], const u32x4 (&pb)[RS]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    u32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x0 = va[2 * i][t >> 1], x1 = va[2 * i + 1][t >> 1];
      a[i] = (t & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
    }
#pragma unroll
    for (int r = 0; r < RS; ++r) rt[r].o[t] = Mma<CT>::run(a, pb[r], rt[r].o[t]);
  }
}

template <typename CT, int RS>
__device__ __forceinline__ void tile_chunk(RowTile<CT> (&rt)[RS], const u32x4 (&ka)[2][4], const u32x4 (&va)[8],
                                           int key0, int lim, int run_seq, int q, float scale_log2) {
  if constexpr (RS == 1) {
    // one row tile: each V^T operand is built right before its product
    const u32x4 pb = tile_probs<CT>(rt[0], ka, key0, lim, run_seq, q, scale_log2);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u32x4 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x0 = va[2 * i][t >> 1], x1 = va[2 * i + 1][t >> 1];
        a[i] = (t & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
      }
      rt[0].o[t] = Mma<CT>::run(a, pb, rt[0].o[t]);
    }
  } else {
    u32x4 pb[RS];
#pragma unroll
    for (int r = 0; r < RS; ++r) pb[r] = tile_probs<CT>(rt[r], ka, key0, lim, run_seq, q, scale_log2);
    tile_pv<CT, RS>(rt, va, pb);
  }
}

// Zero the V fragments of keys at or beyond lim (their probabilities are
// exactly zero, but the cache rows may hold anything, NaN included).
__device__ __forceinline__ void zero_absent_v(u32x4 (&va)[8], int key0, int lim, int q) {
  if (key0 + 32 <= lim) return;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (key0 + key_of(q, e) >= lim) va[e] = u32x4{0u, 0u, 0u, 0u};
}

template <typename KVT>
struct KvElem {
  typedef uint16_t type;
};
template <>
struct KvElem<fp8_e4m3_t> {
  typedef uint8_t type;
};
template <>
struct KvElem<mxfp4_t> {
  typedef uint8_t type;
};

// ---------------------------------------------------------------------------
// register fragments of one 32-key chunk, loaded straight from HBM. The loads
// are unconditional (absent chunks read the zero page), so the compiler can
// keep the next chunk's loads in flight while the current one is multiplied.
// They carry the non-temporal hint: each chunk is read once per call here,
// and on the MI355X streaming reads with the hint reach ~6.7 TB/s against
// ~6.1 TB/s without it (microbenchmark, 4 GB read with 16-byte loads).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T ld_stream(const void* ptr) {
  return __builtin_nontemporal_load((const T*)ptr);
}
template <typename CT, typename KVT>
struct Frag;

template <typename CT>
struct Frag<CT, CT> {  // 16-bit cache: fragments are used as loaded
  u32x4 ka[2][4];
  u32x4 va[8];
  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, const uint8_t*, const uint8_t*, int q,
                                       int c) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[j][s] = ld_stream<u32x4>(kb + (16 * j + c) * kD + kmap(s, q));
#pragma unroll
    for (int e = 0; e < 8; ++e) va[e] = ld_stream<u32x4>(vb + key_of(q, e) * kD + 8 * c);
  }
  template <int RS>
  __device__ __forceinline__ void compute(RowTile<CT> (&rt)[RS], int key0, int lim, int seq, int q, float sl2) {
    zero_absent_v(va, key0, lim, q);
    tile_chunk<CT, RS>(rt, ka, va, key0, lim, seq, q, sl2);
  }
};

template <typename CT>
struct Frag<CT, fp8_e4m3_t> {  // e4m3fn cache: raw bytes until the chunk is used
  u32x4 kr[2][2];
  u32x2 vr[8];
  __device__ __forceinline__ void load(const uint8_t* kb, const uint8_t* vb, const uint8_t*, const uint8_t*, int q,
                                       int c) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) kr[j][pp] = ld_stream<u32x4>(kb + (16 * j + c) * kD + 64 * pp + 16 * q);
#pragma unroll
    for (int e = 0; e < 8; ++e) vr[e] = ld_stream<u32x2>(vb + key_of(q, e) * kD + 8 * c);
  }
  template <int RS>
  __device__ __forceinline__ void compute(RowTile<CT> (&rt)[RS], int key0, int lim, int seq, int q, float sl2) {
    u32x4 ka[2][4], va[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        ka[j][2 * pp] = widen8<CT>(u32x2{kr[j][pp][0], kr[j][pp][1]});
        ka[j][2 * pp + 1] = widen8<CT>(u32x2{kr[j][pp][2], kr[j][pp][3]});
      }
#pragma unroll
    for (int e = 0; e < 8; ++e) va[e] = widen8<CT>(vr[e]);
    zero_absent_v(va, key0, lim, q);
    tile_chunk<CT, RS>(rt, ka, va, key0, lim, seq, q, sl2);
  }
};

// MXFP4 cache (OCP microscaling: 32 consecutive values of a row share an
// e8m0 scale; e2m1 codes two a byte, 64 bytes a row, and 4 scale bytes a
// row): raw codes and the rows' scale words until the chunk is used, then
// widened to bf16 with the scale applied. The fragments are those of the
// 16-bit cache: K row 16 j + c, dims 64 pp + 16 q .. +16 (code bytes 32 pp +
// 8 q .. +8, scale 2 pp + q / 2); V row key_of(q, e), dims 8 c .. 8 c + 8
// (code bytes 4 c .. +4, scale c / 4). The V rows of lane group q are rows
// 4 q .. 4 q + 3 and 16 + 4 q .. 16 + 4 q + 3, so their scale words come in
// two 16-byte loads.
template <typename CT>
struct Frag<CT, mxfp4_t> {
  u32x2 kc[2][2];
  uint32_t ks[2];
  uint32_t vc[8];
  u32x4 vs[2];
  __device__ __forceinline__ void load(const uint8_t* kb, const uint8_t* vb, const uint8_t* ksb, const uint8_t* vsb,
                                       int q, int c) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) kc[j][pp] = ld_stream<u32x2>(kb + (16 * j + c) * 64 + 32 * pp + 8 * q);
      ks[j] = ld_stream<uint32_t>(ksb + (16 * j + c) * 4);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vc[e] = ld_stream<uint32_t>(vb + key_of(q, e) * 64 + 4 * c);
    vs[0] = ld_stream<u32x4>(vsb + key_of(q, 0) * 4);
    vs[1] = ld_stream<u32x4>(vsb + key_of(q, 4) * 4);
  }
  template <int RS>
  __device__ __forceinline__ void compute(RowTile<CT> (&rt)[RS], int key0, int lim, int seq, int q, float sl2) {
    static_assert(sizeof(CT) == 2, "MXFP4 caches widen to bf16");
    const int c = threadIdx.x & 15;
    u32x4 ka[2][4], va[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const float sc = e8m0_scale((ks[j] >> (8 * (2 * pp + (q >> 1)))) & 0xFFu);
        ka[j][2 * pp] = widen_fp4(kc[j][pp][0], sc);
        ka[j][2 * pp + 1] = widen_fp4(kc[j][pp][1], sc);
      }
#pragma unroll
    for (int e = 0; e < 8; ++e) va[e] = widen_fp4(vc[e], e8m0_scale((vs[e >> 2][e & 3] >> (8 * (c >> 2))) & 0xFFu));
    zero_absent_v(va, key0, lim, q);
    tile_chunk<CT, RS>(rt, ka, va, key0, lim, seq, q, sl2);
  }
};

// Streams the chain of a residual-free tile and writes its final O and LSE
// (see k_front). The tile's rows are cut into row sets of 16 (1, 2 or 4 for
// tiles of up to 16, 32 or 64 rows); each wave holds RS row sets, which
// share every K/V fragment the wave loads. The nrs / RS wave groups each
// take their row sets, and the waves of a group split the chain's chunks
// (wave w: group w % ngrp, every (4 / ngrp)-th chunk from w / ngrp). Waves
// holding the same rows are merged through LDS. RS = 2 serves one decode
// token with 17 .. 64 query rows, so that four waves stream four distinct
// chunk sequences. An empty chain writes zeros and an LSE of -inf.
template <typename CT, typename KVT, int RS>
__device__ __forceinline__ void stream_chain(const Params& p, int t, int g, int s, int L, int Tq_s,
                                             int64_t q0, int rows, int n_ch, int ppb,
                                             const int* s_chain, const int* s_chain_k,
                                             const int* s_page) {
  typedef typename KvElem<KVT>::type E;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Hkv = p.Hkv;
  __shared__ int64_t s_koff[256];  // element offset of each chunk; -1: absent
  __shared__ float s_o[4][16 * RS][kD + 4];
  __shared__ float s_m[4][16 * RS];
  __shared__ float s_l[4][16 * RS];
  const int Leff = min(L, p.MP * p.P);  // keys the page table can reach
  const int nchunks = n_ch * 4;
  for (int ci = tid; ci < nchunks; ci += 256) {
    const int c = ci >> 2, part = ci & 3;
    const int key0 = kBlk * s_chain[c] + 32 * part;
    const int page = s_page[s_chain_k[c] * ppb + (32 * part) / p.P];
    s_koff[ci] = (key0 < Leff && page >= 0 && page < p.NP)
                     ? (((int64_t)page * Hkv + g) * p.P + (key0 % p.P)) * kD
                     : (int64_t)-1;
  }
  const int nrs = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);  // row sets of 16 rows
  const int ngrp = max(1, nrs / RS);                      // wave groups, RS row sets each
  const int nph = 4 / ngrp;                               // chunk phases per group
  const int grp = wave % ngrp, ph = wave / ngrp;
  const int q = lane >> 4, c = lane & 15;
  RowTile<CT> rt[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int row = 16 * (grp * RS + r) + c;  // the lane's row in the tile
    tile_reset(rt[r]);
    int tok = -1, h = 0;
    rt[r].seq = -1;
    rt[r].pos = -1;
    if (row < rows) {
      tok = t + row / p.G;
      h = g * p.G + (row % p.G);
      rt[r].seq = s;
      rt[r].pos = p.causal ? (int)(L - Tq_s + (tok - q0)) : INT_MAX;
    }
    tile_load_q(rt[r], p, tok, h, q);
  }
  __syncthreads();

  const E* kbase = (const E*)p.k;
  const E* vbase = (const E*)p.v;
  const E* zero = (const E*)p.zero_page;
  // element offsets to byte offsets: MXFP4 codes are half a byte a value,
  // their scales one byte per 32 values
  constexpr int kCodeShift = std::is_same<KVT, mxfp4_t>::value ? 1 : 0;
  auto kaddr = [&](int ci) -> const E* {
    const int64_t off = ci < nchunks ? s_koff[ci] : (int64_t)-1;
    return off >= 0 ? kbase + (off >> kCodeShift) : zero;
  };
  auto vaddr = [&](int ci) -> const E* {
    const int64_t off = ci < nchunks ? s_koff[ci] : (int64_t)-1;
    return off >= 0 ? vbase + (off >> kCodeShift) : zero;
  };
  auto saddr = [&](const uint8_t* base, int ci) -> const uint8_t* {
    if constexpr (!kCodeShift) return nullptr;  // no scales
    const int64_t off = ci < nchunks ? s_koff[ci] : (int64_t)-1;
    return off >= 0 ? base + (off >> 5) : (const uint8_t*)p.zero_page;
  };
  auto key0_of = [&](int ci) { return s_koff[ci] >= 0 ? kBlk * s_chain[ci >> 2] + 32 * (ci & 3) : Leff; };
  const int nmine = (nchunks - ph + nph - 1) / nph;
  if (nmine > 0) {
    Frag<CT, KVT> fa, fb;
    int ci = ph;
    fa.load(kaddr(ci), vaddr(ci), saddr(p.k_scale, ci), saddr(p.v_scale, ci), q, c);
    for (;;) {
      fb.load(kaddr(ci + nph), vaddr(ci + nph), saddr(p.k_scale, ci + nph), saddr(p.v_scale, ci + nph), q, c);
      fa.compute(rt, key0_of(ci), Leff, s, q, p.scale_log2);
      ci += nph;
      if (ci >= nchunks) break;
      fa.load(kaddr(ci + nph), vaddr(ci + nph), saddr(p.k_scale, ci + nph), saddr(p.v_scale, ci + nph), q, c);
      fb.compute(rt, key0_of(ci), Leff, s, q, p.scale_log2);
      ci += nph;
      if (ci >= nchunks) break;
    }
  }

  // merge the waves holding each row
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const float l_row = sum_over_groups(rt[r].l);
    if (q == 0) {
      s_m[wave][16 * r + c] = rt[r].m;
      s_l[wave][16 * r + c] = l_row;
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][16 * r + c][32 * q + 8 * i + tt] = rt[r].o[tt][i];
  }
  __syncthreads();
  for (int it = tid; it < 16 * nrs * 16; it += 256) {
    const int orow = it >> 4, d0 = (it & 15) * 8;  // output row in the tile, its 8 dims
    if (orow >= rows) break;
    const int rset = orow >> 4, rc = orow & 15;
    const int og = rset / RS, lr = 16 * (rset % RS) + rc;  // the row's wave group, its row in those waves
    float M = -INFINITY;
    for (int w = og; w < 4; w += ngrp) M = fmaxf(M, s_m[w][lr]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float wsum = 0.f, acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.f;
    for (int w = og; w < 4; w += ngrp) {
      const float f = exp2f(s_m[w][lr] - Mu);
      wsum += f * s_l[w][lr];
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] += f * s_o[w][lr][d0 + d];
    }
    const int rtok = t + orow / p.G;
    const int rh = g * p.G + (orow % p.G);
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const float lse2 = wsum > 0.f ? Mu + log2f(wsum) : -INFINITY;
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pack2<CT>(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *(u32x4*)((uint16_t*)p.out + ((size_t)rtok * p.Hq + rh) * kD + d0) = pk;
    if (d0 == 0 && p.lse) p.lse[(size_t)rh * p.Tq + rtok] = lse2 * kLn2;
  }
}

// ---------------------------------------------------------------------------
// front kernel: one workgroup per (token t, KV head g) in decode mode, per
// tile otherwise; only tile leaders do work. It classifies the tile's slots
// (chain, covered/residual flags, residual bitmap bits) and, in decode mode,
// when the tile has at most 16 query rows and no residual slot, streams the
// chain's blocks right away: the chain's chunks are split over the four
// waves, each keeping two chunks of K/V in flight in registers, and the
// waves' softmax states are merged through LDS. The chunk addresses are
// resolved once, up front, so no page lookup sits between consecutive loads.
// Every other tile is appended to the tile list. Tokens outside every
// sequence (decode mode) get zero outputs and an LSE of -inf here.
// ---------------------------------------------------------------------------
// A thread's slot of a tile walked in rounds of S slots: idx = tau * K + k,
// moved on by S slots per round without a division (S mod K < K, so one
// carry step suffices).
template <int S>
struct SlotWalk {
  int idx, tau, k;
  int dq, dr;  // S = dq * K + dr
  __device__ __forceinline__ SlotWalk(int first, int K) : idx(first), tau(first / K), k(first - (first / K) * K) {
    dq = S / K;
    dr = S - dq * K;
  }
  __device__ __forceinline__ void next(int K) {
    idx += S;
    tau += dq;
    k += dr;
    if (k >= K) {
      k -= K;
      ++tau;
    }
  }
};

template <typename CT, typename KVT, bool ATTN, int RS>
__global__ __launch_bounds__(256, RS == 1 ? 2 : 1) void k_front(Params p) {
  extern __shared__ int s_sel[];  // [nt][K] picks, -1 where the slot is invalid
  __shared__ int s_chain[64];     // chain blocks
  __shared__ int s_chain_k[64];   // leader slot of each chain block
  __shared__ int s_nres[128];     // residual slots per tile token
  __shared__ int s_page[128];     // pages of the leader's picks (ppb per pick)
  __shared__ int s_nch;
  __shared__ int s_tile_res;      // residual slots of the tile
  __shared__ int s_item_idx;      // the tile kernel's item for this tile (-1: none)
  __shared__ int s_miss[64];      // leader picks missing from some token of the tile
  const int g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = p.K, Hkv = p.Hkv;
  const int Teff = p.T > 0 ? p.T : 1;
  // the last kernel of a call leaves the next call's counter set zeroed (it
  // was used by the previous call, whose kernels have all finished)
  if (p.front_only && blockIdx.x == 0 && blockIdx.y == 0 && p.counters_next && tid < kCntSlots)
    p.counters_next[tid] = 0;
  int t, s;
  int b_raw = -1;
  if (p.stream_narrow) {
    // one workgroup per token; the leader's picks do not depend on the
    // sequence, so their loads are issued before the search
    t = blockIdx.x;
    if (tid < K) b_raw = p.selected[((size_t)t * Hkv + g) * K + tid];
    // a batch of one-token sequences has token t in sequence t: try that
    // first (one round of loads, issued with the picks), search otherwise
    const int sg = min(t, p.B - 1);
    const bool hit = p.B > 0 && p.cu[sg] <= t && t < p.cu[sg + 1];
    s = hit ? sg : wave_seq_of(p.cu, p.B, t);
    if (s < 0) {  // outside every sequence: no keys
      const size_t tg = (size_t)t * Hkv + g;
      if (tid < K) p.slot_flag[tg * K + tid] = 0;
      if (tid == 0) {
        p.tok_chain[tg] = 0;
        p.tok_nres[tg] = 0;
      }
      if constexpr (ATTN) {
        for (int i = tid; i < p.G * 16; i += 256) {
          const int hh = g * p.G + (i >> 4);
          *(u32x4*)((uint16_t*)p.out + ((size_t)t * p.Hq + hh) * kD + 8 * (i & 15)) = u32x4{0u, 0u, 0u, 0u};
          if ((i & 15) == 0 && p.lse) p.lse[(size_t)hh * p.Tq + t] = -INFINITY;
        }
      }
      return;
    }
    if ((t - p.cu[s]) % Teff != 0) return;  // the tile's leader handles this token
  } else {
    // one workgroup per tile
    int64_t t0;
    s = wave_tile_of(p.cu, p.B, p.Tq, Teff, blockIdx.x, &t0);
    if (s < 0) {  // no tile: the tile kernel's item (g, blockIdx.x) has nothing to do
      if (p.tdesc && tid == 0) p.tdesc[2 * ((size_t)g * gridDim.x + blockIdx.x)] = int4{0, 0, 0, 0};
      return;
    }
    t = (int)t0;
    if (tid < K) b_raw = p.selected[((size_t)t * Hkv + g) * K + tid];
  }
  const size_t tg = (size_t)t * Hkv + g;
  const int64_t q0 = p.cu[s], qe = p.cu[s + 1];
  const int64_t q1 = min(qe, (int64_t)p.Tq);
  const int i0 = (int)(t - q0);
  const int nt = (int)min((int64_t)Teff, q1 - t);
  const int rows = nt * p.G;
  // a decode-mode tile of at most 16 rows (of at most 64 when every tile is
  // one token: front-only calls) is streamed here unless it turns out to
  // have residual slots
  const int stream_rows = p.front_only ? kStreamRowsMax : 16;
  const bool stream = ATTN && p.stream_narrow && rows <= stream_rows;
  const int ppb = kBlk / p.P;  // pages per block

  // pages of the leader's picks, looked up while the sequence length loads
  int my_page = -1;
  if (stream && K * ppb <= 64) {
    // picks are already in lanes 0..K-1 of wave 0 (b_raw)
    const int k = lane / ppb, j = lane - (lane / ppb) * ppb;
    const int b = __shfl(b_raw, k, 64);
    const int lp = b * ppb + j;
    if (wave == 0 && lane < K * ppb && b >= 0 && b < p.nb_max && lp < p.MP)
      my_page = p.block_tables[(size_t)s * p.MP + lp];
  } else if (stream && tid < K * ppb) {
    const int k = tid / ppb, j = tid - (tid / ppb) * ppb;
    const int b = p.selected[tg * K + k];
    const int lp = b * ppb + j;
    if (b >= 0 && b < p.nb_max && lp < p.MP) my_page = p.block_tables[(size_t)s * p.MP + lp];
  }
  const int L = p.used[s];
  const int Tq_s = (int)(qe - q0);
  const int nblk = L > 0 ? min((L + kBlk - 1) / kBlk, p.nb_max) : 0;

  // Classification-only launches test set membership through bit masks of
  // the blocks when they fit (one bit test instead of a scan of the top-k):
  // token tau's picks at bits[tau * wb], the chain's at bits[nt * wb]
  uint32_t* bits = nullptr;
  const int wb = (nblk + 31) >> 5;
  bool use_bits = false;
  if constexpr (!ATTN) {
    __shared__ uint32_t s_fbits[kFrontBitWords];
    bits = s_fbits;
    use_bits = p.T > 0 && (nt + 1) * wb <= kFrontBitWords;
    if (use_bits) {
      for (int i = tid; i < (nt + 1) * wb; i += 256) bits[i] = 0u;
      __syncthreads();
    }
  }
  // The slot loops below walk the tile's slots without divisions in
  // classification-only launches (many slots a tile); launches that also
  // stream (a few slots a tile) keep the plain index arithmetic, which needs
  // fewer registers.
  auto load_pick = [&](int idx, int tau, int k) {
    const int b = (idx < K) ? b_raw : p.selected[((size_t)(t + tau) * Hkv + g) * K + k];
    const int64_t pos = (int64_t)L - Tq_s + i0 + tau;
    const bool valid = b >= 0 && b < nblk && (!p.causal || (int64_t)kBlk * b <= pos);
    s_sel[idx] = valid ? b : -1;
    if (use_bits && valid) atomicOr(&bits[tau * wb + (b >> 5)], 1u << (b & 31));
  };
  if constexpr (ATTN) {
    for (int idx = tid; idx < nt * K; idx += 256) {
      const int tau = idx / K;
      load_pick(idx, tau, idx - tau * K);
    }
  } else {
#pragma unroll 4
    for (SlotWalk<256> w(tid, K); w.idx < nt * K; w.next(K)) load_pick(w.idx, w.tau, w.k);
  }
  for (int tau = tid; tau < nt; tau += 256) s_nres[tau] = 0;
  if (tid < 64) s_miss[tid] = 0;
  if (stream && tid < K * ppb) s_page[tid] = my_page;
  __syncthreads();

  // the chain: the leader's valid picks present in every token of the tile.
  // One thread per (token, leader pick) looks for the pick in the token's
  // list; a miss marks the pick.
  if (p.T > 0) {
    auto test_pick = [&](int tau, int k) {
      const int bl = s_sel[k];
      if (bl < 0) return;
      bool found = false;
      if (use_bits) {
        found = (bits[tau * wb + (bl >> 5)] >> (bl & 31)) & 1u;
      } else {
        for (int k2 = 0; k2 < K; ++k2) found |= (s_sel[tau * K + k2] == bl);
      }
      if (!found) s_miss[k] = 1;
    };
    if constexpr (ATTN) {
      for (int idx = tid + K; idx < nt * K; idx += 256) {  // tokens 1 .. nt-1
        const int tau = idx / K;
        test_pick(tau, idx - tau * K);
      }
    } else {
      for (SlotWalk<256> w(tid + K, K); w.idx < nt * K; w.next(K)) test_pick(w.tau, w.k);
    }
  }
  __syncthreads();
  if (wave == 0) {
    bool in_chain = false;
    int bl = -1;
    if (p.T > 0 && lane < K) {
      bl = s_sel[lane];
      in_chain = bl >= 0 && s_miss[lane] == 0;
      for (int k2 = 0; k2 < lane && in_chain; ++k2) in_chain = s_sel[k2] != bl;  // first occurrence only
    }
    const uint64_t mask = __ballot(in_chain);
    if (in_chain) {
      const int rank = __popcll(mask & ((1ull << lane) - 1ull));
      s_chain[rank] = bl;
      s_chain_k[rank] = lane;
      p.chain_blk[tg * K + rank] = bl;
      if (use_bits) atomicOr(&bits[nt * wb + (bl >> 5)], 1u << (bl & 31));
    }
    if (lane == 0) s_nch = __popcll(mask);
  }
  __syncthreads();
  const int n_ch = s_nch;

  // flags, residual bits, residual counts
  auto flag_slot = [&](int idx, int tau, int k) {
    const int b = s_sel[idx];
    uint8_t flag = 0;
    if (b >= 0) {
      bool cov = false;
      if (use_bits) {
        cov = (bits[nt * wb + (b >> 5)] >> (b & 31)) & 1u;
      } else {
        for (int c = 0; c < n_ch; ++c) cov |= (s_chain[c] == b);
      }
      flag = cov ? 1 : 2;
      if (!cov) {
        const int tt = t + tau;
        atomicOr(&p.bitmap[((size_t)b * Hkv + g) * p.W + (tt >> 5)], 1u << (tt & 31));
        atomicAdd(&s_nres[tau], 1);
      }
    }
    p.slot_flag[((size_t)(t + tau) * Hkv + g) * K + k] = flag;
    if (flag == 2) s_sel[idx] = b | kResidualMark;
  };
  if constexpr (ATTN) {
    for (int idx = tid; idx < nt * K; idx += 256) {
      const int tau = idx / K;
      flag_slot(idx, tau, idx - tau * K);
    }
  } else {
    for (SlotWalk<256> w(tid, K); w.idx < nt * K; w.next(K)) flag_slot(w.idx, w.tau, w.k);
  }
  __syncthreads();
  if (p.res_rank) {  // rank of each residual slot among its token's residual slots
    for (int idx = tid; idx < nt * K; idx += 256) {
      if (!(s_sel[idx] & kResidualMark) || s_sel[idx] < 0) continue;
      const int tau = idx / K;
      int rank = 0;
      for (int i = tau * K; i < idx; ++i) rank += (s_sel[i] >= 0 && (s_sel[i] & kResidualMark)) ? 1 : 0;
      p.res_rank[((size_t)(t + tau) * Hkv + g) * K + (idx - tau * K)] = (uint8_t)rank;
    }
  }

  // per-token results; the tile is finished here or listed
  if (wave == 0) {
    int res = 0;
    for (int tau = lane; tau < nt; tau += 64) {
      const size_t tg2 = (size_t)(t + tau) * Hkv + g;
      const int nr = s_nres[tau];
      p.tok_chain[tg2] = n_ch;
      p.tok_nres[tg2] = nr;
      res += nr;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) res += __shfl_xor(res, off, 64);
    if (lane == 0) {
      s_tile_res = res;
      if (res > 0) p.counters[kCntResidual] = 1;  // "some"; the index kernel writes the total
      const bool here = p.stream_narrow && rows <= stream_rows && res == 0;
      int item = -1;  // the tile kernel's item for this tile
      if (!here && p.list_tiles) {
        item = atomicAdd(&p.counters[kCntTiles], 1);
        p.tile_items[item] = (int)tg;
      }
      if (!p.stream_narrow) item = (int)(g * gridDim.x + blockIdx.x);
      s_item_idx = item;
    }
  }
  __syncthreads();
  if (p.tdesc && s_item_idx >= 0 && tid < 64)
    write_tile_desc(p, s_item_idx, t, s, nt, n_ch, L, Tq_s, q0, g, s_chain, tid);
  if constexpr (ATTN) {
    if (stream && s_tile_res == 0)
      stream_chain<CT, KVT, RS>(p, t, g, s, L, Tq_s, q0, rows, n_ch, ppb, s_chain, s_chain_k, s_page);
  }
}

// ---------------------------------------------------------------------------
// wave-per-tile classification (tiles of at most kWaveSlots slots): the same
// rules as k_front's classification, with each wave handling one tile on its
// own, so a workgroup carries four tiles and no workgroup barrier. Used
// outside decode mode, where the front kernel only classifies.
// ---------------------------------------------------------------------------
constexpr int kWaveSlots = 512;  // tile tokens x topk handled by one wave
constexpr int kWaveBitWords = 1024;  // per wave: the tokens' block sets and the chain's, as bit masks
constexpr int kOwnWordBlocks = 512;  // whole-word bitmap stores up to this many blocks a sequence (else atomics)

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


__global__ __launch_bounds__(256) void k_classify_waves(Params p, int ntiles) {
  __shared__ int s_sel[4][kWaveSlots];  // valid picks, -1 where the slot is invalid
  __shared__ uint32_t s_bits[4][kWaveBitWords];  // token tau's picks at [tau * wb], the chain's at [nt * wb]
  __shared__ int s_chain[4][64];
  __shared__ int s_nres[4][128];
  __shared__ unsigned long long s_miss[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.y;
  const int j = blockIdx.x * 4 + wave;
  const int K = p.K, Hkv = p.Hkv;
  const int Teff = p.T > 0 ? p.T : 1;
  if (j >= ntiles) return;
  int64_t t0l;
  const int s = wave_tile_of(p.cu, p.B, p.Tq, Teff, j, &t0l);
  const int item = g * ntiles + j;  // the tile kernel's item (KV head, tile number)
  if (s < 0) {
    if (p.tdesc && lane < 2) p.tdesc[2 * (size_t)item + lane] = int4{0, 0, 0, 0};  // no tile: nothing to do
    return;
  }
  const int t = (int)t0l;
  const size_t tg = (size_t)t * Hkv + g;
  const int64_t q0 = p.cu[s], qe = p.cu[s + 1];
  const int nt = (int)min((int64_t)Teff, min(qe, (int64_t)p.Tq) - t);
  const int L = p.used[s];
  const int Tq_s = (int)(qe - q0);
  const int i0 = (int)(t - q0);
  const int nblk = L > 0 ? min((L + kBlk - 1) / kBlk, p.nb_max) : 0;
  int* sel = s_sel[wave];
  // Set membership (is a leader pick among a token's picks, is a pick in the
  // chain) through bit masks of the blocks when they fit, one bit test each,
  // instead of scans over the top-k
  const int wb = (nblk + 31) >> 5;  // words per block mask
  const bool use_bits = p.T > 0 && (nt + 1) * wb <= kWaveBitWords;
  uint32_t* bits = s_bits[wave];
  if (use_bits) {
    for (int i = lane; i < (nt + 1) * wb; i += 64) bits[i] = 0u;
    wave_lds_sync();
  }
  {
    // every round's pick is requested before the first is used (one round
    // trip instead of one per round)
    constexpr int kRounds = kWaveSlots / 64;
    int braw[kRounds];
    SlotWalk<64> w(lane, K);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      braw[r] = w.idx < nt * K ? p.selected[tg * K + (size_t)w.tau * Hkv * K + w.k] : -1;
      w.next(K);
    }
    w = SlotWalk<64>(lane, K);
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      if (w.idx < nt * K) {
        const int tau = w.tau, b = braw[r];
        const int64_t pos = (int64_t)L - Tq_s + i0 + tau;
        const bool valid = b >= 0 && b < nblk && (!p.causal || (int64_t)kBlk * b <= pos);
        sel[w.idx] = valid ? b : -1;
        if (use_bits && valid) atomicOr(&bits[tau * wb + (b >> 5)], 1u << (b & 31));
      }
      w.next(K);
    }
  }
  for (int tau = lane; tau < nt; tau += 64) s_nres[wave][tau] = 0;
  if (lane == 0) s_miss[wave] = 0ull;
  wave_lds_sync();
  // the chain: the leader's valid picks present in every token of the tile
  if (p.T > 0) {
    unsigned long long miss = 0ull;
    for (SlotWalk<64> w(lane, K); w.idx < nt * K; w.next(K)) {
      if (w.tau == 0) continue;  // the leader itself
      const int tau = w.tau, k = w.k;
      const int bl = sel[k];
      if (bl < 0) continue;
      bool found = false;
      if (use_bits) {
        found = (bits[tau * wb + (bl >> 5)] >> (bl & 31)) & 1u;
      } else {
        for (int k2 = 0; k2 < K; ++k2) found |= (sel[tau * K + k2] == bl);
      }
      if (!found) miss |= 1ull << k;
    }
    if (miss) atomicOr(&s_miss[wave], miss);
  }
  wave_lds_sync();
  bool in_chain = false;
  int bl = -1;
  if (p.T > 0 && lane < K) {
    bl = sel[lane];
    in_chain = bl >= 0 && !((s_miss[wave] >> lane) & 1ull);
    for (int k2 = 0; k2 < lane && in_chain; ++k2) in_chain = sel[k2] != bl;  // first occurrence only
  }
  const uint64_t mask = __ballot(in_chain);
  const int n_ch = __popcll(mask);
  if (in_chain) {
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    s_chain[wave][rank] = bl;
    p.chain_blk[tg * K + rank] = bl;
    if (use_bits) atomicOr(&bits[nt * wb + (bl >> 5)], 1u << (bl & 31));
  }
  wave_lds_sync();
  if (p.tdesc) write_tile_desc(p, item, t, s, nt, n_ch, L, Tq_s, q0, g, s_chain[wave], lane);
  // flags, residual bits, residual counts, and each residual slot's rank
  // among its token's residual slots: the residual lanes of a round before
  // it that hold the same token, plus those of earlier rounds (a token
  // started in an earlier round continues at lane 0; `carry` counts its
  // residual slots so far)
  // A tile whose tokens are exactly one bitmap word (32 tokens from a
  // multiple of 32, or fewer that are the batch's last) is that word's only
  // writer: it builds each residual block's word from the block masks and
  // stores it whole (below) instead of setting bits with device-scope
  // atomics.
  const bool own_words =
      use_bits && (t & 31) == 0 && (nt == 32 || (nt < 32 && t + nt >= p.Tq)) && nblk <= kOwnWordBlocks;
  int res = 0, carry = 0;
  for (SlotWalk<64> w(lane, K); w.idx - lane < nt * K; w.next(K)) {
    const bool act = w.idx < nt * K;
    const int tau = w.tau;
    const int b = act ? sel[w.idx] : -1;
    uint8_t flag = 0;
    if (b >= 0) {
      bool cov = false;
      if (use_bits) {
        cov = (bits[nt * wb + (b >> 5)] >> (b & 31)) & 1u;
      } else {
        for (int c = 0; c < n_ch; ++c) cov |= (s_chain[wave][c] == b);
      }
      flag = cov ? 1 : 2;
      if (!cov) {
        const int tt = t + tau;
        if (!own_words) atomicOr(&p.bitmap[((size_t)b * Hkv + g) * p.W + (tt >> 5)], 1u << (tt & 31));
        atomicAdd(&s_nres[wave][tau], 1);
        ++res;
      }
    }
    if (act) p.slot_flag[tg * K + (size_t)tau * Hkv * K + w.k] = flag;
    const uint64_t resm = __ballot(flag == 2);
    if (p.res_rank) {
      const int st = lane - w.k;  // the lane of the token's first slot in this round
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      const uint64_t from = st > 0 ? (~0ull << st) : ~0ull;
      const int rank = (st < 0 ? carry : 0) + __popcll(resm & below & from);
      if (flag == 2) p.res_rank[tg * K + (size_t)tau * Hkv * K + w.k] = (uint8_t)rank;
      const int st63 = 63 - __builtin_amdgcn_readlane(w.k, 63);  // the last lane's token
      carry = (st63 < 0 ? carry : 0) + __popcll(resm & (st63 > 0 ? (~0ull << st63) : ~0ull));
    }
  }
  wave_lds_sync();  // the residual counts
  if (own_words) {
    // block b's word: bit tau for each token that picked b outside the chain
    // (the masks hold valid picks only; reads of one round share two words)
    for (int b = lane; b < nblk; b += 64) {
      const int wi = b >> 5, sh = b & 31;
      uint32_t word = 0u;
      for (int tau = 0; tau < nt; ++tau) word |= ((bits[tau * wb + wi] >> sh) & 1u) << tau;
      if (word != 0u && !((bits[nt * wb + wi] >> sh) & 1u)) p.bitmap[((size_t)b * Hkv + g) * p.W + (t >> 5)] = word;
    }
  }
  for (int tau = lane; tau < nt; tau += 64) {
    const size_t tg2 = tg + (size_t)tau * Hkv;
    p.tok_chain[tg2] = n_ch;
    p.tok_nres[tg2] = s_nres[wave][tau];
  }
  const bool any_res = __any(res > 0);
  if (lane == 0) {
    if (any_res) p.counters[kCntResidual] = 1;  // "some"; the index kernel writes the total
    if (p.list_tiles) p.tile_items[atomicAdd(&p.counters[kCntTiles], 1)] = (int)tg;
  }
}

// ---------------------------------------------------------------------------
// exhaustive-test entry: widen e4m3fn bytes exactly as the kernels do
// ---------------------------------------------------------------------------
template <typename CT>
__global__ void k_widen(const uint8_t* __restrict__ in, int64_t n16, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n16) return;
  const u32x4 raw = *(const u32x4*)(in + 16 * i);
  *(u32x4*)(out + 16 * i) = widen8<CT>(u32x2{raw[0], raw[1]});
  *(u32x4*)(out + 16 * i + 8) = widen8<CT>(u32x2{raw[2], raw[3]});
}

hipError_t launch_widen_fp8(const void* in, int64_t n, int out_elem, void* out, hipStream_t st) {
  const int64_t n16 = n / 16;
  if (n16 <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n16 + 255) / 256);
  if (out_elem == kElemBF16)
    hipLaunchKernelGGL(k_widen<bf16_t>, dim3(blocks), dim3(256), 0, st, (const uint8_t*)in, n16, (uint16_t*)out);
  else
    hipLaunchKernelGGL(k_widen<f16_t>, dim3(blocks), dim3(256), 0, st, (const uint8_t*)in, n16, (uint16_t*)out);
  return hipGetLastError();
}

template <typename CT, typename KVT, bool ATTN>
static hipError_t launch_front_t(const ProfSpan& sp, const Params& p, hipStream_t st) {
  const int Teff = p.T > 0 ? p.T : 1;
  const size_t lds = (size_t)Teff * p.K * sizeof(int);
  const unsigned gx = p.stream_narrow ? (unsigned)p.Tq : (unsigned)((p.Tq + Teff - 1) / Teff + p.B);
  // one-token tiles of more than 16 query rows: two row sets per wave
  if (ATTN && p.front_only && p.G > 16)
    return launch_k(sp, true, true, k_front<CT, KVT, ATTN, 2>, dim3(gx, p.Hkv), dim3(256), (uint32_t)lds, st, p);
  return launch_k(sp, true, true, k_front<CT, KVT, ATTN, 1>, dim3(gx, p.Hkv), dim3(256), (uint32_t)lds, st, p);
}

hipError_t launch_front(const Params& p, int q_elem, int kv_elem, hipStream_t st) {
  const ProfSpan sp = profile_begin(kKFront);
  hipError_t e;
  // outside decode mode the front kernel only classifies: the light
  // instantiation (no attention registers or LDS) keeps many workgroups per CU
  const int Teff = p.T > 0 ? p.T : 1;
  if (!p.stream_narrow && Teff * p.K <= kWaveSlots) {
    // every tile is listed or enumerated: one wave per tile
    const int ntiles = (p.Tq + Teff - 1) / Teff + p.B;
    e = launch_k(sp, true, true, k_classify_waves, dim3((ntiles + 3) / 4, p.Hkv), dim3(256), 0, st, p, ntiles);
  } else if (q_elem < 0 || !p.stream_narrow)
    e = launch_front_t<bf16_t, bf16_t, false>(sp, p, st);
  else if (q_elem == kElemBF16)
    e = kv_elem == kElemFP8   ? launch_front_t<bf16_t, fp8_e4m3_t, true>(sp, p, st)
        : kv_elem == kElemFP4 ? launch_front_t<bf16_t, mxfp4_t, true>(sp, p, st)
                              : launch_front_t<bf16_t, bf16_t, true>(sp, p, st);
  else
    e = kv_elem == kElemFP8 ? launch_front_t<f16_t, fp8_e4m3_t, true>(sp, p, st)
                            : launch_front_t<f16_t, f16_t, true>(sp, p, st);
  profile_end(sp, e == hipSuccess);
  return e;
}

}  // namespace msa
