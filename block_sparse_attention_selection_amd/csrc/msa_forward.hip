// msa_forward.hip -- KV-stationary block-sparse attention on gfx950 MFMA.
//
// fw-ai/minimax-kernels README, intro: a selected KV block is loaded once
// and every query that selected it is processed against it. Work arrives as
//   chain items  a tile of consecutive tokens of one sequence (x the G query
//                heads of KV head g) and the blocks that every token of the
//                tile selected: query rows stay in registers while the
//                blocks stream past (decode is the one-token case);
//   units        up to Tu tokens that picked one block outside their tile's
//                chain (KV-outer proper): the block is staged once in LDS
//                and all the units' rows are multiplied against it.
// Each wave owns 16 query rows. Scores are computed transposed,
// S^T = K * Q^T, so that a lane's D fragment holds one query row; the
// probabilities are then already laid out as the B operand of
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

#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

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

// One 32-key chunk: scores, masked online softmax, P*V.
//   ka[j][s]  K fragment: key 16j + c, dims of k-step s
//   va[e]     V fragment: key key_of(q, e), dims 8c .. 8c+7
//   key0      token index of key 0 of the chunk; keys at or beyond lim are absent
//   run_seq   sequence the chunk belongs to (rows of other sequences skip it)
template <typename CT>
__device__ __forceinline__ void tile_chunk(RowTile<CT>& rt, const u32x4 (&ka)[2][4],
                                           const u32x4 (&va)[8], int key0, int lim, int run_seq,
                                           int q, float scale_log2) {
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
  const float m_new = fmaxf(rt.m, cmax);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = exp2f(rt.m - m_use);
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2f(x[e] - m_use);
    psum += p[e];
  }
  rt.l = rt.l * alpha + psum;
  rt.m = m_new;
  u32x4 pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = pack2<CT>(p[2 * i], p[2 * i + 1]);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    rt.o[t] *= alpha;
    u32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x0 = va[2 * i][t >> 1], x1 = va[2 * i + 1][t >> 1];
      a[i] = (t & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
    }
    rt.o[t] = Mma<CT>::run(a, pb, rt.o[t]);
  }
}

template <typename KVT>
struct KvElem {
  typedef uint16_t type;
};
template <>
struct KvElem<fp8_e4m3_t> {
  typedef uint8_t type;
};

// Locate one 32-key chunk of block b of sequence s, KV head g.
// Returns the number of present keys (0: nothing to do) and sets the bases.
template <typename KVT>
__device__ __forceinline__ int chunk_base(const Params& p, int s, int g, int b, int part, int L,
                                          const typename KvElem<KVT>::type*& kb,
                                          const typename KvElem<KVT>::type*& vb) {
  typedef typename KvElem<KVT>::type E;
  const int key0 = kBlk * b + 32 * part;
  if (key0 >= L) return 0;  // L is already clamped to the page table's reach
  const int page = p.block_tables[(size_t)s * p.MP + key0 / p.P];
  if (page < 0 || page >= p.NP) return 0;
  const size_t off = (((size_t)page * p.Hkv + g) * p.P + (key0 % p.P)) * kD;
  kb = (const E*)p.k + off;
  vb = (const E*)p.v + off;
  return min(32, L - key0);
}

// ---------------------------------------------------------------------------
// global -> register fragments of one chunk (narrow kernel). Raw cache bytes
// are held until the chunk is multiplied, so the loads of the next chunk
// stay in flight while the current one is being computed.
// ---------------------------------------------------------------------------
template <typename CT, typename KVT>
struct Frag;

template <typename CT>
struct Frag<CT, CT> {  // 16-bit cache: fragments are used as loaded
  u32x4 ka[2][4];
  u32x4 va[8];
  int key0;
  int nv;  // keys present in the chunk (0: skip)
  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, int q, int c) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int key = 16 * j + c;
      const bool ok = key < nv;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        ka[j][s] = ok ? *(const u32x4*)(kb + key * kD + kmap(s, q)) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = key_of(q, e);
      va[e] = (key < nv) ? *(const u32x4*)(vb + key * kD + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void compute(RowTile<CT>& rt, int L, int s, int q, float sl2) const {
    tile_chunk(rt, ka, va, key0, L, s, q, sl2);
  }
};

template <typename CT>
struct Frag<CT, fp8_e4m3_t> {  // e4m3fn cache: 16 raw bytes per K pair, 8 per V row
  u32x4 kr[2][2];
  u32x2 vr[8];
  int key0;
  int nv;
  __device__ __forceinline__ void load(const uint8_t* kb, const uint8_t* vb, int q, int c) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int key = 16 * j + c;
      const bool ok = key < nv;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        kr[j][pp] = ok ? *(const u32x4*)(kb + key * kD + 64 * pp + 16 * q) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = key_of(q, e);
      vr[e] = (key < nv) ? *(const u32x2*)(vb + key * kD + 8 * c) : u32x2{0u, 0u};
    }
  }
  __device__ __forceinline__ void compute(RowTile<CT>& rt, int L, int s, int q, float sl2) const {
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
    tile_chunk(rt, ka, va, key0, L, s, q, sl2);
  }
};

// Fragments of chunk ci (block ci/4, keys 32*(ci%4) ..) of a chain.
template <typename CT, typename KVT>
__device__ __forceinline__ void fetch_chunk(Frag<CT, KVT>& f, const Params& p, const int32_t* blocks,
                                            int nchunks, int ci, int s, int g, int L, int q, int c) {
  typedef typename KvElem<KVT>::type E;
  f.nv = 0;
  if (ci >= nchunks) return;
  const int b = blocks[ci >> 2], part = ci & 3;
  const E* kb = nullptr;
  const E* vb = nullptr;
  f.nv = chunk_base<KVT>(p, s, g, b, part, L, kb, vb);
  f.key0 = kBlk * b + 32 * part;
  if (f.nv > 0) f.load(kb, vb, q, c);
}

// ---------------------------------------------------------------------------
// narrow kernel: chain items with at most 16 rows (decode and tiny tiles).
// The item's chunks are split over the four waves, each streaming its K/V
// fragments straight from HBM into registers; the waves' softmax states are
// merged through LDS at the end.
// ---------------------------------------------------------------------------
template <typename CT, typename KVT>
__global__ __launch_bounds__(256) void k_fwd_narrow(Params p) {
  __shared__ float s_o[4][16][kD + 4];
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int n_items = p.counters[kCntNarrow];
  const int Teff = p.T > 0 ? p.T : 1;

  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int code = p.narrow_items[it];
    const int t0 = code / p.Hkv, g = code - (code / p.Hkv) * p.Hkv;
    const int s = seq_of(p.cu, p.B, t0);
    const int64_t q0 = p.cu[s], q1 = min(p.cu[s + 1], (int64_t)p.Tq);
    const int Tq_s = (int)(p.cu[s + 1] - q0);
    const int L = min(p.used[s], p.MP * p.P);  // keys the page table can reach
    const int nt = (int)min((int64_t)Teff, q1 - t0);
    const int rows = nt * p.G;
    const int nch = p.tok_chain[(size_t)t0 * p.Hkv + g];
    const int32_t* blocks = p.chain_blk + ((size_t)t0 * p.Hkv + g) * p.K;

    RowTile<CT> rt;
    tile_reset(rt);
    int tok = -1, h = 0;
    if (c < rows) {
      tok = t0 + c / p.G;
      h = g * p.G + (c % p.G);
      rt.pos = p.causal ? (int)(p.used[s] - Tq_s + (tok - q0)) : INT_MAX;
      rt.seq = s;
    } else {
      rt.pos = -1;
      rt.seq = -1;
    }
    tile_load_q(rt, p, tok, h, q);

    // software pipeline: fragments of the next chunk are in flight while
    // the current one is multiplied
    const int nchunks = nch * 4;
    Frag<CT, KVT> fa, fb;
    int ci = wave;
    fetch_chunk<CT, KVT>(fa, p, blocks, nchunks, ci, s, g, L, q, c);
    while (ci < nchunks) {
      fetch_chunk<CT, KVT>(fb, p, blocks, nchunks, ci + 4, s, g, L, q, c);
      if (fa.nv > 0) fa.compute(rt, L, s, q, p.scale_log2);
      ci += 4;
      if (ci >= nchunks) break;
      fetch_chunk<CT, KVT>(fa, p, blocks, nchunks, ci + 4, s, g, L, q, c);
      if (fb.nv > 0) fb.compute(rt, L, s, q, p.scale_log2);
      ci += 4;
    }

    // merge the four waves
    const float l_row = sum_over_groups(rt.l);
    if (q == 0) {
      s_m[wave][c] = rt.m;
      s_l[wave][c] = l_row;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][c][32 * q + 8 * r + t] = rt.o[t][r];
    __syncthreads();
    {
      const int row = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
      if (row < rows) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][row]);
        const float Mu = (M == -INFINITY) ? 0.f : M;
        float wsum = 0.f, acc[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f = exp2f(s_m[w][row] - Mu);
          wsum += f * s_l[w][row];
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[d] += f * s_o[w][row][d0 + d];
        }
        const int rtok = t0 + row / p.G;
        const int rh = g * p.G + (row % p.G);
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        const float lse2 = wsum > 0.f ? Mu + log2f(wsum) : -INFINITY;
        if (p.tok_nres[(size_t)rtok * p.Hkv + g] == 0) {
          u32x4 pk;
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[i] = pack2<CT>(acc[2 * i] * inv, acc[2 * i + 1] * inv);
          *(u32x4*)((uint16_t*)p.out + ((size_t)rtok * p.Hq + rh) * kD + d0) = pk;
          if (d0 == 0 && p.lse) p.lse[(size_t)rh * p.Tq + rtok] = lse2 * kLn2;
        } else {
          float* dst = p.cpart + ((size_t)rtok * p.Hq + rh) * kD + d0;
#pragma unroll
          for (int d = 0; d < 8; ++d) dst[d] = acc[d] * inv;
          if (d0 == 0) p.clse[(size_t)rtok * p.Hq + rh] = lse2;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// wide kernel: chain items with more than 16 rows, then KV-outer units.
// Each block is staged once in LDS (K and V, 16-bit, 16-byte chunks XOR-
// swizzled by row so both operand read patterns are bank-conflict free) and
// every wave multiplies its one or two 16-row tiles against it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

template <typename CT, typename KVT>
struct BlockStager;

template <typename CT>
struct BlockStager<CT, CT> {
  // 128 rows x 16 chunks per tensor; 8 chunks of K and 8 of V per thread
  static __device__ __forceinline__ void stage(u32x4* sk, u32x4* sv, const Params& p, int s, int g,
                                               int b, int L) {
    for (int i = 0; i < 8; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int row = idx >> 4, ch = idx & 15;
      const int tok = kBlk * b + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (tok < L) {
        const int page = p.block_tables[(size_t)s * p.MP + tok / p.P];
        if (page >= 0 && page < p.NP) {
          const size_t off = (((size_t)page * p.Hkv + g) * p.P + (tok % p.P)) * kD + 8 * ch;
          kv = *(const u32x4*)((const uint16_t*)p.k + off);
          vv = *(const u32x4*)((const uint16_t*)p.v + off);
        }
      }
      sk[swz(row, ch)] = kv;
      sv[swz(row, ch)] = vv;
    }
  }
};

template <typename CT>
struct BlockStager<CT, fp8_e4m3_t> {
  // 128 rows x 8 chunks of 16 fp8 per tensor; 4 chunks of K and 4 of V per thread
  static __device__ __forceinline__ void stage(u32x4* sk, u32x4* sv, const Params& p, int s, int g,
                                               int b, int L) {
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int row = idx >> 3, ch = idx & 7;
      const int tok = kBlk * b + row;
      u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
      if (tok < L) {
        const int page = p.block_tables[(size_t)s * p.MP + tok / p.P];
        if (page >= 0 && page < p.NP) {
          const size_t off = (((size_t)page * p.Hkv + g) * p.P + (tok % p.P)) * kD + 16 * ch;
          kr = *(const u32x4*)((const uint8_t*)p.k + off);
          vr = *(const u32x4*)((const uint8_t*)p.v + off);
        }
      }
      sk[swz(row, 2 * ch)] = widen8<CT>(u32x2{kr[0], kr[1]});
      sk[swz(row, 2 * ch + 1)] = widen8<CT>(u32x2{kr[2], kr[3]});
      sv[swz(row, 2 * ch)] = widen8<CT>(u32x2{vr[0], vr[1]});
      sv[swz(row, 2 * ch + 1)] = widen8<CT>(u32x2{vr[2], vr[3]});
    }
  }
};

template <typename CT>
__device__ __forceinline__ void lds_fragments(u32x4 (&ka)[2][4], u32x4 (&va)[8], const u32x4* sk,
                                              const u32x4* sv, int part, int q, int c) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 32 * part + 16 * j + c;
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[j][s] = sk[swz(row, kmap(s, q) >> 3)];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) va[e] = sv[swz(32 * part + key_of(q, e), c)];
}

template <typename CT, typename KVT>
__global__ __launch_bounds__(256) void k_fwd_wide(Params p) {
  __shared__ u32x4 s_k[kBlk * 16];
  __shared__ u32x4 s_v[kBlk * 16];
  __shared__ int s_tok[128];
  __shared__ int s_seq[128];
  __shared__ int s_item;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, c = lane & 15;
  const int n_chain = p.counters[kCntWide];
  const int total = n_chain + p.counters[kCntUnits];
  const int Teff = p.T > 0 ? p.T : 1;

  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(&p.counters[kCntWideNext], 1);
    __syncthreads();
    const int it = s_item;
    if (it >= total) break;

    // ---- item description
    int g, ntok, nblocks, b_unit = 0, e0 = 0;
    const int32_t* blocks = nullptr;
    const bool is_chain = it < n_chain;
    if (is_chain) {
      const int code = p.wide_items[it];
      const int t0 = code / p.Hkv;
      g = code - t0 * p.Hkv;
      const int s = seq_of(p.cu, p.B, t0);
      ntok = (int)min((int64_t)Teff, min(p.cu[s + 1], (int64_t)p.Tq) - t0);
      nblocks = p.tok_chain[(size_t)t0 * p.Hkv + g];
      blocks = p.chain_blk + ((size_t)t0 * p.Hkv + g) * p.K;
      if (threadIdx.x < ntok) {
        s_tok[threadIdx.x] = t0 + threadIdx.x;
        s_seq[threadIdx.x] = s;
      }
    } else {
      const int u = it - n_chain;
      int lo = 0, hi = p.NR;  // largest r with unit_off[r] <= u
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.unit_off[mid] <= u)
          lo = mid;
        else
          hi = mid;
      }
      const int r = lo;
      b_unit = r / p.Hkv;
      g = r - b_unit * p.Hkv;
      e0 = p.row_off[r] + (u - p.unit_off[r]) * p.Tu;
      ntok = min(p.Tu, p.row_off[r + 1] - e0);
      nblocks = 1;
      if (threadIdx.x < ntok) {
        const int slot = p.ent[e0 + threadIdx.x];
        const int tk = slot / (p.Hkv * p.K);
        s_tok[threadIdx.x] = tk;
        s_seq[threadIdx.x] = seq_of(p.cu, p.B, tk);
      }
    }
    __syncthreads();
    const int rows = ntok * p.G;

    // ---- the wave's row tiles (w and w + 4)
    RowTile<CT> rt[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      tile_reset(rt[i]);
      const int rho = 16 * (wave + 4 * i) + c;
      int tok = -1, h = 0;
      rt[i].seq = -1;
      rt[i].pos = -1;
      if (rho < rows) {
        const int tau = rho / p.G;
        tok = s_tok[tau];
        h = g * p.G + (rho - tau * p.G);
        const int s = s_seq[tau];
        rt[i].seq = s;
        const int64_t q0 = p.cu[s];
        rt[i].pos = p.causal ? (int)(p.used[s] - (p.cu[s + 1] - q0) + (tok - q0)) : INT_MAX;
      }
      tile_load_q(rt[i], p, tok, h, q);
    }
    const bool has0 = 16 * wave < rows, has1 = 16 * (wave + 4) < rows;

    // ---- blocks (a unit may span several sequences: one run per sequence)
    int run_start = 0;
    for (int bi = 0; bi < nblocks;) {
      int s_run, b;
      if (is_chain) {
        s_run = s_seq[0];
        b = blocks[bi];
      } else {
        s_run = s_seq[run_start];
        b = b_unit;
      }
      const int L = min(p.used[s_run], p.MP * p.P);  // keys the page table can reach
      BlockStager<CT, KVT>::stage(s_k, s_v, p, s_run, g, b, L);
      __syncthreads();
      const int nparts = min(4, (L - kBlk * b + 31) / 32);
      for (int part = 0; part < nparts; ++part) {
        u32x4 ka[2][4], va[8];
        lds_fragments<CT>(ka, va, s_k, s_v, part, q, c);
        const int key0 = kBlk * b + 32 * part;
        if (has0) tile_chunk(rt[0], ka, va, key0, L, s_run, q, p.scale_log2);
        if (has1) tile_chunk(rt[1], ka, va, key0, L, s_run, q, p.scale_log2);
      }
      __syncthreads();
      if (is_chain) {
        ++bi;
      } else {
        int nxt = run_start;
        while (nxt < ntok && s_seq[nxt] == s_run) ++nxt;
        run_start = nxt;
        if (run_start >= ntok) bi = nblocks;
      }
    }

    // ---- results of the wave's tiles
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float l_row = sum_over_groups(rt[i].l);
      const int rho = 16 * (wave + 4 * i) + c;
      if (rho >= rows) continue;
      const int tau = rho / p.G;
      const int hr = rho - tau * p.G;
      const int tok = s_tok[tau];
      const int h = g * p.G + hr;
      const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
      const float mu = rt[i].m == -INFINITY ? 0.f : rt[i].m;
      const float lse2 = l_row > 0.f ? mu + log2f(l_row) : -INFINITY;
      if (is_chain && p.tok_nres[(size_t)tok * p.Hkv + g] == 0) {
        uint16_t* dst = (uint16_t*)p.out + ((size_t)tok * p.Hq + h) * kD + 32 * q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x4 pk;
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2)
            pk[k2] = pack2<CT>(rt[i].o[2 * k2][r] * inv, rt[i].o[2 * k2 + 1][r] * inv);
          *(u32x4*)(dst + 8 * r) = pk;
        }
        if (q == 0 && p.lse) p.lse[(size_t)h * p.Tq + tok] = lse2 * kLn2;
      } else {
        float* dst;
        float* lsd;
        if (is_chain) {
          dst = p.cpart + ((size_t)tok * p.Hq + h) * kD;
          lsd = p.clse + (size_t)tok * p.Hq + h;
        } else {
          const size_t pos = (size_t)(e0 + tau);
          dst = p.opart + (pos * p.G + hr) * kD;
          lsd = p.lpart + pos * p.G + hr;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 a, bq;
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) {
            a[k2] = rt[i].o[k2][r] * inv;
            bq[k2] = rt[i].o[4 + k2][r] * inv;
          }
          *(f32x4*)(dst + 32 * q + 8 * r) = a;
          *(f32x4*)(dst + 32 * q + 8 * r + 4) = bq;
        }
        if (q == 0) *lsd = lse2;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// combine: merge the chain partial and the residual partials of (t, g) by
// their log-sum-exp; writes out[t, h, :] and lse[h, t]
// ---------------------------------------------------------------------------
template <typename CT>
__global__ __launch_bounds__(128) void k_combine(Params p) {
  const int t = blockIdx.x, g = blockIdx.y;
  const size_t tg = (size_t)t * p.Hkv + g;
  const int nch = p.tok_chain[tg];
  const int nres = p.tok_nres[tg];
  if (nch > 0 && nres == 0) return;  // the chain item wrote the final rows
  const int K = p.K;
  for (int idx = threadIdx.x; idx < p.G * 16; idx += 128) {
    const int r = idx >> 4, d0 = (idx & 15) * 8;
    const int h = g * p.G + r;
    float M = -INFINITY;
    if (nch > 0) M = p.clse[(size_t)t * p.Hq + h];
    for (int k = 0; k < K; ++k)
      if (p.slot_flag[tg * K + k] == 2) M = fmaxf(M, p.lpart[(size_t)p.slot_pos[tg * K + k] * p.G + r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float wsum = 0.f, acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.f;
    if (nch > 0) {
      const float f = exp2f(p.clse[(size_t)t * p.Hq + h] - Mu);
      const float* src = p.cpart + ((size_t)t * p.Hq + h) * kD + d0;
      wsum += f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] += f * src[d];
    }
    for (int k = 0; k < K; ++k) {
      if (p.slot_flag[tg * K + k] != 2) continue;
      const size_t pos = (size_t)p.slot_pos[tg * K + k];
      const float f = exp2f(p.lpart[pos * p.G + r] - Mu);
      const float* src = p.opart + (pos * p.G + r) * kD + d0;
      wsum += f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] += f * src[d];
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = pack2<CT>(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    *(u32x4*)((uint16_t*)p.out + ((size_t)t * p.Hq + h) * kD + d0) = pk;
    if (d0 == 0 && p.lse) p.lse[(size_t)h * p.Tq + t] = wsum > 0.f ? (Mu + log2f(wsum)) * kLn2 : -INFINITY;
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

template <typename CT, typename KVT>
static hipError_t launch_forward_t(const Params& p, int num_cu, hipStream_t st) {
  const int max_items = p.Tq * p.Hkv;
  int narrow_grid = min(max_items, num_cu * 8);
  if (narrow_grid < 1) narrow_grid = 1;
  hipLaunchKernelGGL((k_fwd_narrow<CT, KVT>), dim3(narrow_grid), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_fwd_wide<CT, KVT>), dim3(num_cu * 2), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_combine<CT>), dim3(p.Tq, p.Hkv), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_forward(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st) {
  if (q_elem == kElemBF16)
    return kv_elem == kElemFP8 ? launch_forward_t<bf16_t, fp8_e4m3_t>(p, num_cu, st)
                               : launch_forward_t<bf16_t, bf16_t>(p, num_cu, st);
  return kv_elem == kElemFP8 ? launch_forward_t<f16_t, fp8_e4m3_t>(p, num_cu, st)
                             : launch_forward_t<f16_t, f16_t>(p, num_cu, st);
}

}  // namespace msa
