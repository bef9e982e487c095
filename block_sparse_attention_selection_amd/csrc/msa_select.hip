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
// Work: one workgroup of 4 waves per (tile of 16 or 64 consecutive tokens of
// one sequence, KV head). The waves split the tile's blocks; each computes
// S^T = K . Q^T with 16x16x32 MFMA for 16 keys at a time, K read from the
// paged cache straight into operand registers (a lane reads 32 contiguous
// dims of one key row), and max-pools it into a [tokens][blocks] fp32 table
// in LDS. Then each wave takes rows of the table and extracts the top-k with
// wave-wide arg-max rounds.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

constexpr int kSelThreads = 256;
constexpr int kSelPerLane = kSelMaxBlocks / 64;  // score registers per lane in the top-k phase

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

template <typename QT, typename KT, int NRB>
__global__ __launch_bounds__(kSelThreads) void k_select(SelectParams p) {
  constexpr int T = 16 * NRB;  // tokens per tile
  extern __shared__ float s_sc[];  // [T][nb_cap]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.y;
  int64_t t0 = 0;
  const int s = wave_tile_of(p.cu, p.B, p.Tq, T, blockIdx.x, &t0);
  if (s < 0) return;
  const int64_t c0 = p.cu[s], c1 = p.cu[s + 1];
  const int64_t tq_end = min(c1, (int64_t)p.Tq);
  const int ntok = (int)min((int64_t)T, tq_end - t0);
  int L = p.used[s];
  L = min(L, p.MP * p.P);  // a sequence reaches no further than its page table
  const int64_t tq_s = c1 - c0;
  // position of tile row r (bottom-right causal alignment); L - 1 when not causal
  auto pos_of = [&](int r) -> int64_t { return p.causal ? (int64_t)L - tq_s + (t0 + r - c0) : (int64_t)L - 1; };
  const int nb = min((L + 127) / 128, p.nb_cap);
  const int64_t pos_max = pos_of(ntok - 1);
  const int nscan = (L <= 0 || pos_max < 0) ? 0 : (int)min((int64_t)nb, pos_max / 128 + 1);

  if (nscan > 0) {
    // index queries of the tile as MFMA B operands: lane holds token row
    // (lane & 15) of row block rb, dims 32 (lane >> 4) + 8 st + [0, 8)
    const int h = lane >> 4, col = lane & 15;
    u32x4 qf[NRB][4];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 16 + col;
      if (r < ntok) {
        const u32x4* q = (const u32x4*)((const uint16_t*)p.q + ((t0 + r) * p.Hkv + g) * (int64_t)kD + 32 * h);
#pragma unroll
        for (int st = 0; st < 4; ++st) qf[rb][st] = q[st];
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) qf[rb][st] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    int64_t posr[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) posr[rb] = pos_of(rb * 16 + col);
    const int32_t* bt = p.bt + (int64_t)s * p.MP;
    // the key row this lane reads for group gi of this wave's blocks
    auto key_ptr = [&](int j) -> const void* {
      if (j >= L) return nullptr;  // L <= MP * P, so the table read below stays inside the row
      const int page = bt[j / p.P];
      if (page < 0 || page >= p.num_pages) return nullptr;
      const int64_t row = ((int64_t)page * p.Hkv + g) * p.P + (j % p.P);
      return (const uint8_t*)p.k + row * KeyBytes<KT>::kRow;
    };
    const int nblk_w = nscan > wave ? (nscan - wave + 3) / 4 : 0;  // blocks wave, wave + 4, ...
    const int ngroups = nblk_w * 8;
    KeyRow<QT, KT> cur, nxt;
    nxt.zero();
    auto fetch = [&](KeyRow<QT, KT>& kr, int gi) {
      const int b = wave + 4 * (gi >> 3);
      const int j = 128 * b + 16 * (gi & 7) + col;
      const void* ptr = key_ptr(j);
      if (ptr)
        kr.load(ptr, h);
      else
        kr.zero();
    };
    if (ngroups > 0) fetch(cur, 0);
    float m[NRB];
    for (int gi = 0; gi < ngroups; ++gi) {
      if (gi + 1 < ngroups) fetch(nxt, gi + 1);
      const int b = wave + 4 * (gi >> 3);
      if ((gi & 7) == 0) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) m[rb] = -INFINITY;
      }
      const int jbase = 128 * b + 16 * (gi & 7) + 4 * h;  // keys of this lane's accumulator rows
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = Mma<QT>::run(cur.frag(st), qf[rb][st], acc);
        float v = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = jbase + i;
          const bool vis = j < L && (int64_t)j <= posr[rb];
          v = fmaxf(v, vis ? acc[i] : -INFINITY);
        }
        m[rb] = fmaxf(m[rb], max_over_groups(v));
      }
      if ((gi & 7) == 7 && h == 0) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          if (rb * 16 + col < ntok) s_sc[(rb * 16 + col) * p.nb_cap + b] = m[rb];
      }
      cur = nxt;
    }
  }
  __syncthreads();

  // top-k per row: rows wave, wave + 4, ...
  for (int r = wave; r < ntok; r += 4) {
    const int64_t t = t0 + r;
    const int64_t pos = pos_of(r);
    const int nr = (L <= 0 || pos < 0) ? 0 : (int)min((int64_t)nb, pos / 128 + 1);
    int32_t* out = p.selected + (t * p.Hkv + g) * (int64_t)p.topk;
    float v[kSelPerLane];
#pragma unroll
    for (int i = 0; i < kSelPerLane; ++i) {
      const int b = lane + 64 * i;
      float x = b < nr ? s_sc[r * p.nb_cap + b] : -INFINITY;
      if (p.scores && b < p.nb_cap) p.scores[(t * p.Hkv + g) * (int64_t)p.nb_cap + b] = x;
      v[i] = (x != x) ? -INFINITY : x;  // a NaN score is never selected
    }
    int k = 0;
    if (p.force_local && nr > 0 && p.topk > 0) {
      const int lb = (int)(pos / 128);  // the token's own block (the last one when not causal)
      float own = -INFINITY;
#pragma unroll
      for (int i = 0; i < kSelPerLane; ++i)
        if (lane + 64 * i == lb) own = v[i];
      if (__shfl(own, lb & 63, 64) > -INFINITY) {  // it holds the token itself: only a NaN score fails
#pragma unroll
        for (int i = 0; i < kSelPerLane; ++i)
          if (lane + 64 * i == lb) v[i] = -INFINITY;
        if (lane == 0) out[0] = lb;
        k = 1;
      }
    }
    for (; k < p.topk; ++k) {
      float bv = -INFINITY;
      int bb = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < kSelPerLane; ++i)
        if (sel_better(v[i], lane + 64 * i, bv, bb)) {
          bv = v[i];
          bb = lane + 64 * i;
        }
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
#pragma unroll
      for (int i = 0; i < kSelPerLane; ++i)
        if (lane + 64 * i == bb) v[i] = -INFINITY;
    }
    for (int i = k + lane; i < p.topk; i += 64) out[i] = -1;
  }
}

template <typename QT, typename KT>
static hipError_t launch_select_t(const SelectParams& p, int nrb, hipStream_t st) {
  const int T = 16 * nrb;
  const int64_t tiles = ((int64_t)p.Tq + T - 1) / T + p.B;  // each sequence adds at most one partial tile
  const dim3 grid((unsigned)tiles, (unsigned)p.Hkv), block(kSelThreads);
  const size_t lds = (size_t)T * p.nb_cap * sizeof(float);
  if (nrb == 4)
    hipLaunchKernelGGL((k_select<QT, KT, 4>), grid, block, lds, st, p);
  else
    hipLaunchKernelGGL((k_select<QT, KT, 1>), grid, block, lds, st, p);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, int q_elem, bool fp8_keys, int nrb, hipStream_t st) {
  if (p.Tq == 0 || p.Hkv == 0) return hipSuccess;
  if (q_elem == kElemBF16)
    return fp8_keys ? launch_select_t<bf16_t, fp8_e4m3_t>(p, nrb, st) : launch_select_t<bf16_t, bf16_t>(p, nrb, st);
  return fp8_keys ? launch_select_t<f16_t, fp8_e4m3_t>(p, nrb, st) : launch_select_t<f16_t, f16_t>(p, nrb, st);
}

}  // namespace msa
