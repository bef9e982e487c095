// msa_tiles.hip -- query rows in groups of 32 per wave on
// v_mfma_f32_32x32x16 (gfx950).
//
// Two kernels of the prefill-shaped path (fw-ai/minimax-kernels README,
// intro: a selected KV block is loaded once and every query that selected it
// is processed against it):
//   k_units  KV-outer units, 4 waves (pieces of up to 128 query rows). A unit
//            (window) is up to Tu tokens that picked block b of KV head g
//            outside their tile's chain; its rows are the tokens x the G
//            query heads of g. The block is staged once in LDS per sequence
//            and every piece is multiplied against it, writing one
//            normalised bf16/fp16 partial O and one LSE per (residual slot,
//            head).
//   k_tiles  8 waves, one tile of up to 256 query rows per item: the chain
//            (blocks picked by every token of the tile) streams through a
//            ring of LDS chunk slots while the tile's rows stay in
//            registers; the unit partials of the tile's residual slots are
//            then merged by their LSE and the final O and LSE are written
//            (the combine of the pages' design, fused into the tile's
//            epilogue).
//
// Each wave owns 32 query rows. Scores are computed transposed,
// S^T = K Q^T, so that the D fragment of a lane holds 16 keys of one query
// row; those probabilities are the B operand of O^T = V^T P^T as they stand.
// The V^T operand is read from the row-major LDS tile with the transposing
// ds_read_b64_tr_b16, so no register shuffles are needed.
//
// MFMA 32x32x16 fragment layout (lane l, h = l / 32, c = l % 32):
//   A: lane holds A[m = c][k = 8h + e], e = 0..7
//   B: lane holds B[k = 8h + e][n = c]
//   D: lane holds D[m = 8(j/4) + 4h + (j%4)][n = c], j = 0..15
// QK k-step s (0..7) covers head dims 16s .. 16s+15 (lane: 16s + 8h + e).
// PV k-step s' (0..1) of a 32-key chunk covers keys 16s' .. 16s'+15, with
// key(s', 8h + e) = 16s' + 8(e/4) + 4h + (e%4), which is where the score
// accumulator already holds them. O^T d-tile t (0..3) covers d = 32t + m.
//
// LDS tiles of 32 keys x 128 dims (16-bit) are stored row-major with the
// 16-byte pieces of row r XOR-swizzled (K tiles by r & 15, V tiles by
// 4 (r & 3)), which keeps the K-operand reads (one row per lane) and the
// transposing V reads conflict-light.
#include <limits.h>

#include <type_traits>

#include "msa_device.hpp"
#include "msa_index_dev.hpp"
#include "msa_internal.hpp"

namespace msa {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// c + a.lo * b.lo + a.hi * b.hi for two packed 16-bit values of T, in fp32
// (v_dot2_f32_bf16 / v_dot2_f32_f16). With b = (w, 0) or (0, w) it scales one
// element of a packed pair and accumulates it in a single instruction.
template <typename T>
struct Dot2;

template <>
struct Dot2<bf16_t> {
  typedef __bf16 t2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float run(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(t2, a), __builtin_bit_cast(t2, b), c, false);
  }
};

template <>
struct Dot2<f16_t> {
  typedef _Float16 t2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float run(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(t2, a), __builtin_bit_cast(t2, b), c, false);
  }
};

template <typename T>
struct Mma32;

template <>
struct Mma32<bf16_t> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};

template <>
struct Mma32<f16_t> {
  static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
};

constexpr int kChunkU4 = 512;       // one 32-key tile of K or V (16-bit): 8 KB
constexpr int kSlotU4 = 1024;       // one ring slot: the K tile, then the V tile
constexpr int kRing = 4;            // ring slots (bf16/fp16 caches)
constexpr int kUnitWindow = kUnitWindowTokens;
constexpr float kRescale32 = 8.0f;  // lazy rescale threshold (powers of two)


// Workgroup barrier that orders LDS accesses (compiler level) without the
// vmcnt(0) a release fence would add: the ring's direct-to-LDS loads are
// waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier of the tile kernel's chunk loop: every LDS read the loop issues
// is consumed within its iteration (or, for the next iteration's first V
// fragments, reads a slot no load overwrites before the following
// iteration), so no LDS wait is needed before it.
__device__ __forceinline__ void loop_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Swizzled 16-byte pieces of a 32 x 128 16-bit tile (row = key). The K tile
// XORs the piece index with row & 15: a K-operand read has lane c reading
// row c, so 16 consecutive lanes hit 16 different pieces. The V tile XORs it
// with 4 (row & 3): a transposing read has 32 lanes reading 4 rows x 4
// pieces of one d-tile, which then land on 16 different pieces.
__device__ __forceinline__ int pieceK(int row, int lc) { return row * 16 + (lc ^ (row & 15)); }
__device__ __forceinline__ int pieceV(int row, int lc) { return row * 16 + (lc ^ ((row & 3) << 2)); }

// ---------------------------------------------------------------------------
// the wave's 32 query rows
// ---------------------------------------------------------------------------
struct Rows32 {
  u32x4 qb[8];   // Q^T B fragments: k-step s holds dims 16s + 8h .. +7 of row c
  f32x16 o[4];   // O^T accumulators: d-tile t, element j -> d = 32t + 8(j/4) + 4h + (j%4)
  float m;       // running reference max of the row (log2 units)
  float l;       // this lane's share of the row sum
  int pos;       // causal position (INT_MAX when not causal or padding)
  int seq;       // owning sequence (-1: padding row)
};

__device__ __forceinline__ void rows_reset(Rows32& rt) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) rt.o[t][j] = 0.f;
  rt.m = -INFINITY;
  rt.l = 0.f;
}

__device__ __forceinline__ void rows_load_q(Rows32& rt, const Params& p, int tok, int head, int h) {
  if (tok < 0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) rt.qb[s] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const uint16_t* base = (const uint16_t*)p.q + ((size_t)tok * p.Hq + head) * kD + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) rt.qb[s] = *(const u32x4*)(base + 16 * s);
}

// The three stages of one 32-key chunk staged in LDS (sK: K tile, sV: V
// tile). rows_scores: S^T = K Q^T. rows_probs: online-softmax step (lazy
// rescale) giving the P^T B fragments; keys at or beyond lim, keys after a
// row's causal position and rows of another sequence are removed by select
// when `mask` is set (the caller clears it only for chunks fully visible to
// every row). It moves a row's reference max only when the chunk's max
// exceeds it by more than 2^kRescale32 and returns the factor the
// accumulators must be scaled by (1 when it did not move); the row sum is
// already scaled. rows_pv: O^T += V^T P^T.
template <typename CT>
__device__ __forceinline__ f32x16 rows_scores(const Rows32& rt, const u32x4* sK) {
  const int lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
  f32x16 sa;
#pragma unroll
  for (int j = 0; j < 16; ++j) sa[j] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) sa = Mma32<CT>::run(sK[pieceK(c, 2 * s + h)], rt.qb[s], sa);
  return sa;
}

template <typename CT>
__device__ __forceinline__ float rows_probs(Rows32& rt, f32x16 sa, int key0, int lim, int run_seq, bool mask,
                                            float sl2, u32x4 (&pb)[2]) {
  if (mask) {
    // key (key0 + 4h + the element's offset) is visible iff it is <= bound
    const int h = (threadIdx.x & 63) >> 5;
    const int bound = rt.seq == run_seq ? min(rt.pos, lim - 1) : -1;
    const int rel = bound - key0 - 4 * h;
#pragma unroll
    for (int j = 0; j < 16; ++j) sa[j] = (8 * (j >> 2) + (j & 3)) <= rel ? sa[j] : -INFINITY;
  }
  // the row max of the raw scores; sl2 > 0 commutes with max
  float cmax = sa[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) cmax = fmaxf(cmax, sa[j]);
  {
    // with the other half-wave's value (lane l ^ 32): the swap leaves one of
    // the two in each output, so their max is the pair's max in every lane
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cmax), __float_as_uint(cmax), false, false);
    cmax = __builtin_amdgcn_fmed3f(__uint_as_float(sw[0]), __uint_as_float(sw[1]), INFINITY) * sl2;
  }
  const float m_new = cmax > rt.m + kRescale32 ? cmax : rt.m;
  const float alpha = m_new == rt.m ? 1.f : exp2f(rt.m - m_new);  // 0 when the old max was -inf
  rt.m = m_new;
  const float nmu = (m_new == -INFINITY) ? 0.f : -m_new;
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * i], sl2, nmu));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * i + 1], sl2, nmu));
    pb[i >> 2][i & 3] = pack2<CT>(p0, p1);
    ls += p0 + p1;  // fp32 sum of the unrounded probabilities (the LSE needs it)
  }
  rt.l = __builtin_fmaf(rt.l, alpha, ls);
  return alpha;
}

__device__ __forceinline__ void rows_rescale(Rows32& rt, float alpha) {
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) rt.o[t] *= alpha;
  }
}

// V^T fragments by transposing reads: lane (h, c) receives V[key][32t + c]
// for the four keys 16s' + 8r + 4h + i (i = 0..3); its source lanes read 8
// bytes each at row 16s' + 8r + 4h + i (i = (l >> 2) & 3), logical piece
// 4t + 2((l >> 4) & 1) + ((l & 3) >> 1), half l & 1. With the V swizzle the
// physical piece is 4(t ^ i) + the low two bits.
template <typename CT>
__device__ __forceinline__ void rows_pv(Rows32& rt, const u32x4 (&pb)[2], const u32x4* sV) {
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int i4 = (lane >> 2) & 3;
  const int rsub = 4 * h + i4;                                 // 0..7
  const int psub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // 0..3
  const int half = 8 * (lane & 1);
  const char* vbytes = (const char*)sV;
#pragma unroll
  for (int sp = 0; sp < 2; ++sp) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 a;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 16 * sp + 8 * r + rsub;
        const int off = row * 256 + ((4 * (t ^ i4) + psub) << 4) + half;
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbytes + off));
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        a[2 * r] = w[0];
        a[2 * r + 1] = w[1];
      }
      rt.o[t] = Mma32<CT>::run(a, pb[sp], rt.o[t]);
    }
  }
}

// One chunk, the three stages in order.
template <typename CT>
__device__ __forceinline__ void rows_chunk(Rows32& rt, const u32x4* sK, const u32x4* sV, int key0, int lim,
                                           int run_seq, bool mask, float sl2) {
  const f32x16 sa = rows_scores<CT>(rt, sK);
  u32x4 pb[2];
  rows_rescale(rt, rows_probs<CT>(rt, sa, key0, lim, run_seq, mask, sl2, pb));
  rows_pv<CT>(rt, pb, sV);
}

// V^T fragment of d-tile t and key step sp of a staged V tile (transposing
// reads): lane (h, c) receives V[key][32t + c] for the four keys
// 16sp + 8r + 4h + i; its source lanes read 8 bytes each at row
// 16sp + 8r + 4h + i (i = (l >> 2) & 3), logical piece 4t + 2((l >> 4) & 1)
// + ((l & 3) >> 1), half l & 1. With the V swizzle the physical piece is
// 4(t ^ i) + the low two bits.
__device__ __forceinline__ u32x4 vfrag_at(const char* vtile, int t, int sp, int lane = threadIdx.x & 63) {
  const int h = lane >> 5;
  const int i4 = (lane >> 2) & 3;
  const int rsub = 4 * h + i4;
  const int psub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int half = 8 * (lane & 1);
  u32x4 a;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 16 * sp + 8 * r + rsub;
    const int off = row * 256 + ((4 * (t ^ i4) + psub) << 4) + half;
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtile + off)));
    a[2 * r] = w[0];
    a[2 * r + 1] = w[1];
  }
  return a;
}

// A whole staged block against the rows at once (the unit kernel): the first
// NQ chunks of the block at sblk (chunk q: K at q * kSlotU4, V kChunkU4
// after it), chunk q's keys [key0[q], lim[q]) present, masked when bit q of
// mmask is set (as in rows_probs; a unit's rows all belong to the staged
// block's sequence). The scores of all NQ chunks are formed first (NQ
// independent accumulation chains), then one softmax over the row's keys of
// the block -- its maximum is final, so nothing is ever rescaled -- then
// O^T = V^T P^T over the NQ chunks. The row state must be the reset one;
// rt.o is written here.
template <typename CT, int NQ>
__device__ __forceinline__ void rows_block(Rows32& rt, const u32x4* sblk, const int (&key0)[4], const int (&lim)[4],
                                           unsigned mmask, float sl2) {
  // the lane index, opaque to the compiler: the LDS addresses derived from it
  // are formed here, once per call, instead of being held in registers across
  // the whole kernel
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int h = lane >> 5, c = lane & 31;
  f32x16 sa[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int j = 0; j < 16; ++j) sa[q][j] = 0.f;
  // k-step s of every chunk: its K fragments are read one stage ahead
  u32x4 kf[2][NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) kf[0][q] = sblk[q * kSlotU4 + pieceK(c, h)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 1 < 8) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) kf[(s + 1) & 1][q] = sblk[q * kSlotU4 + pieceK(c, 2 * (s + 1) + h)];
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) sa[q] = Mma32<CT>::run(kf[s & 1][q], rt.qb[s], sa[q]);
    // the reads first, then the products
    if (s + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, NQ, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NQ, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  float cmax = -INFINITY;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if ((mmask >> q) & 1u) {
      // key (key0 + 4h + the element's offset) is visible iff it is <= bound
      const int rel = min(rt.pos, lim[q] - 1) - key0[q] - 4 * h;
#pragma unroll
      for (int j = 0; j < 16; ++j) sa[q][j] = (8 * (j >> 2) + (j & 3)) <= rel ? sa[q][j] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) cmax = fmaxf(cmax, sa[q][j]);
  }
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cmax), __float_as_uint(cmax), false, false);
    cmax = __builtin_amdgcn_fmed3f(__uint_as_float(sw[0]), __uint_as_float(sw[1]), INFINITY) * sl2;
  }
  const float nmu = cmax == -INFINITY ? 0.f : -cmax;
  u32x4 pb[NQ][2];
  float ls = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[q][2 * i], sl2, nmu));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[q][2 * i + 1], sl2, nmu));
      pb[q][i >> 2][i & 3] = pack2<CT>(p0, p1);
      ls += p0 + p1;
    }
  rt.m = cmax;
  rt.l = ls;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) rt.o[t][j] = 0.f;
  // key step (q, sp): the four V^T fragments of the next step are read
  // while this step's four products run
  u32x4 vf[2][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) vf[0][t] = vfrag_at((const char*)(sblk + kChunkU4), t, 0, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 2 * NQ; ++k) {
    if (k + 1 < 2 * NQ) {
      const char* vn = (const char*)(sblk + ((k + 1) >> 1) * kSlotU4 + kChunkU4);
#pragma unroll
      for (int t = 0; t < 4; ++t) vf[(k + 1) & 1][t] = vfrag_at(vn, t, (k + 1) & 1, lane);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) rt.o[t] = Mma32<CT>::run(vf[k & 1][t], pb[k >> 1][k & 1], rt.o[t]);
    if (k + 1 < 2 * NQ) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The max instructions as they stand. fmaxf would first quiet a possible
// signalling NaN in each operand that does not come from arithmetic the
// compiler can see (matrix-core results, lane swaps), one instruction per
// operand; scores hold no NaN (masked ones are -inf), so the chunk step
// takes the hardware's max directly.
__device__ __forceinline__ float hw_max(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float hw_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Byte offset, within a K tile, of the fragment a lane reads for product
// st of a chunk: 16 pieceK(c, 2 st + h) = 256 c + 16 ((2 st + h) ^ (c & 15)).
// The swizzle leaves st in bits 5-7 of the offset, where it enters by XOR:
// the offset is that of product 0 XOR 32 st. Bits 5-7 of a tile base that
// is a multiple of 256 bytes are zero, so the XOR can be applied to base +
// offset: one register per lane, one add per chunk and one XOR per read.
__device__ __forceinline__ uint32_t k_lane_offset0() {
  const int lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
  return 16u * (uint32_t)pieceK(c, h);
}

// One iteration of the tile kernel's chunk pipeline, scheduled by hand:
// O^T += V(prev)^T P(prev)^T, sn = S of the next chunk, and the softmax step
// of sc (this chunk's scores) giving pn. The work is cut into eight stages:
// stage i holds the P V product i, the Q K product i - 1, the LDS reads of
// the products two stages later and a slice of the vector work;
// sched_barrier keeps the compiler from regrouping them, so the vector ALU
// runs while the matrix core is busy and every LDS read has two stages to
// land. The first two V fragments (vpre) were read by the previous
// iteration, before the barrier; this one reads those of the current
// chunk's V for the next iteration (vnext). The K reads start one stage
// after the barrier that makes the next chunk visible. Returns the
// accumulator rescale factor (see rows_probs).
template <typename CT, bool kMask>
__device__ __forceinline__ float tile_iter(Rows32& rt, const f32x16& sc, const u32x4 (&pp)[2], const char* vprev,
                                           const u32x4 (&vpre)[2], const char* vcur, const u32x4* knext,
                                           uint32_t koff0, int key0, int lim, float sl2, f32x16& sn,
                                           u32x4 (&pn)[2], u32x4 (&vnext)[2]) {
  const int h = (threadIdx.x & 63) >> 5;
  // knext is a slot of a ring that starts on a 256-byte boundary
  const uint32_t ka0 = lds_addr(knext) + koff0;
  auto kfrag = [&](int st) { return *(const lds_u32x4*)(uintptr_t)(ka0 ^ (32u * st)); };

  f32x16 sa = sc;
  u32x4 va[8], ka[8];
  va[0] = vpre[0];
  va[1] = vpre[1];
  ka[0] = kfrag(0);
#pragma unroll
  for (int j = 0; j < 16; ++j) sn[j] = 0.f;
  float cmax = 0.f, alpha = 1.f, nmu = 0.f, ls = 0.f;
  int rel = 0;
  if (kMask) {
    const int bound = min(rt.pos, lim - 1);
    rel = bound - key0 - 4 * h;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i + 2 < 8) va[i + 2] = vfrag_at(vprev, (i + 2) & 3, (i + 2) >> 2);
    if (i + 1 < 8) ka[i + 1] = kfrag(i + 1);
    rt.o[i & 3] = Mma32<CT>::run(va[i], pp[i >> 2], rt.o[i & 3]);
    if (i > 0) sn = Mma32<CT>::run(ka[i - 1], rt.qb[i - 1], sn);
    if (i == 0) {
      // masking, then the row max of the raw scores (sl2 > 0 commutes with max)
      if (kMask) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sa[j] = (8 * (j >> 2) + (j & 3)) <= rel ? sa[j] : -INFINITY;
      }
      cmax = hw_max3(hw_max3(hw_max3(sa[0], sa[1], sa[2]), sa[3], sa[4]), sa[5], sa[6]);
    } else if (i == 1) {
      cmax = hw_max3(hw_max3(hw_max3(cmax, sa[7], sa[8]), sa[9], sa[10]), sa[11], sa[12]);
      cmax = hw_max(hw_max3(cmax, sa[13], sa[14]), sa[15]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cmax), __float_as_uint(cmax), false, false);
      cmax = hw_max(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
      const float m_new = cmax > rt.m + kRescale32 ? cmax : rt.m;
      // a new maximum exceeds the old by more than 2^kRescale32, so the
      // factor is below 2^-8: the hardware exponential (results below the
      // normal range flush to zero) is exact enough for it
      alpha = m_new == rt.m ? 1.f : __builtin_amdgcn_exp2f(rt.m - m_new);
      rt.m = m_new;
      nmu = (m_new == -INFINITY) ? 0.f : -m_new;
    } else {
      // pairs of probabilities: stage 2 takes pairs 0-1, stage 3 pair 2, ...
      const int q0 = i == 2 ? 0 : (i == 3 ? 2 : (i == 4 ? 3 : (i == 5 ? 4 : (i == 6 ? 6 : 7))));
      const int q1 = i == 2 ? 2 : (i == 3 ? 3 : (i == 4 ? 4 : (i == 5 ? 6 : (i == 6 ? 7 : 8))));
#pragma unroll
      for (int q = q0; q < q1; ++q) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * q], sl2, nmu));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * q + 1], sl2, nmu));
        pn[q >> 2][q & 3] = pack2<CT>(p0, p1);
        ls = q == 0 ? p0 + p1 : ls + (p0 + p1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  sn = Mma32<CT>::run(ka[7], rt.qb[7], sn);
  vnext[0] = vfrag_at(vcur, 0, 0);
  vnext[1] = vfrag_at(vcur, 1, 0);
  // used here, so that the vector work is not sunk past the caller's
  // rarely taken rescale branch
  asm volatile("" ::"v"(pn[0]), "v"(pn[1]), "v"(ls));
  rt.l = __builtin_fmaf(rt.l, alpha, ls);
  return alpha;
}

// Final row state: total sum over the lane pair, reference max, log2 LSE.
__device__ __forceinline__ float rows_total(const Rows32& rt) { return rt.l + __shfl_xor(rt.l, 32, 64); }

// 16-bit row stores/loads in the D layout: for d-tile t and group a the lane
// holds d = 32t + 8a + 4h + (0..3), i.e. 8 contiguous bytes.
//
// Stores pair the two half-waves first: for groups a = 2u and 2u + 1,
// v_permlane32_swap hands the upper half's group-2u words to the lower half
// and the lower half's group-(2u+1) words to the upper half, so lane (h, c)
// then holds the 16 contiguous bytes d = 32t + 16u + 8h + (0..7) of its row,
// i.e. 16-byte chunk 4t + 2u + h. The same swap undoes it after a load.
template <typename CT>
__device__ __forceinline__ u32x4 paired16(const Rows32& rt, int t, int u, float scale) {
  const uint32_t x0 = pack2<CT>(rt.o[t][8 * u] * scale, rt.o[t][8 * u + 1] * scale);
  const uint32_t x1 = pack2<CT>(rt.o[t][8 * u + 2] * scale, rt.o[t][8 * u + 3] * scale);
  const uint32_t y0 = pack2<CT>(rt.o[t][8 * u + 4] * scale, rt.o[t][8 * u + 5] * scale);
  const uint32_t y1 = pack2<CT>(rt.o[t][8 * u + 6] * scale, rt.o[t][8 * u + 7] * scale);
  // upper lanes of the first operand <-> lower lanes of the second
  const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// a row-major 16-bit row of 128
template <typename CT>
__device__ __forceinline__ void store_row16(uint16_t* row, const Rows32& rt, float scale) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) *(u32x4*)(row + 32 * t + 16 * u + 8 * h) = paired16<CT>(rt, t, u, scale);
}

// Residual partials are stored in blocks of 32 rows (row = residual position
// x G + query head within the group): for each 16-byte chunk k of a row
// (d = 8k .. 8k + 7) the block holds the chunk of its 32 rows side by side,
// row r's chunk k at byte (r >> 5) * 8192 + k * 512 + (r & 31) * 16. A wave
// storing 32 consecutive rows writes 512 contiguous bytes per chunk (two runs
// when its rows cross a block), and a residual slot's G query heads share
// one line per chunk when the merge reads them back.
__device__ __forceinline__ size_t part_offset(size_t row) { return (row >> 5) * 8192 + (row & 31) * 16; }

// base: the row's part_offset plus 512 h (chunk 4t + 2u + h at base + (4t + 2u) * 512)
template <typename CT>
__device__ __forceinline__ void store_part(char* base, const Rows32& rt, float scale) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) *(u32x4*)(base + (4 * t + 2 * u) * 512) = paired16<CT>(rt, t, u, scale);
}

// ---------------------------------------------------------------------------
// chunk staging
// ---------------------------------------------------------------------------
// 16-bit caches: direct-to-LDS 16-byte buffer loads. One chunk is 32 key
// rows of K and of V (8 KB each); each thread issues two loads per tensor.
// Lane i of wave w's j-th load fills LDS piece (2w + j) * 64 + i; the piece
// of global memory it reads (a per-lane constant, DmaLane) is chosen so that
// LDS holds the swizzled layout. The chunk's address and extent go into the
// buffer descriptor (scalar registers): rows at or beyond `nrows` (keys past
// the used length, whose cache rows may hold anything) and absent chunks
// (off < 0) fall outside the descriptor's range, and out-of-range buffer
// loads return zeros -- a masked probability is exactly zero, but 0 * NaN is
// not.

struct DmaLane {
  int k0, k1, v0, v1;  // byte offsets within a chunk of the lane's two K and two V loads
  __device__ __forceinline__ void init() {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pc0 = (2 * wave) * 64 + lane, pc1 = pc0 + 64;
    const int r0 = pc0 >> 4, f0 = pc0 & 15, r1 = pc1 >> 4, f1 = pc1 & 15;
    k0 = r0 * 256 + ((f0 ^ (r0 & 15)) << 4);
    k1 = r1 * 256 + ((f1 ^ (r1 & 15)) << 4);
    v0 = r0 * 256 + ((f0 ^ ((r0 & 3) << 2)) << 4);
    v1 = r1 * 256 + ((f1 ^ ((r1 & 3) << 2)) << 4);
  }
};

// off and nrows must be the same in every lane of the wave
// wave-uniform value, held in a scalar register
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The tile kernel's 512 threads: one K piece and one V piece each per chunk.
struct DmaLane512 {
  int k0, v0;
  __device__ __forceinline__ void init() {
    const int pc = threadIdx.x;  // 0..511
    const int r = pc >> 4, f = pc & 15;
    k0 = r * 256 + ((f ^ (r & 15)) << 4);
    v0 = r * 256 + ((f ^ ((r & 3) << 2)) << 4);
  }
};




// chunk into the ring slot at LDS byte address slot (K tile, then V tile)
__device__ __forceinline__ void issue_chunk16_512(const void* kb, const void* vb, int64_t off_any, int nrows_any,
                                                  const DmaLane512& dl, uint32_t slot) {
  const int wave = threadIdx.x >> 6;
  const int64_t off = uniform64(off_any);
  const int nrows = __builtin_amdgcn_readfirstlane(nrows_any);
  const bool present = off >= 0 && nrows > 0;
  const int64_t ob = present ? off * 2 : 0;
  const int nrec = present ? min(nrows, 32) * 256 : 0;
  dma16(make_rsrc((const char*)kb + ob, nrec), slot + 1024 * wave, dl.k0);
  dma16(make_rsrc((const char*)vb + ob, nrec), slot + 16 * kChunkU4 + 1024 * wave, dl.v0);
}

__device__ __forceinline__ void issue_chunk16(const void* kb, const void* vb, int64_t off_any, int nrows_any,
                                              const DmaLane& dl, u32x4* sK, u32x4* sV) {
  const int wave = threadIdx.x >> 6;
  const int64_t off = uniform64(off_any);
  const int nrows = __builtin_amdgcn_readfirstlane(nrows_any);
  const bool present = off >= 0 && nrows > 0;
  const int64_t ob = present ? off * 2 : 0;
  const int nrec = present ? min(nrows, 32) * 256 : 0;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)kb + ob), (short)0, nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)vb + ob), (short)0, nrec, kRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(sK + (2 * wave) * 64), 16, dl.k0, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(sK + (2 * wave + 1) * 64), 16, dl.k1, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(sV + (2 * wave) * 64), 16, dl.v0, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(sV + (2 * wave + 1) * 64), 16, dl.v1, 0, 0, 0);
}

// e4m3fn caches: each thread loads 16 raw bytes of K and of V (16 dims of
// one key row) into registers, then widens them exactly into two swizzled
// 16-bit pieces.
struct Raw8 {
  u32x4 k, v;
};

__device__ __forceinline__ Raw8 load_chunk8(const uint8_t* kb, const uint8_t* vb, int64_t off, int nrows,
                                            const void* zero) {
  const int row = threadIdx.x >> 3, lc = threadIdx.x & 7;
  const int64_t e = (int64_t)row * kD + 16 * lc;
  const bool ok = off >= 0 && row < nrows;
  Raw8 r;
  r.k = ok ? *(const u32x4*)(kb + off + e) : *(const u32x4*)((const char*)zero + 16 * (threadIdx.x & 63));
  r.v = ok ? *(const u32x4*)(vb + off + e) : *(const u32x4*)((const char*)zero + 16 * (threadIdx.x & 63));
  return r;
}

template <typename CT>
__device__ __forceinline__ void store_chunk8(const Raw8& r, u32x4* sK, u32x4* sV) {
  const int row = threadIdx.x >> 3, lc = threadIdx.x & 7;
  sK[pieceK(row, 2 * lc)] = widen8<CT>(u32x2{r.k[0], r.k[1]});
  sK[pieceK(row, 2 * lc + 1)] = widen8<CT>(u32x2{r.k[2], r.k[3]});
  sV[pieceV(row, 2 * lc)] = widen8<CT>(u32x2{r.v[0], r.v[1]});
  sV[pieceV(row, 2 * lc + 1)] = widen8<CT>(u32x2{r.v[2], r.v[3]});
}

// MXFP4 caches: each thread loads the 8 code bytes of the same 16 dims of
// one key row and the row's scale word, then widens them (the scale of dims
// 16 lc .. 16 lc + 15 is byte lc / 2) into the same two swizzled pieces.
// off is the chunk's element offset: its codes start at off / 2 bytes, its
// scales at off / 32.
struct Raw4 {
  u32x2 k, v;
  uint32_t ks, vs;
};

__device__ __forceinline__ Raw4 load_chunk4(const Params& p, int64_t off, int nrows) {
  const int row = threadIdx.x >> 3, lc = threadIdx.x & 7;
  const bool ok = off >= 0 && row < nrows;
  const int64_t ec = (off >> 1) + (int64_t)row * 64 + 8 * lc, es = (off >> 5) + (int64_t)row * 4;
  const char* zero = (const char*)p.zero_page + 8 * (threadIdx.x & 63);
  Raw4 r;
  r.k = ok ? *(const u32x2*)((const uint8_t*)p.k + ec) : *(const u32x2*)zero;
  r.v = ok ? *(const u32x2*)((const uint8_t*)p.v + ec) : *(const u32x2*)zero;
  r.ks = ok ? *(const uint32_t*)(p.k_scale + es) : 0u;  // absent rows: zero codes
  r.vs = ok ? *(const uint32_t*)(p.v_scale + es) : 0u;
  return r;
}

template <typename CT>
__device__ __forceinline__ void store_chunk4(const Raw4& r, u32x4* sK, u32x4* sV) {
  static_assert(std::is_same<CT, bf16_t>::value, "MXFP4 caches widen to bf16");
  const int row = threadIdx.x >> 3, lc = threadIdx.x & 7;
  const uint32_t sh = 8 * (lc >> 1);
  const float sk = e8m0_scale((r.ks >> sh) & 0xFFu), sv = e8m0_scale((r.vs >> sh) & 0xFFu);
  sK[pieceK(row, 2 * lc)] = widen_fp4(r.k[0], sk);
  sK[pieceK(row, 2 * lc + 1)] = widen_fp4(r.k[1], sk);
  sV[pieceV(row, 2 * lc)] = widen_fp4(r.v[0], sv);
  sV[pieceV(row, 2 * lc + 1)] = widen_fp4(r.v[1], sv);
}

// ---------------------------------------------------------------------------
// Tokens with ranks [rank0, rank0 + n) among the set bits of row r (one
// wave): the word holding rank0 is found by two rounds of sampled loads of
// the row's exclusive popcount prefix, then consecutive words are scanned
// 64 at a time, each lane expanding its own word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unit_tokens(const Params& p, int r, int rank0, int n, int* s_tok) {
  const int lane = threadIdx.x & 63;
  const uint32_t* pre = p.wordpre + (size_t)r * p.W;
  const uint32_t* bits = p.wordbits + (size_t)r * p.W;
  int lo = 0, hi = p.W;  // the word is the largest w with pre[w] <= rank0
  while (hi - lo > 64) {
    const int stride = (hi - lo + 63) / 64;
    const int w = lo + lane * stride;
    const bool le = w < hi && (int)pre[w] <= rank0;
    const int cnt = __popcll(__ballot(le));
    lo = lo + (cnt - 1) * stride;
    hi = min(lo + stride, hi);
  }
  {
    const int w = lo + lane;
    const bool le = w < hi && (int)pre[w] <= rank0;
    lo = lo + __popcll(__ballot(le)) - 1;
  }
  for (int wb = lo; wb < p.W; wb += 64) {
    const int w = wb + lane;
    uint32_t x = 0u;
    int rk = 0;
    if (w < p.W) {
      x = bits[w];
      rk = (int)pre[w];
    }
    while (x) {
      const int bit = __ffs(x) - 1;
      x &= x - 1u;
      if (rk >= rank0 && rk < rank0 + n) s_tok[rk - rank0] = w * 32 + bit;
      ++rk;
    }
    if (!__any(w < p.W && rk < rank0 + n)) break;  // every lane is past the unit's last rank
  }
}

// ---------------------------------------------------------------------------
// XCD-aware work queue. Workgroups of a launch are dispatched round-robin
// over the 8 XCDs, each with its own L2, so workgroup i runs on XCD i % 8.
// The item space [0, total) is cut into 8 contiguous ranges, one per XCD;
// neighbouring items (tiles of one KV head and nearby tokens, units of one
// block) share KV blocks, which then stay in that XCD's L2. A workgroup's
// first item is fixed by its rank on the XCD, later ones come from the XCD's
// own counter. Returns the item, or -1 when the range is exhausted.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

// Returning atomic add whose result is waited for explicitly (wait_vmcnt,
// then settle()): the compiler does not see it as a load in flight.
__device__ __forceinline__ int atomic_add_nowait(int32_t* ptr, int val) {
  int r;
  asm volatile("global_atomic_add %0, %1, %2, off sc0" : "=v"(r) : "v"(ptr), "v"(val) : "memory");
  return r;
}
__device__ __forceinline__ int settle(int x) {
  asm volatile("" : "+v"(x));
  return x;
}


struct XcdQueue {
  int lo, hi, rank, nwg;
  int32_t* head;
  __device__ __forceinline__ void init(int total, int32_t* heads) {
    const int x = blockIdx.x % kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    lo = min(x * per, total);
    hi = min(lo + per, total);
    rank = blockIdx.x / kXcds;
    nwg = (gridDim.x - x + kXcds - 1) / kXcds;  // workgroups on this XCD
    head = heads + x;
  }
  __device__ __forceinline__ int next(bool first) {
    const int i = lo + (first ? rank : nwg + atomicAdd(head, 1));
    return i < hi ? i : -1;
  }
};

// ---------------------------------------------------------------------------
// k_units: KV-outer units, KV-stationary. Work item = one window of the
// residual order: up to Tu consecutive entries (tokens) of one row (block b,
// KV head g). The window is cut into pieces -- runs of tokens of one
// sequence, at most 128 / G tokens each, i.e. at most 128 query rows -- and
// the pieces are multiplied one after another against the block, which stays
// staged in LDS until the sequence or the row changes.
//
// Vector memory operations complete in issue order, and a wait for a load
// also waits for every store issued before it. So every load a piece needs is
// issued before the stores of the piece before it: the next piece's Q while
// the current one is multiplied; at the end of a piece, the next piece's block
// (when it changes) and, at the end of a window, the next window's first Q,
// both ahead of the current piece's partial stores. The next window's token
// list is built in a second LDS buffer at the end of the current window; its
// descriptor and tokens are loaded during the current window, and the work
// queue slot of the window after it is taken at the current window's start.
// ---------------------------------------------------------------------------
constexpr int kSeqLds = 256;  // cu_seqlens / used_kv_lens cached in LDS up to this many sequences
// vector memory instructions per lane of the partial stores of a piece
// (store_part: eight 16-byte stores, then the LSE)
constexpr int kUnitStoreOps = 9;
// buffer offset of a store to drop: past the end of any descriptor it meets
constexpr int kDropOff = 1 << 30;
// cache policy operand of the buffer builtins: the non-temporal hint
constexpr int kBufNT = 2;

__device__ __forceinline__ void load_q8(u32x4 (&qb)[8], const Params& p, int tok, int head, int h) {
  if (tok < 0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const uint16_t* base = (const uint16_t*)p.q + ((size_t)tok * p.Hq + head) * kD + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = *(const u32x4*)(base + 16 * s);
}

// The unit kernel's Q rows: every lane loads a row, a lane without a token
// that of token 0 (its results are never stored), so that each call is the
// same eight loads in every wave and no register is cleared while a load into
// it may be in flight.
__device__ __forceinline__ void load_q8_rows(u32x4 (&qb)[8], const Params& p, int tok, int head, int h) {
  const uint16_t* base = (const uint16_t*)p.q + ((size_t)max(tok, 0) * p.Hq + head) * kD + 8 * h;
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = *(const u32x4*)(base + 16 * s);
}

// chunk into LDS (K tile at byte address sK, V tile at sV) by the unit
// kernel's 256 threads, two 16-byte pieces of K and two of V per lane
__device__ __forceinline__ void issue_chunk16_256(const void* kb, const void* vb, int64_t off_any, int nrows_any,
                                                  const DmaLane& dl, uint32_t sK, uint32_t sV) {
  const int wave = threadIdx.x >> 6;
  const int64_t off = uniform64(off_any);
  const int nrows = __builtin_amdgcn_readfirstlane(nrows_any);
  const bool present = off >= 0 && nrows > 0;
  const int64_t ob = present ? off * 2 : 0;
  const int nrec = present ? min(nrows, 32) * 256 : 0;
  const i32x4v rk = make_rsrc((const char*)kb + ob, nrec), rv = make_rsrc((const char*)vb + ob, nrec);
  dma16(rk, sK + 2048 * wave, dl.k0);
  dma16(rk, sK + 2048 * wave + 1024, dl.k1);
  dma16(rv, sV + 2048 * wave, dl.v0);
  dma16(rv, sV + 2048 * wave + 1024, dl.v1);
}

template <typename CT, typename KVT>
__global__ __launch_bounds__(256, 2) void k_units(Params p) {
  constexpr bool kFp8 = sizeof(KVT) == 1;  // e4m3fn or MXFP4: staged through registers
  constexpr bool kFp4 = std::is_same<KVT, mxfp4_t>::value;
  __shared__ u32x4 s_blk[kRing * kSlotU4];  // the staged block: chunk q at q * kSlotU4 (K), + kChunkU4 (V)
  __shared__ int s_tok[2][kUnitWindow];     // token lists of two consecutive windows
  __shared__ int s_seq[2][kUnitWindow];
  __shared__ int64_t s_cu[kSeqLds + 1];
  __shared__ int s_used[kSeqLds];
  __shared__ int s_item[2];
  const int nU = p.counters[kCntUnits];
  if (nU == 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int G = p.G, Hkv = p.Hkv, K = p.K;
  const int Tp = max(1, 128 / G);  // tokens per piece
  const bool seq_lds = p.B <= kSeqLds;
  if (seq_lds) {
    for (int i = tid; i <= p.B; i += 256) s_cu[i] = p.cu[i];
    for (int i = tid; i < p.B; i += 256) s_used[i] = p.used[i];
  }
  // sequence bounds from LDS, or from global memory for large batches (never
  // through a generic pointer: a flat load is counted with the vector memory
  // operations, and waiting for it would wait for every load and store in
  // flight)
  auto cu_at = [&](int i) -> int64_t {
    if (seq_lds) {
      int64_t v = s_cu[i];
      asm volatile("" : "+v"(v));  // keeps the two loads apart (else merged into one flat load)
      return v;
    }
    return p.cu[i];
  };
  // the same at a uniform index (the piece's sequence), by scalar loads
  auto cu_u = [&](int i) { return sload64(p.cu + __builtin_amdgcn_readfirstlane(i)); };
  auto used_u = [&](int i) { return sload32(p.used + __builtin_amdgcn_readfirstlane(i)); };
  auto seq_of_tok = [&](int64_t t) {  // as seq_of
    if (p.B <= 0 || t < cu_at(0)) return -1;
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_at(mid) <= t)
        lo = mid;
      else
        hi = mid;
    }
    return t < cu_at(lo + 1) ? lo : -1;
  };
  int st_s = -1, st_b = -1, st_g = -1;  // staged block (uniform)
  unsigned st_absent = 0u;              // bit q: chunk q of the staged block has no keys (page outside the pool)
  DmaLane dl;
  dl.init();
  XcdQueue wq;
  wq.init(nU, p.counters + kCntXcdU);
  const int64_t slots_per_tok = (int64_t)Hkv * K;
  // a window's tokens (two per thread) come from the materialised residual
  // order; otherwise from the row's bitmap words, and the window then writes
  // its own residual list entries
  const bool have_ent = p.ent_ready != 0;
  // (the residual order entries themselves; prepare() turns them into tokens,
  // so that nothing waits for these loads before then)
  auto load_tokens = [&](int4 wd, int (&tk)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      tk[i] = (have_ent && e < min(wd.w, p.Tu)) ? p.ent[wd.z + e] : -1;
    }
  };
  // token list and sequences of window wd into buffer bf (every thread calls
  // it; the caller synchronises before they are read)
  auto prepare = [&](int bf, int4 wd, const int (&tk)[2]) {
    const int r = wd.x, e0 = wd.z, n = min(wd.w, p.Tu);
    if (!have_ent) {
      const int b = r / Hkv, g = r - (r / Hkv) * Hkv;
      for (int i = tid; i < n; i += 256) s_tok[bf][i] = -1;
      __syncthreads();
      if (wave == 0) unit_tokens(p, r, wd.y, n, s_tok[bf]);
      __syncthreads();
      for (int idx = tid; idx < n * K; idx += 256) {
        const int tau = idx / K, k = idx - tau * K;
        if (s_tok[bf][tau] < 0) continue;
        const size_t slot = ((size_t)s_tok[bf][tau] * Hkv + g) * K + k;
        if (p.selected[slot] == b && p.slot_flag[slot] == 2) p.res_list[slot - k + p.res_rank[slot]] = e0 + tau;
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i;
      if (e < n) {
        const int tok = have_ent ? (tk[i] < 0 ? -1 : (int)(tk[i] / slots_per_tok)) : s_tok[bf][e];
        s_tok[bf][e] = tok;
        s_seq[bf][e] = tok >= 0 ? seq_of_tok(tok) : -1;
      }
    }
  };
  // pieces [a0, a1): a run of one sequence, at most Tp tokens
  auto piece_end = [&](int bf, int n, int a0) {
    const int sq = s_seq[bf][a0];
    const int lim = min(n, a0 + Tp);
    int e = a0 + 1;
    while (e < lim && s_seq[bf][e] == sq) ++e;
    return e;
  };
  const int rho = 32 * wave + c;
  const int hr = rho % G;
  auto row_token = [&](int bf, int a0, int a1) {  // the lane's token in piece [a0, a1), or -1
    const int tau = rho / G;
    return (a0 + tau < a1 && s_seq[bf][a0 + tau] >= 0) ? s_tok[bf][a0 + tau] : -1;
  };
  // the block (sequence s_run, block b, KV head g) into s_blk: 16-bit caches
  // by direct-to-LDS loads, waited for by the caller; e4m3fn caches through
  // registers, widened and written to LDS here
  auto stage = [&](int s_run_any, int b_any, int g_any) {
    // uniform: the page table reads below are scalar loads
    const int s_run = __builtin_amdgcn_readfirstlane(s_run_any);
    const int b = __builtin_amdgcn_readfirstlane(b_any), g = __builtin_amdgcn_readfirstlane(g_any);
    const int Leff = min(used_u(s_run), p.MP * p.P);
    // the page table entries of the four chunks in one load (lane q & 3
    // reads chunk q's), instead of four dependent round trips
    int pg = -1;
    {
      const int key0 = kBlk * b + 32 * (lane & 3);
      if (key0 < Leff) pg = p.block_tables[(size_t)s_run * p.MP + key0 / p.P];
    }
    int64_t offs[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int key0 = kBlk * b + 32 * q;
      const int page = __builtin_amdgcn_readlane(pg, q);
      offs[q] = (key0 >= Leff || page < 0 || page >= p.NP)
                    ? (int64_t)-1
                    : (((int64_t)page * p.Hkv + g) * p.P + (key0 % p.P)) * 128;
    }
    st_absent = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) st_absent |= offs[q] < 0 ? 1u << q : 0u;
    if constexpr (kFp4) {
      Raw4 raw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[q] = load_chunk4(p, offs[q], Leff - (kBlk * b + 32 * q));
#pragma unroll
      for (int q = 0; q < 4; ++q) store_chunk4<CT>(raw[q], s_blk + q * kSlotU4, s_blk + q * kSlotU4 + kChunkU4);
    } else if constexpr (kFp8) {
      Raw8 raw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        raw[q] = load_chunk8((const uint8_t*)p.k, (const uint8_t*)p.v, offs[q], Leff - (kBlk * b + 32 * q),
                             p.zero_page);
#pragma unroll
      for (int q = 0; q < 4; ++q) store_chunk8<CT>(raw[q], s_blk + q * kSlotU4, s_blk + q * kSlotU4 + kChunkU4);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        issue_chunk16_256(p.k, p.v, offs[q], Leff - (kBlk * b + 32 * q), dl, lds_addr(s_blk + q * kSlotU4),
                          lds_addr(s_blk + q * kSlotU4 + kChunkU4));
    }
    st_s = s_run;
    st_b = b;
    st_g = g;
  };

  // the first window, its token list, its first piece's Q and block
  if (tid == 0) s_item[0] = wq.next(true);
  __syncthreads();
  int u = __builtin_amdgcn_readfirstlane(s_item[0]);
  __syncthreads();
  if (u < 0) return;
  int4 wd = p.win_desc[u];
  int bf = 0;
  {
    int tk[2];
    load_tokens(wd, tk);
    if (tid == 0) s_item[0] = wq.next(false);
    prepare(0, wd, tk);
  }
  __syncthreads();
  int un = __builtin_amdgcn_readfirstlane(s_item[0]);  // the next window's item
  int n = min(wd.w, p.Tu);
  int a0 = 0, a1 = piece_end(0, n, 0);
  Rows32 rt;
  {
    const int b = wd.x / Hkv, g = wd.x - (wd.x / Hkv) * Hkv;
    load_q8_rows(rt.qb, p, row_token(0, a0, a1), g * G + hr, h);
    if (s_seq[0][0] >= 0) stage(s_seq[0][0], b, g);
    wait_vmcnt<0>();
    __syncthreads();
  }

  for (;;) {
    const int r = wd.x, e0 = wd.z;
    const int b = r / Hkv, g = r - (r / Hkv) * Hkv;
    const int head = g * G + hr;
    // the next window's descriptor (its item was taken during this window's
    // predecessor) and, from workgroup-thread 0, the item of the window after
    // it, neither waited for here
    const int4 wdn = un >= 0 ? p.win_desc[__builtin_amdgcn_readfirstlane(un)] : int4{0, 0, 0, 0};
    int nn = 0;
    if (tid == 0 && un >= 0) nn = atomic_add_nowait(wq.head, 1);  // XcdQueue::next(false)
    int tkn[2] = {-1, -1};
    bool tokens_issued = false;
    u32x4 qn[8];  // the next piece's Q (at the window's end: the next window's first piece)
    for (;;) {
      const int s_run = __builtin_amdgcn_readfirstlane(s_seq[bf][a0]);
      const bool last = a1 >= n;
      const int a2 = last ? a1 : piece_end(bf, n, a1);
      if (!last) load_q8_rows(qn, p, row_token(bf, a1, a2), head, h);  // the next piece's Q, in flight
      rows_reset(rt);
      const int rows = (a1 - a0) * G;
      const bool valid = rho < rows;
      const int tok = valid ? s_tok[bf][a0 + rho / G] : -1;
      rt.seq = s_run;
      rt.pos = INT_MAX;
      if (s_run >= 0) {
        const int L = used_u(s_run);
        const int Leff = min(L, p.MP * p.P);
        const int64_t c0 = cu_u(s_run), c1 = cu_u(s_run + 1);
        const int base = (int)(L - (c1 - c0) - c0);  // pos = base + token
        if (p.causal && tok >= 0) rt.pos = base + tok;
        const int pmin = p.causal ? base + s_tok[bf][a0] : INT_MAX;
        const int pmax = p.causal ? base + s_tok[bf][a1 - 1] : INT_MAX;
        if (32 * wave < rows) {
          // the block's chunks that some row of the piece sees: a prefix
          // (keys below the used length and at or before the last row's
          // position); chunk q's keys [key0, lim) are present (none when its
          // page is absent), and it is masked unless all 32 are present and
          // visible to every row
          int key0[4], lim[4], nq = 0;
          unsigned mmask = 0u;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            key0[q] = kBlk * b + 32 * q;
            lim[q] = ((st_absent >> q) & 1u) ? key0[q] : min(Leff, key0[q] + 32);
            if (key0[q] < Leff && key0[q] <= pmax) nq = q + 1;
            if (!(lim[q] == key0[q] + 32 && key0[q] + 31 <= pmin)) mmask |= 1u << q;
          }
          nq = __builtin_amdgcn_readfirstlane(nq);  // uniform: the piece's, not the lane's
          mmask = __builtin_amdgcn_readfirstlane(mmask);
          switch (nq) {
            case 1: rows_block<CT, 1>(rt, s_blk, key0, lim, mmask, p.scale_log2); break;
            case 2: rows_block<CT, 2>(rt, s_blk, key0, lim, mmask, p.scale_log2); break;
            case 3: rows_block<CT, 3>(rt, s_blk, key0, lim, mmask, p.scale_log2); break;
            case 4: rows_block<CT, 4>(rt, s_blk, key0, lim, mmask, p.scale_log2); break;
            default: break;
          }
        }
      }
      // the next window's tokens, once its descriptor has landed
      if (!tokens_issued) {
        load_tokens(wdn, tkn);
        tokens_issued = true;
      }
      // the block of the piece after this one
      int nseq, nb = b, ng = g;
      if (!last) {
        nseq = s_seq[bf][a1];
      } else {
        // end of the window: the next window's token list into the other
        // buffer (its last readers finished before this window began) and
        // the item of the window after it
        if (un >= 0) prepare(bf ^ 1, wdn, tkn);
        if (tid == 0) {
          wait_vmcnt<0>();  // the queue slot taken at the window's start
          const int v = settle(nn);
          s_item[bf] = un >= 0 && wq.lo + wq.nwg + v < wq.hi ? wq.lo + wq.nwg + v : -1;
        }
        __syncthreads();  // the token list and the item are visible; every wave is done with s_blk
        nseq = un >= 0 ? s_seq[bf ^ 1][0] : -1;
        nb = wdn.x / Hkv;
        ng = wdn.x - nb * Hkv;
      }
      // partial result of the piece's rows: normalised O, packed to 16 bits
      // here (the accumulators are free before the block is staged), and
      // log2 LSE
      const float l_row = rows_total(rt);
      u32x4 pk[8];
      float lse_row;
      {
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u) pk[2 * t + u] = paired16<CT>(rt, t, u, inv);
        const float mu = rt.m == -INFINITY ? 0.f : rt.m;
        lse_row = l_row > 0.f ? mu + log2f(l_row) : -INFINITY;
      }
      const int nseq_u = __builtin_amdgcn_readfirstlane(nseq);
      const bool restage = nseq_u >= 0 && (nseq_u != st_s || nb != st_b || ng != st_g);
      if (restage) {
        if (!last) ring_barrier();  // every wave is done with the staged block
        stage(nseq_u, nb, ng);
      }
      if (last && un >= 0) {
        // the next window's first piece's Q, ahead of the stores below
        const int na1 = piece_end(bf ^ 1, min(wdn.w, p.Tu), 0);
        load_q8_rows(qn, p, row_token(bf ^ 1, 0, na1), ng * G + hr, h);
      }
      // Every wave issues the same kUnitStoreOps stores: buffer stores through
      // a descriptor over the two 32-row groups of the partial layout that
      // the wave's 32 rows can touch, where a row outside the piece takes an
      // offset past the descriptor's end, so the hardware drops its store
      // (no memory write, and still one instruction in the wave's count).
      // The partials are read once, by the tile kernel, long after they leave
      // L2: they are written and read with the non-temporal hint (same-box
      // A/B: tile kernel 430 -> 357 us on the MQA batch, 950 -> 926 us on the
      // shared-selection prefill).
      {
        const int64_t wrow = uniform64((int64_t)(e0 + a0) * G + 32 * wave);  // the wave's first row
        const int64_t grp = wrow >> 5;
        const int64_t pidx = wrow + c;  // row (e0 + a0 + rho / G) * G + hr
        const int ooff = valid ? (int)((pidx >> 5) - grp) * 8192 + (int)(pidx & 31) * 16 + 512 * h : kDropOff;
        const int loff = valid && h == 0 ? (int)(pidx - 32 * grp) * 4 : kDropOff;
        const __amdgpu_buffer_rsrc_t ro =
            __builtin_amdgcn_make_buffer_rsrc((char*)p.opart + grp * 8192, (short)0, 2 * 8192, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rl =
            __builtin_amdgcn_make_buffer_rsrc(p.lpart + 32 * grp, (short)0, 64 * 4, kRsrcWord3);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(pk[2 * t + u], ro, ooff + (4 * t + 2 * u) * 512, 0, kBufNT);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_row), rl, loff, 0, kBufNT);
      }
      if (restage) {
        // the block's loads were issued before the stores: wait for them but
        // not for the stores
        if constexpr (!kFp8) wait_vmcnt<kUnitStoreOps>();
        ring_barrier();
      }
      if (last) break;
      a0 = a1;
      a1 = a2;
#pragma unroll
      for (int s = 0; s < 8; ++s) rt.qb[s] = qn[s];
    }
    if (un < 0) break;
    u = un;
    wd = wdn;
    un = __builtin_amdgcn_readfirstlane(s_item[bf]);
    bf ^= 1;
    n = min(wd.w, p.Tu);
    a0 = 0;
    a1 = piece_end(bf, n, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) rt.qb[s] = qn[s];
  }
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup
}

// ---------------------------------------------------------------------------
// k_tiles: one tile per item. The classifier wrote each item's descriptor
// and chunk table (write_tile_desc: the chunks fully visible to every row of
// the tile first). The chain's chunks stream through a ring of LDS slots
// that runs on from one item into the next: once the current item's chunks
// are all issued, the next item's first chunks follow in the same slots, so
// the next item starts with its data in place. Then the residual partials of
// each row are merged and O / LSE are written.
//
// Everything an item needs besides Q and the partials reaches LDS by
// direct-to-LDS loads issued early and ordered by the ring's own waits: the
// next item's descriptor and chunk table and the current item's residual
// counts and positions, at the start of the current item; the item after
// next is requested from the work queue at the same time. No load the
// compiler tracks is waited for inside the chunk loop, so the ring's loads
// stay in flight across the item boundary. Workgroup 0 also clears the
// counter set of the next call.
// ---------------------------------------------------------------------------
constexpr int kTileThreads = 512;  // 8 waves: 256 query rows per tile
constexpr int kAhead = 6;           // chunks in flight ahead of the one being multiplied
constexpr int kRingT = kAhead + 2;  // ring slots: chunks ci-1 .. ci+1 in use, kAhead - 1 more landing
constexpr int kTabMax = 4 * 64;     // chunk table entries (top-k <= 64)
constexpr int kPosMax = 4096;       // residual positions of one item held in LDS
constexpr int kTokMax = 256;        // tokens of one tile

// 4-byte direct-to-LDS buffer load per lane (lane i's bytes at lds + 4 i)
__device__ __forceinline__ void dma4(i32x4v rsrc, uint32_t lds, int voff) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"{m0}"(a), "v"(voff), "s"(rsrc) : "memory");
}

template <typename CT, typename KVT>
__global__ __launch_bounds__(kTileThreads, 1) void k_tiles(Params p) {
  constexpr bool kFp8 = sizeof(KVT) == 1;  // e4m3fn or MXFP4: staged through registers
  constexpr bool kFp4 = std::is_same<KVT, mxfp4_t>::value;
  using RawT = typename std::conditional<kFp4, Raw4, Raw8>::type;
  auto ld_raw = [&](int64_t off, int nr) -> RawT {
    if constexpr (kFp4)
      return load_chunk4(p, off, nr);
    else
      return load_chunk8((const uint8_t*)p.k, (const uint8_t*)p.v, off, nr, p.zero_page);
  };
  auto st_raw = [&](const RawT& r, u32x4* sK, u32x4* sV) {
    if constexpr (kFp4)
      store_chunk4<CT>(r, sK, sV);
    else
      store_chunk8<CT>(r, sK, sV);
  };
  __shared__ __attribute__((aligned(256))) u32x4 s_ring[kRingT * kSlotU4];
  __shared__ int4 s_tab[2][kTabMax];  // chunk tables of the current and the next item
  __shared__ int4 s_desc[2][2];       // their descriptors
  __shared__ int s_pos[kPosMax];      // the current item's residual positions, [token][rank]
  __shared__ int s_nres[kTokMax];     // and residual counts
  __shared__ int s_item;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const uint32_t koff0 = k_lane_offset0();
  if (blockIdx.x == 0 && p.counters_next)
    for (int i = tid; i < kCntSlots; i += kTileThreads) p.counters_next[i] = 0;
  const int G = p.G, Hkv = p.Hkv, K = p.K, K4 = 4 * p.K;
  const int Teff = p.T > 0 ? p.T : 1;
  // decode mode: the listed tiles; otherwise every tile, enumerated as
  // (KV head, tile number) so that an XCD's range holds neighbouring tiles
  // of one KV head
  const bool listed = p.stream_narrow != 0;
  const int ntiles = (p.Tq + Teff - 1) / Teff + p.B;  // bound on the tile count
  const int total = listed ? p.counters[kCntTiles] : ntiles * Hkv;
  if (total == 0) return;
  DmaLane512 dl;
  dl.init();
  const uint32_t ring0 = lds_addr(s_ring);
  XcdQueue wq;
  wq.init(total, p.counters + kCntXcd);

  // descriptor and chunk table of item i into buffer bf (direct-to-LDS:
  // lane l of wave w < 4 brings table entry 64 w + l; wave 0 also the
  // descriptor)
  auto fetch_meta = [&](int i, int bf) {
    if (wave < kTabMax / 64)
      dma16(make_rsrc(p.ctab + (size_t)i * K4, K4 * 16), lds_addr(&s_tab[bf][64 * wave]), 16 * (64 * wave + lane));
    if (wave == 0 && lane < 2) dma16(make_rsrc(p.tdesc + 2 * (size_t)i, 32), lds_addr(&s_desc[bf][0]), 16 * lane);
  };
  // residual counts and positions of the item's tokens (nt tokens from t0,
  // KV head g), the positions when they fit
  auto fetch_res = [&](int t0, int nt, int g) {
    const size_t tg0 = (size_t)t0 * Hkv + g;
    if (wave * 64 < nt) {
      const i32x4v rn = make_rsrc(p.tok_nres + tg0, ((nt - 1) * Hkv + 1) * 4);
      dma4(rn, lds_addr(&s_nres[64 * wave]), 4 * (64 * wave + lane) * Hkv);
    }
    if (nt * K <= kPosMax) {
      const i32x4v rp = make_rsrc(p.res_list + tg0 * K, ((nt - 1) * Hkv + 1) * K * 4);
      for (int j = 64 * wave; j < nt * K; j += kTileThreads) {
        const int e = j + lane, tau = e / K;
        dma4(rp, lds_addr(&s_pos[j]), 4 * (tau * Hkv * K + (e - tau * K)));
      }
    }
  };
  // chunk ci of table bf (n chunks): element offset (-1: skip) and rows present
  auto chunk_of = [&](int bf, int ci, int n, int64_t& off, int& nrows) {
    if (ci < n) {
      const int4 e = s_tab[bf][ci];
      off = (int64_t)(((uint64_t)(uint32_t)e.y << 32) | (uint32_t)e.x);
      nrows = e.w;
    } else {
      off = -1;
      nrows = 0;
    }
  };
  // the same entry of item `item`'s table, by a scalar load from global
  // memory: the tables are written by an earlier kernel and only read by
  // this one, so the constant address space applies, and the chunk step
  // spends no vector instruction or LDS read on it
  auto chunk_const = [&](int item, int ci, int n, int64_t& off, int& nrows) {
    if (ci < n) {
      const int4 e = const_load(p.ctab + (size_t)item * K4 + ci);
      off = (int64_t)(((uint64_t)(uint32_t)e.y << 32) | (uint32_t)e.x);
      nrows = e.w;
    } else {
      off = -1;
      nrows = 0;
    }
  };
  auto slot_addr = [&](int x) { return ring0 + 16 * kSlotU4 * (x & (kRingT - 1)); };
  auto slot_ptr = [&](int x) { return s_ring + (x & (kRingT - 1)) * kSlotU4; };

  const int rho = 32 * wave + c;  // the lane's row within the tile
  Rows32 rt;
  auto load_q_item = [&](int4 i0, int4 i1) {
    const int nrows = i0.z * G;
    load_q8(rt.qb, p, rho < nrows ? i0.x + rho / G : -1, i1.z * G + rho % G, h);
  };

  // start: the first item (a fixed one per workgroup) and the next
  int cur = wq.next(true);
  if (cur < 0) return;
  if (tid == 0) s_item = wq.next(false);
  fetch_meta(cur, 0);
  wait_vmcnt<0>();
  __syncthreads();
  int nxt = s_item;
  int bf = 0;               // table buffer of the current item
  int rbase = 0;            // ring slot of the current item's chunk 0
  int first_real = kAhead;  // the current item's chunks below this are not in flight yet
  load_q_item(s_desc[0][0], s_desc[0][1]);

  for (;;) {
    const int4 d0 = s_desc[bf][0], d1 = s_desc[bf][1];
    const int t0 = d0.x, s = d0.y, nt = d0.z;
    const int nck = nt > 0 ? d0.w : 0;  // chunks in the item's table
    const int nfull = min(d1.w, nck);
    const int base = d1.y, g = d1.z;
    const int rows = nt * G;
    const int pmin = p.causal ? base + t0 : INT_MAX;
    const bool lds_res = nt * K <= kPosMax;
    const bool valid = rho < rows;
    const int tau = valid ? rho / G : 0;
    const int hr = rho - tau * G;
    const int tok = t0 + tau;
    const int head = g * G + hr;
    rows_reset(rt);
    rt.seq = s;
    rt.pos = (valid && p.causal) ? base + tok : INT_MAX;
    // early loads: this item's residual data, the next item's table, the
    // item after next
    if (nt > 0) fetch_res(t0, nt, g);
    if (nxt >= 0) fetch_meta(nxt, bf ^ 1);
    int nn = 0;
    if (tid == 0) nn = atomic_add_nowait(wq.head, 1);  // XcdQueue::next(false), not waited for here

    if (nck > 0) {
      if constexpr (kFp8) {
        wait_vmcnt<0>();
        __syncthreads();
        // register-staged double buffer: chunk ci+1 loads while ci is multiplied
        int64_t off;
        int nr;
        const bool stager = tid < 256;  // 32 rows x 8 pieces of K and of V
        chunk_of(bf, 0, nck, off, nr);
        RawT raw{};
        if (stager) {
          raw = ld_raw(off, nr);
          st_raw(raw, s_ring, s_ring + kChunkU4);
        }
        if constexpr (kFp4) {
          // MXFP4 chunks are 6 registers of raw bytes a thread: two are kept
          // in flight (chunk ci+1 in one set, ci+2 loading into the other,
          // the sets swapping roles every chunk; a set is loaded again only
          // after its chunk went to LDS)
          RawT rb{};
          chunk_of(bf, 1 < nck ? 1 : 0, nck, off, nr);
          if (stager) rb = ld_raw(off, nr);
          __syncthreads();
          auto step = [&](int ci, const RawT& next, RawT& after) {
            chunk_of(bf, ci + 2 < nck ? ci + 2 : ci, nck, off, nr);
            if (stager) after = ld_raw(off, nr);
            const u32x4* sK = s_ring + (ci & 1) * kSlotU4;
            const int4 e = s_tab[bf][ci];
            if (32 * wave < rows && !(e.x == -1 && e.y == -1)) {
              const bool full = e.w == 32 && e.z + 31 <= pmin;
              rows_chunk<CT>(rt, sK, sK + kChunkU4, e.z, e.z + e.w, s, !full, p.scale_log2);
            }
            if (stager && ci + 1 < nck)
              st_raw(next, s_ring + ((ci + 1) & 1) * kSlotU4, s_ring + ((ci + 1) & 1) * kSlotU4 + kChunkU4);
            __syncthreads();
          };
          for (int ci = 0; ci < nck; ci += 2) {
            step(ci, rb, raw);
            if (ci + 1 < nck) step(ci + 1, raw, rb);
          }
        } else {
          __syncthreads();
          for (int ci = 0; ci < nck; ++ci) {
            chunk_of(bf, ci + 1 < nck ? ci + 1 : ci, nck, off, nr);
            if (stager) raw = ld_raw(off, nr);
            const u32x4* sK = s_ring + (ci & 1) * kSlotU4;
            const int4 e = s_tab[bf][ci];
            if (32 * wave < rows && !(e.x == -1 && e.y == -1)) {
              // keys [e.z, e.z + e.w) are present (e.w < 32 only at the used length)
              const bool full = e.w == 32 && e.z + 31 <= pmin;
              rows_chunk<CT>(rt, sK, sK + kChunkU4, e.z, e.z + e.w, s, !full, p.scale_log2);
            }
            if (stager && ci + 1 < nck)
              st_raw(raw, s_ring + ((ci + 1) & 1) * kSlotU4, s_ring + ((ci + 1) & 1) * kSlotU4 + kChunkU4);
            __syncthreads();
          }
        }
      } else {
        // chunks not brought in by the previous item's loop
        if (first_real > 0) {
          for (int ci = 0; ci < first_real; ++ci) {
            int64_t off;
            int nr;
            chunk_of(bf, ci, nck, off, nr);
            issue_chunk16_512(p.k, p.v, off, nr, dl, slot_addr(rbase + ci));
          }
          wait_vmcnt<0>();
        } else {
          wait_vmcnt<2 * (kAhead - 1)>();  // chunk 0 has landed (chunks 1 .. kAhead-1 may be in flight)
        }
        ring_barrier();
        // the state carried from one iteration to the next: the scores of
        // the current chunk, the probabilities of the previous one and the
        // first two V fragments of the next products. The loops run two
        // iterations per trip with the roles of A and B swapped, so the
        // state is never copied.
        struct Pipe {
          f32x16 sc;
          u32x4 pp[2];
          u32x4 vpre[2];
        } A, B;
        A.sc = rows_scores<CT>(rt, slot_ptr(rbase));
        A.pp[0] = u32x4{0u, 0u, 0u, 0u};  // P of chunk -1 (nothing)
        A.pp[1] = u32x4{0u, 0u, 0u, 0u};
        A.vpre[0] = vfrag_at((const char*)(slot_ptr(rbase) + kChunkU4), 0, 0);  // chunk 0 stands in for chunk -1
        A.vpre[1] = vfrag_at((const char*)(slot_ptr(rbase) + kChunkU4), 1, 0);
        // software pipeline over the chunks: iteration ci multiplies V(ci-1)
        // by P(ci-1), computes the scores S(ci+1) and the probabilities of
        // S(ci) (tile_iter). Iteration ci reads chunks ci-1 .. ci+1, so
        // once every wave has passed its barrier the slot of chunk ci-2
        // takes chunk ci + kAhead: this item's, else the next item's.
        auto step = [&](int ci, bool mask, const Pipe& in, Pipe& out) {
          const int nx = ci + kAhead;
          int64_t off = -1;
          int nr = 0;
          if (nx < nck) chunk_const(cur, nx, nck, off, nr);
          wait_vmcnt<2 * (kAhead - 2)>();  // chunk ci+1 has landed
          loop_barrier();                  // ... for every wave; and slot (ci - 2) % kRingT is free
          if (nx >= nck && nxt >= 0 && (ci >= kAhead - 1 || first_real > 0)) {
            // a chunk of the next item (its first chunks are issued by this
            // loop once it is past chunk kAhead - 1, or after a top-up)
            const int4 dn = const_load(p.tdesc + 2 * (size_t)nxt);
            chunk_const(nxt, nx - nck, dn.z > 0 ? dn.w : 0, off, nr);
          }
          issue_chunk16_512(p.k, p.v, off, nr, dl, slot_addr(rbase + nx));
          // a masked chunk's keys [key0, lim) are present: none when its page
          // is absent or no row sees it, fewer than 32 at the used length
          const int4 ec = mask ? s_tab[bf][ci] : int4{0, 0, 0, 0};
          const int key0 = ec.z, lim = ec.z + ec.w;
          const char* vprev = (const char*)(slot_ptr(rbase + (ci > 0 ? ci - 1 : 0)) + kChunkU4);
          const char* vcur = (const char*)(slot_ptr(rbase + ci) + kChunkU4);
          const u32x4* knext = slot_ptr(rbase + (ci + 1 < nck ? ci + 1 : ci));
          const float alpha = mask ? tile_iter<CT, true>(rt, in.sc, in.pp, vprev, in.vpre, vcur, knext, koff0, key0,
                                                         lim, p.scale_log2, out.sc, out.pp, out.vpre)
                                   : tile_iter<CT, false>(rt, in.sc, in.pp, vprev, in.vpre, vcur, knext, koff0, key0,
                                                          lim, p.scale_log2, out.sc, out.pp, out.vpre);
          rows_rescale(rt, alpha);
        };
        int ci = 0;
        for (; ci + 2 <= nfull; ci += 2) {
          step(ci, false, A, B);
          step(ci + 1, false, B, A);
        }
        if (ci < nfull) {
          step(ci++, false, A, B);
          A = B;
        }
        for (; ci + 2 <= nck; ci += 2) {
          step(ci, true, A, B);
          step(ci + 1, true, B, A);
        }
        if (ci < nck) {
          step(ci++, true, A, B);
          A = B;
        }
        rows_pv<CT>(rt, A.pp, slot_ptr(rbase + nck - 1) + kChunkU4);
      }
    }
    // The next item's chunks j < kAhead that this loop issued: those of
    // iterations from kAhead - 1 on (all of them, after a top-up), i.e.
    // j >= 2 kAhead - 1 - nck (j >= kAhead - nck); the rest is issued when
    // the next item starts.
    int next_first_real = kAhead;
    if (!kFp8 && nck > 0)
      next_first_real = first_real > 0 ? max(0, kAhead - nck) : min(kAhead, max(0, 2 * kAhead - 1 - nck));
    // This item's residual data, the next item's table and the queue slot
    // taken at the start were issued before chunk kAhead of this item: they
    // have landed once the loop has waited for that chunk, else (short
    // items, and the 8-bit path, which issues no ring loads) they are
    // drained here.
    if (!kFp8 && nck >= kAhead) {
      wait_vmcnt<2 * kAhead>();
    } else {
      wait_vmcnt<0>();
    }
    if (tid == 0) {
      const int v = settle(nn);
      s_item = nxt >= 0 && wq.lo + wq.nwg + v < wq.hi ? wq.lo + wq.nwg + v : -1;
    }
    ring_barrier();  // every wave is done with the ring slots of this item and s_tab[bf]
    if (nxt >= 0) load_q_item(s_desc[bf ^ 1][0], s_desc[bf ^ 1][1]);

    // merge with the unit partials of the row's residual slots, then write.
    // Two partials are in flight while one is merged (their positions are in
    // LDS). The reference max M moves only when a partial's LSE exceeds it
    // by more than 2^kRescale32.
    // Every lane runs the same number of iterations and stores (rows outside
    // the tile into a scratch row): with no branch around loads or stores,
    // the compiler's waits count exactly the loads they need.
    const float l_tot = rows_total(rt);
    {
      const size_t tg = valid ? (size_t)tok * Hkv + g : 0;
      const int nr_ = lds_res ? s_nres[tau] : p.tok_nres[tg];
      const int nres = valid ? min(nr_, K) : 0;
      int nres_w = nres;  // the wave's largest count
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) nres_w = max(nres_w, __shfl_xor(nres_w, off, 64));
      nres_w = __builtin_amdgcn_readfirstlane(nres_w);
      const int ntot = p.counters[kCntResidual];  // positions are below this
      float M = rt.m;  // O and W are relative to 2^M
      float W = l_tot;
      // a partial row is read as 16-byte chunks (lane (h, c): chunk 4t + 2u +
      // h, d = 32t + 16u + 8h + (0..7)) and put into the D layout by the same
      // half-wave swap as paired16, just before it is merged
      const char* obase = (const char*)p.opart + 512 * h;
      struct Part {
        float l;
        u32x4 d[8];
      };
      auto pos_of = [&](int i) {
        const int ii = min(i, K - 1);
        const int v = lds_res ? s_pos[tau * K + ii] : p.res_list[tg * K + ii];
        return i < nres ? v : -1;
      };
      auto fetch = [&](int pos, Part& pt) {
        const bool ok = pos >= 0 && pos < ntot;
        const size_t pidx = ok ? (size_t)pos * G + hr : 0;
        const float lv = __builtin_nontemporal_load(p.lpart + pidx);
        pt.l = ok ? lv : -INFINITY;
        const char* src = obase + part_offset(pidx);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u) pt.d[2 * t + u] = __builtin_nontemporal_load((const u32x4*)(src + (4 * t + 2 * u) * 512));
      };
      auto merge = [&](const Part& pt) {
        const float lc = pt.l;
        const bool use = lc != -INFINITY;
        const bool lift = use && (M == -INFINITY || lc > M + kRescale32);
        const float m_new = lift ? lc : M;
        const float sc = (lift && M != -INFINITY) ? exp2f(M - lc) : (lift ? 0.f : 1.f);
        if (__any(lift)) {
          W *= sc;
#pragma unroll
          for (int t = 0; t < 4; ++t) rt.o[t] *= sc;
        }
        M = m_new;
        const float fi = use ? exp2f(lc - M) : 0.f;
        W += fi;
        // the weight as a 16-bit value beside a zero: one dot2 instruction
        // scales and accumulates one element of a packed pair (the weight's
        // rounding to 16 bits moves O by at most 2^-9 of this partial's share;
        // the row sum W keeps the fp32 weight)
        const uint32_t wlo = pack2<CT>(fi, 0.f), whi = wlo << 16;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const u32x4 v = pt.d[2 * t + u];
            const auto s0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
#pragma unroll
            for (int e = 0; e < 2; ++e) {  // group a = 2u + e: words s0[e], s1[e]
              const int a = 2 * u + e;
              rt.o[t][4 * a] = Dot2<CT>::run(s0[e], wlo, rt.o[t][4 * a]);
              rt.o[t][4 * a + 1] = Dot2<CT>::run(s0[e], whi, rt.o[t][4 * a + 1]);
              rt.o[t][4 * a + 2] = Dot2<CT>::run(s1[e], wlo, rt.o[t][4 * a + 2]);
              rt.o[t][4 * a + 3] = Dot2<CT>::run(s1[e], whi, rt.o[t][4 * a + 3]);
            }
          }
      };
      if (nres_w > 0) {
        Part pa, pb;
        fetch(pos_of(0), pa);
        fetch(pos_of(1), pb);
        for (int i = 0; i < nres_w; i += 2) {
          merge(pa);
          fetch(pos_of(i + 2), pa);
          merge(pb);
          fetch(pos_of(i + 3), pb);
        }
      }
      const float inv = W > 0.f ? 1.f / W : 0.f;
      uint16_t* orow = valid ? (uint16_t*)p.out + ((size_t)tok * p.Hq + head) * kD : (uint16_t*)p.scratch_row;
      store_row16<CT>(orow, rt, inv);
      float* lrow = (valid && h == 0 && p.lse) ? p.lse + (size_t)head * p.Tq + tok : (float*)p.scratch_row + 64 + lane;
      *lrow = W > 0.f ? (M + log2f(W)) * kLn2 : -INFINITY;
    }
    ring_barrier();  // s_item visible; every wave is done with s_pos / s_nres
    if (nxt < 0) break;
    rbase = (rbase + nck) & (kRingT - 1);
    first_real = next_first_real;
    bf ^= 1;
    cur = nxt;
    nxt = s_item;
  }
  wait_vmcnt<0>();  // no load into LDS outlives the workgroup
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename CT, typename KVT>
static hipError_t launch_units_t(const ProfSpan& sp, const Params& p, int num_cu, hipStream_t st) {
  return launch_k(sp, true, true, k_units<CT, KVT>, dim3(num_cu * 2), dim3(256), 0, st, p);
}

template <typename CT, typename KVT>
static hipError_t launch_tiles_t(const ProfSpan& sp, const Params& p, int num_cu, hipStream_t st) {
  return launch_k(sp, true, true, k_tiles<CT, KVT>, dim3(num_cu), dim3(kTileThreads), 0, st, p);
}

hipError_t launch_units(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st) {
  const ProfSpan sp = profile_begin(kKUnits);
  hipError_t e;
  if (q_elem == kElemBF16)
    e = kv_elem == kElemFP8   ? launch_units_t<bf16_t, fp8_e4m3_t>(sp, p, num_cu, st)
        : kv_elem == kElemFP4 ? launch_units_t<bf16_t, mxfp4_t>(sp, p, num_cu, st)
                              : launch_units_t<bf16_t, bf16_t>(sp, p, num_cu, st);
  else
    e = kv_elem == kElemFP8 ? launch_units_t<f16_t, fp8_e4m3_t>(sp, p, num_cu, st)
                            : launch_units_t<f16_t, f16_t>(sp, p, num_cu, st);
  profile_end(sp, e == hipSuccess);
  return e;
}

hipError_t launch_tiles(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st) {
  const ProfSpan sp = profile_begin(kKTiles);
  hipError_t e;
  if (q_elem == kElemBF16)
    e = kv_elem == kElemFP8   ? launch_tiles_t<bf16_t, fp8_e4m3_t>(sp, p, num_cu, st)
        : kv_elem == kElemFP4 ? launch_tiles_t<bf16_t, mxfp4_t>(sp, p, num_cu, st)
                              : launch_tiles_t<bf16_t, bf16_t>(sp, p, num_cu, st);
  else
    e = kv_elem == kElemFP8 ? launch_tiles_t<f16_t, fp8_e4m3_t>(sp, p, num_cu, st)
                            : launch_tiles_t<f16_t, f16_t>(sp, p, num_cu, st);
  profile_end(sp, e == hipSuccess);
  return e;
}

}  // namespace msa
