// msa_device.hpp -- device-side types and helpers for the gfx950 kernels.
//
// Register-fragment conventions used by every attention kernel (one wave,
// 16 query rows, MFMA v_mfma_f32_16x16x32_{bf16,f16}):
//   lane l = 16*q + c   (q = l / 16 in 0..3, c = l % 16)
//   A operand: lane holds 8 consecutive k-values of row m = c
//   B operand: lane holds 8 consecutive k-values of column n = c
//   D (4 fp32): lane holds rows m = 4*q + r (r = 0..3) of column n = c
// Both operands pair their k-values by (lane group q, element e), so any
// assignment of the contraction index to (q, e) is valid as long as A and B
// use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kD = 128;    // head dimension
constexpr int kBlk = 128;  // tokens per selection block
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

struct fp8_e4m3_t {  // storage tag for e4m3fn caches
  uint8_t bits;
};
struct mxfp4_t {  // storage tag for MXFP4 caches: e2m1 codes, two a byte, and e8m0 scales
  uint8_t bits;
};

// ---------------------------------------------------------------------------
// MFMA on raw 128-bit fragments, by 16-bit element type
// ---------------------------------------------------------------------------
template <typename T>
struct Mma;

template <>
struct Mma<bf16_t> {
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<f16_t> {
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// fp32 -> 16-bit (round to nearest even) and packing
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ uint32_t to_bits16(float x);

template <>
__device__ __forceinline__ uint32_t to_bits16<bf16_t>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <>
__device__ __forceinline__ uint32_t to_bits16<f16_t>(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// two values, one v_cvt_pk_{bf16,f16}_f32
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef T t2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), t2));
}

template <typename T>
__device__ __forceinline__ float from_bits16(uint32_t b);

template <>
__device__ __forceinline__ float from_bits16<bf16_t>(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

template <>
__device__ __forceinline__ float from_bits16<f16_t>(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// ---------------------------------------------------------------------------
// e4m3fn -> 16-bit widening (exact: every e4m3fn value is a bf16 and an fp16
// value). Uses the gfx950 scaled conversion with scale 1.0.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ uint32_t widen2_lo(uint32_t w);  // bytes 0,1 of w
template <typename T>
__device__ __forceinline__ uint32_t widen2_hi(uint32_t w);  // bytes 2,3 of w

template <>
__device__ __forceinline__ uint32_t widen2_lo<bf16_t>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen2_hi<bf16_t>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
template <>
__device__ __forceinline__ uint32_t widen2_lo<f16_t>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen2_hi<f16_t>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// 8 e4m3fn values (two dwords) -> 8 16-bit values (four dwords)
template <typename T>
__device__ __forceinline__ u32x4 widen8(u32x2 v) {
  u32x4 r;
  r[0] = widen2_lo<T>(v[0]);
  r[1] = widen2_hi<T>(v[0]);
  r[2] = widen2_lo<T>(v[1]);
  r[3] = widen2_hi<T>(v[1]);
  return r;
}

// An e8m0 scale byte b as the float 2^(b - 127) (b = 0: 2^-127, a denormal;
// b = 255, the format's NaN, is not supported and reads as infinity)
__device__ __forceinline__ float e8m0_scale(uint32_t b) {
  return __uint_as_float(b ? b << 23 : 0x00400000u);
}

// 8 e2m1 codes (one dword, the code of value 2i in the low nibble of byte i)
// times scale -> 8 bf16 values (four dwords), exactly while the products are
// within bf16's range (the conversion instruction scales before rounding)
__device__ __forceinline__ u32x4 widen_fp4(uint32_t w, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

// ---------------------------------------------------------------------------
// cross-lane reductions over the four lane groups holding one row
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_over_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Scalar loads of read-only data at a wave-uniform address (taken from the
// first lane), waited for in the same statement. They are counted by
// lgkmcnt, so waiting for them never waits for the vector memory operations
// in flight.
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t a = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t sload64(const int64_t* ptr) {
  int64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(ptr)) : "memory");
  return v;
}
__device__ __forceinline__ int sload32(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(ptr)) : "memory");
  return v;
}

// 16 bytes at a wave-uniform address, through the constant address space:
// the compiler issues a scalar load and places its wait. Only for memory
// that no kernel running at the same time writes. The pointer is rebuilt
// from its (wave-uniform) integer value, else the compiler turns the load
// back into a global one, which it makes scalar only where no store of the
// kernel may precede it.
__device__ __forceinline__ int4 const_load(const int4* ptr) {
  typedef int v4 __attribute__((ext_vector_type(4)));
  const uint64_t a = (uint64_t)uniform_ptr(ptr);
  const v4 v = *(const __attribute__((address_space(4))) v4*)a;
  return int4{v.x, v.y, v.z, v.w};
}

// Owner sequence of token t: the largest s with cu[s] <= t, provided
// t < cu[s+1]; -1 when t lies in no sequence. Stays inside cu[0..B].
__device__ __forceinline__ int seq_of(const int64_t* __restrict__ cu, int B, int64_t t) {
  if (B <= 0 || t < cu[0]) return -1;
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  return (t < cu[lo + 1]) ? lo : -1;
}

// Wave-cooperative version of seq_of: every lane of the wave gets the same
// answer after at most two rounds of parallel loads (B <= 4095), falling
// back to a scalar binary search for larger batches. For a non-decreasing
// cu it returns the largest s with cu[s] <= t, then checks t < cu[s+1].
__device__ __forceinline__ int wave_seq_of(const int64_t* __restrict__ cu, int B, int64_t t) {
  if (B <= 0) return -1;
  const int n = B + 1;
  if (n > 64 * 64) return seq_of(cu, B, t);
  const int lane = threadIdx.x & 63;
  int base = 0;
  if (n > 64) {
    const int nb = (n + 63) / 64;
    const bool le = lane < nb && cu[64 * lane] <= t;
    const int c1 = __popcll(__ballot(le));
    if (c1 == 0) return -1;
    base = 64 * (c1 - 1);
  }
  const int idx = base + lane;
  const bool le = idx < n && cu[idx] <= t;
  const int c2 = __popcll(__ballot(le));
  if (c2 == 0) return -1;
  int s = base + c2 - 1;
  if (s > B - 1) s = B - 1;
  return (cu[s] <= t && t < cu[s + 1]) ? s : -1;
}

// Largest i in [0, n) with a[i] <= x, for a non-decreasing a with
// a[0] <= x (one wave; every lane gets the answer). Each round of 64 sampled
// loads narrows the range 64-fold, so n <= 4096 takes two dependent loads.
__device__ __forceinline__ int wave_last_le(const int32_t* __restrict__ a, int n, int x) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;  // the answer lies in [lo, hi)
  while (hi - lo > 64) {
    const int stride = (hi - lo + 63) / 64;
    const int i = lo + lane * stride;
    const bool le = i < hi && a[i] <= x;
    lo = lo + (__popcll(__ballot(le)) - 1) * stride;
    hi = min(lo + stride, hi);
  }
  const int i = lo + lane;
  const bool le = i < hi && a[i] <= x;
  return lo + __popcll(__ballot(le)) - 1;
}

// Tile j of the batch, tiles being runs of T consecutive tokens numbered
// sequence by sequence: returns its sequence and sets its first token, or
// returns -1 beyond the last tile. Token ranges are clamped to [0, Tq).
__device__ __forceinline__ int wave_tile_of(const int64_t* __restrict__ cu, int B, int Tq, int T, int j,
                                            int64_t* t0) {
  const int lane = threadIdx.x & 63;
  const int per = (B + 63) / 64;
  const int s0 = min(lane * per, B), s1 = min(s0 + per, B);
  // token counts are below Tq (an int): 32-bit divisions
  int cnt = 0;
  for (int s = s0; s < s1; ++s) {
    const int64_t n = min(cu[s + 1], (int64_t)Tq) - max(cu[s], (int64_t)0);
    if (n > 0) cnt += ((int)n + T - 1) / T;
  }
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const int excl = incl - cnt;
  const uint64_t m = __ballot(j >= excl && j < incl);
  if (m == 0) return -1;
  const int owner = __ffsll((unsigned long long)m) - 1;
  int s_out = -1, t_out = 0;
  if (lane == owner) {
    int jj = j - excl;
    for (int s = s0; s < s1; ++s) {
      const int64_t a = max(cu[s], (int64_t)0);
      const int64_t n = min(cu[s + 1], (int64_t)Tq) - a;
      const int nt = n > 0 ? ((int)n + T - 1) / T : 0;
      if (jj < nt) {
        s_out = s;
        t_out = (int)(a + (int64_t)jj * T);
        break;
      }
      jj -= nt;
    }
  }
  s_out = __shfl(s_out, owner, 64);
  *t0 = __shfl(t_out, owner, 64);
  return s_out;
}

// ---------------------------------------------------------------------------
// direct-to-LDS buffer loads (shared by the tile, unit and selection kernels)
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4], lgkmcnt[11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte direct-to-LDS buffer load per lane: lane i's bytes land at LDS
// byte address lds + 16 i. Issued from inline assembly so that the compiler
// does not treat every later LDS read as a possible reader of the load (it
// would wait for all loads in flight before the first one): the ring's
// protocol orders these loads with wait_vmcnt and barriers instead.
typedef int i32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void dma16(i32x4v rsrc, uint32_t lds, int voff) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"{m0}"(a), "v"(voff), "s"(rsrc) : "memory");
}

// raw buffer descriptor of nrec bytes at base (stride 0)
__device__ __forceinline__ i32x4v make_rsrc(const void* base, int nrec) {
  const uint64_t b = (uint64_t)base;
  i32x4v r;
  r.x = (int)__builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu);
  r.z = (int)__builtin_amdgcn_readfirstlane((uint32_t)nrec);
  r.w = kRsrcWord3;
  return r;
}

// LDS byte address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

}  // namespace msa
