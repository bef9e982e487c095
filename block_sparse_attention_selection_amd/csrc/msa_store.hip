// msa_store.hip -- the paged K/V store, the step before the attention pass:
// the keys and values of new tokens go to their slots of the paged caches,
// and an fp8 e4m3fn cache receives them through an unscaled cast (sglang pull
// request "Speed up MiniMax-M3 sparse attention on Hopper": the fused K/V
// store casts 16-bit values to fp8_e4m3 without a scale, bit-exact with
// clamping to +-448 and rounding to nearest even).
//
// A thread moves one 32-byte piece (16 values) of a row (new token, KV head)
// of K or of V: 8 consecutive threads read a row's 256 contiguous bytes and
// write its 256 (16-bit cache) or 128 (fp8 cache) contiguous bytes. The work
// is pure data movement, bound by HBM; one piece per thread (many small
// workgroups) measured faster than 2, 4, 8 or 16 pieces per thread.
#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {

// e4m3fn codes of two floats: clamped to [-448, 448] and rounded to nearest
// even by the gfx950 conversion (OCP e4m3); a NaN keeps its sign bit and
// becomes the NaN code, 0x7F | sign.
__device__ __forceinline__ uint32_t fp8_pair(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  const uint32_t sa = (__builtin_bit_cast(uint32_t, a) >> 24) & 0x80u;
  const uint32_t sb = (__builtin_bit_cast(uint32_t, b) >> 24) & 0x80u;
  if (a != a) w = (w & 0xFF00u) | 0x7Fu | sa;
  if (b != b) w = (w & 0x00FFu) | ((0x7Fu | sb) << 8);
  return w;
}

constexpr int kStoreThreads = 256;
constexpr int kStoreUnroll = 1;  // 32-byte pieces per thread (loads of all of them issued before any store)

template <typename IT, bool kFp8>
__global__ __launch_bounds__(kStoreThreads) void k_store_kv(const uint16_t* kn, const uint16_t* vn,
                                                            const int64_t* loc, void* kc, void* vc, int N,
                                                            int Hkv, int P, int64_t nslots, int ntensors) {
  // piece p of a tensor: row p >> 3 = (token, KV head), 16 values at 16 * (p & 7);
  // pieces [0, per) are K's, [per, 2 per) V's (ntensors = 2)
  const int per = N * Hkv * 8;
  const int base = blockIdx.x * (kStoreThreads * kStoreUnroll) + threadIdx.x;
  u32x4 in[kStoreUnroll][2];
  int64_t dst[kStoreUnroll];
#pragma unroll
  for (int j = 0; j < kStoreUnroll; ++j) {
    dst[j] = -1;
    const int gp = base + j * kStoreThreads;
    if (gp >= ntensors * per) continue;
    const bool is_v = gp >= per;
    const int r = is_v ? gp - per : gp;
    const int row = r >> 3, piece = r & 7;
    const int i = row / Hkv, g = row - i * Hkv;
    const int64_t slot = loc[i];
    if (slot < 0 || slot >= nslots) continue;
    // page sizes are powers of two (64 or 128): a shift, not a 64-bit division
    const int64_t page = slot >> __builtin_ctz((unsigned)P), off = slot & (P - 1);
    const u32x4* src = (const u32x4*)((is_v ? vn : kn) + (int64_t)row * kD + 16 * piece);
    in[j][0] = src[0];
    in[j][1] = src[1];
    dst[j] = ((page * Hkv + g) * P + off) * kD + 16 * piece;  // element index in the cache
    if (is_v) dst[j] |= int64_t(1) << 62;                     // marks V (element indices stay below 2^40)
  }
#pragma unroll
  for (int j = 0; j < kStoreUnroll; ++j) {
    if (dst[j] < 0) continue;
    const bool is_v = (dst[j] >> 62) & 1;
    const int64_t e = dst[j] & ((int64_t(1) << 62) - 1);
    if constexpr (kFp8) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = in[j][w >> 1][2 * (w & 1)], b = in[j][w >> 1][2 * (w & 1) + 1];
        const uint32_t lo = fp8_pair(from_bits16<IT>(a & 0xFFFFu), from_bits16<IT>(a >> 16));
        const uint32_t hi = fp8_pair(from_bits16<IT>(b & 0xFFFFu), from_bits16<IT>(b >> 16));
        o[w] = lo | (hi << 16);
      }
      *(u32x4*)((uint8_t*)(is_v ? vc : kc) + e) = o;
    } else {
      u32x4* d = (u32x4*)((uint16_t*)(is_v ? vc : kc) + e);
      d[0] = in[j][0];
      d[1] = in[j][1];
    }
  }
}

hipError_t launch_store_kv(const void* kn, const void* vn, const int64_t* loc, void* kc, void* vc, int N, int Hkv,
                           int P, int64_t num_pages, int in_elem, bool fp8_cache, hipStream_t st) {
  const int ntensors = vn ? 2 : 1;  // no V: the K rows only (an index key cache)
  const int64_t pieces = ntensors * (int64_t)N * Hkv * 8;
  if (pieces == 0) return hipSuccess;
  const int64_t per_block = kStoreThreads * kStoreUnroll;
  const dim3 grid((unsigned)((pieces + per_block - 1) / per_block)), block(kStoreThreads);
  const int64_t nslots = num_pages * P;
  const uint16_t* k16 = (const uint16_t*)kn;
  const uint16_t* v16 = (const uint16_t*)vn;
  const ProfSpan sp = profile_begin(kKStore);
  hipError_t e;
  if (in_elem == kElemBF16) {
    if (fp8_cache)
      e = launch_k(sp, true, true, k_store_kv<bf16_t, true>, grid, block, 0, st, k16, v16, loc, kc, vc, N, Hkv, P,
                   nslots, ntensors);
    else
      e = launch_k(sp, true, true, k_store_kv<bf16_t, false>, grid, block, 0, st, k16, v16, loc, kc, vc, N, Hkv, P,
                   nslots, ntensors);
  } else {
    if (fp8_cache)
      e = launch_k(sp, true, true, k_store_kv<f16_t, true>, grid, block, 0, st, k16, v16, loc, kc, vc, N, Hkv, P,
                   nslots, ntensors);
    else
      e = launch_k(sp, true, true, k_store_kv<f16_t, false>, grid, block, 0, st, k16, v16, loc, kc, vc, N, Hkv, P,
                   nslots, ntensors);
  }
  profile_end(sp, e == hipSuccess);
  return e;
}

}  // namespace msa
