// msa_rates.hip -- a standalone program that measures the device rates the
// kernels' designs rest on:
//   hbm     streaming reads of 4 GiB with plain and with non-temporal 16-byte
//           loads (GB/s)
//   launch  an empty kernel launched back to back (us per launch)
//   lds     the tile kernel's two LDS read patterns: K rows by ds_read_b128,
//           V^T fragments by ds_read_b64_tr_b16 (bytes per clock and CU)
//   mix     v_mfma_f32_32x32x16_bf16 alone, independent VALU work alone, and
//           both in one loop (cycles per iteration and SIMD, two waves)
//   chain   the tile kernel's chunk iteration (tile_iter, compiled from the
//           tile source itself) over a fixed ring of LDS slots, and copies of
//           it with parts removed (cycles per 32-key chunk and SIMD)
// Cycle figures are time x 2.4 GHz, the nominal shader clock. Every figure is
// the best of three timed runs after one untimed run.
//   block_sparse_attention_selection_amd/lib/msa_rates [hbm|launch|lds|mix|chain]...
#include <stdio.h>
#include <string.h>

#include "msa_tiles.hip"

namespace msa {
// the tile source's launchers reference the library's kernel timing hooks
ProfSpan profile_begin(int) { return ProfSpan{}; }
void profile_end(const ProfSpan&, bool) {}
}  // namespace msa

using namespace msa;

namespace {

constexpr double kClockHz = 2.4e9;

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

// best of three timed runs (ms) of launch(), after one untimed run
template <typename F>
float best_ms(F launch) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();
  float best = 1e30f;
  for (int r = 0; r < 3; ++r) {
    CHECK(hipEventRecord(a));
    launch();
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms;
    CHECK(hipEventElapsedTime(&ms, a, b));
    best = ms < best ? ms : best;
  }
  CHECK(hipGetLastError());
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return best;
}

// ---------------------------------------------------------------------------
// hbm: 8 loads in flight per lane, grid-strided over the buffer
// ---------------------------------------------------------------------------
template <bool NT>
__global__ __launch_bounds__(256) void k_stream(const u32x4* __restrict__ src, size_t n16, unsigned* out) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (size_t i = tid; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = NT ? __builtin_nontemporal_load(&src[i + u * stride]) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][3];
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads
}

void run_hbm() {
  const size_t bytes = (size_t)4 << 30;
  u32x4* src;
  unsigned* out;
  CHECK(hipMalloc(&src, bytes));
  CHECK(hipMalloc(&out, 64));
  CHECK(hipMemset(src, 1, bytes));
  const size_t n16 = bytes / 16;
  // the loop covers whole rounds of 8 x stride; the rest is not read
  const size_t stride = (size_t)8192 * 256, read16 = n16 / (8 * stride) * (8 * stride);
  const float tp = best_ms([&] { k_stream<false><<<8192, 256>>>(src, n16, out); });
  const float tn = best_ms([&] { k_stream<true><<<8192, 256>>>(src, n16, out); });
  printf("hbm    plain 16-byte loads            %8.1f GB/s\n", read16 * 16.0 / (tp * 1e-3) / 1e9);
  printf("hbm    non-temporal 16-byte loads     %8.1f GB/s\n", read16 * 16.0 / (tn * 1e-3) / 1e9);
  CHECK(hipFree(src));
  CHECK(hipFree(out));
}

// ---------------------------------------------------------------------------
// launch: an empty kernel, 1000 launches back to back
// ---------------------------------------------------------------------------
__global__ void k_empty() {}

void run_launch() {
  const int n = 1000;
  const float ms = best_ms([&] {
    for (int i = 0; i < n; ++i) k_empty<<<1, 64>>>();
  });
  printf("launch empty kernel, back to back     %8.2f us\n", ms * 1e3 / n);
}

// ---------------------------------------------------------------------------
// lds: the K-operand reads (one row per lane, pieces XOR-swizzled by row & 15)
// and the transposing V reads of the tile kernel, 8 KB per wave per iteration
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(512) void k_lds(unsigned* out, int iters) {
  __shared__ u32x4 s[4096];  // four 16 KB slots
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  for (int i = tid; i < 4096; i += blockDim.x) s[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    const int slot = (it & 3) * 1024;
    if (MODE == 0) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 v = s[slot + pieceK(c, 2 * st + h)];
        acc ^= v[0] + v[3];
      }
    } else {
      const char* vt = (const char*)(s + slot + kChunkU4);
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4 v = vfrag_at(vt, t, sp);
          acc ^= v[0] + v[3];
        }
    }
  }
  out[blockIdx.x * blockDim.x + tid] = acc;
}

void run_lds() {
  unsigned* out;
  CHECK(hipMalloc(&out, 256 * 512 * sizeof(unsigned)));
  const int iters = 8192;
  const float tk = best_ms([&] { k_lds<0><<<256, 512>>>(out, iters); });
  const float tv = best_ms([&] { k_lds<1><<<256, 512>>>(out, iters); });
  const double bytes = 8.0 * iters * 8192.0;  // per CU: 8 waves x 8 KB per iteration
  printf("lds    K rows, ds_read_b128            %8.1f B/clk/CU\n", bytes / (tk * 1e-3 * kClockHz));
  printf("lds    V^T, ds_read_b64_tr_b16         %8.1f B/clk/CU\n", bytes / (tv * 1e-3 * kClockHz));
  CHECK(hipFree(out));
}

// ---------------------------------------------------------------------------
// mix: per iteration 16 MFMAs (five accumulators), NF three-operand FMAs and
// NE exponentials on 16 independent chains; 8 waves per CU (two per SIMD)
// ---------------------------------------------------------------------------
template <int NF, int NE, bool MF>
__global__ __launch_bounds__(512, 1) void k_mix(float* out, int iters, float seed) {
  float x[16], y[16], z[16];
  for (int i = 0; i < 16; ++i) {
    x[i] = seed * (threadIdx.x + i);
    y[i] = seed * (i + 3) * 0.01f;
    z[i] = seed * i * 0.001f;
  }
  f32x16 acc[5];
  for (int j = 0; j < 5; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  u32x4 a = u32x4{__float_as_uint(seed), 1u, 2u, 3u}, b = u32x4{3u, 2u, 1u, __float_as_uint(seed)};
  asm volatile("" : "+v"(a), "+v"(b));
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(y[i]), "+v"(z[i]));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MF) acc[r % 5] = Mma32<bf16_t>::run(a, b, acc[r % 5]);
#pragma unroll
      for (int i = 0; i < NF / 16; ++i) {
        const int q = (r + 5 * i) & 15;
        x[q] = __builtin_fmaf(x[q], y[(q + 1) & 15], z[(q + 2) & 15]);
      }
#pragma unroll
      for (int i = 0; i < NE / 16; ++i) x[(r + 8 * i) & 15] = __builtin_amdgcn_exp2f(x[(r + 8 * i) & 15]);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += x[i];
  for (int j = 0; j < 5; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int NF, int NE, bool MF>
void mix_line(float* out, const char* name) {
  const int iters = 4000;
  const float ms = best_ms([&] { k_mix<NF, NE, MF><<<256, 512>>>(out, iters, 0.5f); });
  printf("mix    %-32s %8.0f cycles/iteration/SIMD\n", name, ms * 1e-3 * kClockHz / iters);
}

void run_mix() {
  float* out;
  CHECK(hipMalloc(&out, 256 * 512 * sizeof(float)));
  mix_line<0, 0, true>(out, "16 MFMA");
  mix_line<96, 0, false>(out, "96 FMA");
  mix_line<0, 32, false>(out, "32 exp");
  mix_line<96, 0, true>(out, "16 MFMA + 96 FMA");
  mix_line<0, 32, true>(out, "16 MFMA + 32 exp");
  mix_line<96, 16, true>(out, "16 MFMA + 96 FMA + 16 exp");
  CHECK(hipFree(out));
}

// ---------------------------------------------------------------------------
// chain: tile_iter, and a copy of it whose parts can be removed
// ---------------------------------------------------------------------------
enum { kNoLds = 1, kNoMfma = 2, kNoValu = 4, kNoBranch = 8, kOwn = 16 };

// The chunk iteration of the tile kernel (unmasked), stage for stage, with
// parts switched off: kNoLds takes the K and V fragments from registers,
// kNoMfma drops the products (keeping their operands live), kNoValu drops
// the softmax.
template <int VAR>
__device__ __forceinline__ float iter_parts(Rows32& rt, const f32x16& sc, const u32x4 (&pp)[2], const char* vprev,
                                            const u32x4 (&vpre)[2], const char* vcur, const u32x4* knext,
                                            uint32_t koff0, float sl2, f32x16& sn, u32x4 (&pn)[2],
                                            u32x4 (&vnext)[2]) {
  const uint32_t ka0 = lds_addr(knext) + koff0;
  auto kfrag = [&](int st) {
    return (VAR & kNoLds) ? rt.qb[(st + 3) & 7] : *(const lds_u32x4*)(uintptr_t)(ka0 ^ (32u * st));
  };
  auto vfrag = [&](int t, int sp) { return (VAR & kNoLds) ? rt.qb[(t + 2 * sp) & 7] : vfrag_at(vprev, t, sp); };
  const f32x16 sa = sc;
  u32x4 va[8], ka[8];
  va[0] = vpre[0];
  va[1] = vpre[1];
  ka[0] = kfrag(0);
#pragma unroll
  for (int j = 0; j < 16; ++j) sn[j] = 0.f;
  float cmax = 0.f, alpha = 1.f, nmu = 0.f, ls = 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i + 2 < 8) va[i + 2] = vfrag((i + 2) & 3, (i + 2) >> 2);
    if (i + 1 < 8) ka[i + 1] = kfrag(i + 1);
    if (!(VAR & kNoMfma)) {
      rt.o[i & 3] = Mma32<bf16_t>::run(va[i], pp[i >> 2], rt.o[i & 3]);
      if (i > 0) sn = Mma32<bf16_t>::run(ka[i - 1], rt.qb[i - 1], sn);
    } else {
      asm volatile("" ::"v"(va[i]), "v"(ka[i]));
    }
    if (!(VAR & kNoValu)) {
      if (i == 0) {
        cmax = hw_max3(hw_max3(hw_max3(sa[0], sa[1], sa[2]), sa[3], sa[4]), sa[5], sa[6]);
      } else if (i == 1) {
        cmax = hw_max3(hw_max3(hw_max3(cmax, sa[7], sa[8]), sa[9], sa[10]), sa[11], sa[12]);
        cmax = hw_max(hw_max3(cmax, sa[13], sa[14]), sa[15]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(cmax), __float_as_uint(cmax), false, false);
        cmax = hw_max(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sl2;
        const float m_new = cmax > rt.m + kRescale32 ? cmax : rt.m;
        alpha = m_new == rt.m ? 1.f : __builtin_amdgcn_exp2f(rt.m - m_new);
        rt.m = m_new;
        nmu = (m_new == -INFINITY) ? 0.f : -m_new;
      } else {
        const int q0 = i == 2 ? 0 : (i == 3 ? 2 : (i == 4 ? 3 : (i == 5 ? 4 : (i == 6 ? 6 : 7))));
        const int q1 = i == 2 ? 2 : (i == 3 ? 3 : (i == 4 ? 4 : (i == 5 ? 6 : (i == 6 ? 7 : 8))));
#pragma unroll
        for (int q = q0; q < q1; ++q) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * q], sl2, nmu));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[2 * q + 1], sl2, nmu));
          pn[q >> 2][q & 3] = pack2<bf16_t>(p0, p1);
          ls = q == 0 ? p0 + p1 : ls + (p0 + p1);
        }
      }
    } else if (i == 7) {
      pn[0] = u32x4{__float_as_uint(sa[0]), 0u, 0u, 0u};
      pn[1] = pn[0];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!(VAR & kNoMfma)) {
    sn = Mma32<bf16_t>::run(ka[7], rt.qb[7], sn);
  } else {
    asm volatile("" ::"v"(ka[7]));
#pragma unroll
    for (int j = 0; j < 16; ++j) sn[j] = sa[j] * 0.5f;
  }
  vnext[0] = (VAR & kNoLds) ? rt.qb[1] : vfrag_at(vcur, 0, 0);
  vnext[1] = (VAR & kNoLds) ? rt.qb[2] : vfrag_at(vcur, 1, 0);
  asm volatile("" ::"v"(pn[0]), "v"(pn[1]), "v"(ls));
  rt.l = __builtin_fmaf(rt.l, alpha, ls);
  return alpha;
}

// 8 waves of 32 rows (one workgroup per CU, as the tile kernel), an 8-slot
// ring of bf16 K/V chunks, one barrier per chunk
template <int VAR>
__global__ __launch_bounds__(512, 1) void k_chain(float* out, int steps, uint32_t seed) {
  __shared__ __attribute__((aligned(256))) u32x4 ring[8 * kSlotU4];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 8 * kSlotU4; i += 512) {
    uint32_t w[4];
    for (int e = 0; e < 4; ++e) {
      uint32_t x = (uint32_t)(i * 4 + e) * 2654435761u ^ seed;
      x ^= x >> 13;
      x *= 0x5bd1e995u;
      w[e] = pack2<bf16_t>((x & 0xffff) / 32768.f - 1.f, (x >> 16) / 32768.f - 1.f);  // values in [-1, 1)
    }
    ring[i] = u32x4{w[0], w[1], w[2], w[3]};
  }
  __syncthreads();
  Rows32 rt;
  rows_reset(rt);
  rt.pos = INT_MAX;
  rt.seq = 0;
  for (int s = 0; s < 8; ++s) rt.qb[s] = ring[(s * 64 + lane + 7 * (tid >> 6)) & 1023];
  struct Pipe {
    f32x16 sc;
    u32x4 pp[2];
    u32x4 vpre[2];
  } A, B;
  for (int j = 0; j < 16; ++j) A.sc[j] = 0.f;
  A.pp[0] = A.pp[1] = u32x4{0u, 0u, 0u, 0u};
  A.vpre[0] = A.vpre[1] = ring[lane];
  const float sl2 = 0.1275f;  // 128^-0.5 * log2(e)
  const uint32_t koff0 = k_lane_offset0();
  auto slot = [&](int ci) { return ring + (ci & 7) * kSlotU4; };
  auto step = [&](int ci, const Pipe& in, Pipe& o) {
    loop_barrier();
    const char* vprev = (const char*)(slot(ci + 7) + kChunkU4);
    const char* vcur = (const char*)(slot(ci) + kChunkU4);
    const u32x4* knext = slot(ci + 1);
    float alpha;
    if (VAR & kOwn)
      alpha = tile_iter<bf16_t, false>(rt, in.sc, in.pp, vprev, in.vpre, vcur, knext, koff0, 0, 32, sl2, o.sc, o.pp,
                                       o.vpre);
    else
      alpha = iter_parts<VAR>(rt, in.sc, in.pp, vprev, in.vpre, vcur, knext, koff0, sl2, o.sc, o.pp, o.vpre);
    if (VAR & kNoBranch)
      rt.l += alpha;  // no rescale branch
    else
      rows_rescale(rt, alpha);
  };
  for (int ci = 0; ci < steps; ci += 2) {
    step(ci, A, B);
    step(ci + 1, B, A);
  }
  float s = rt.l + rt.m;
  for (int t = 0; t < 4; ++t)
    for (int j = 0; j < 16; ++j) s += rt.o[t][j];
  out[blockIdx.x * 512 + tid] = s;
}

template <int VAR>
void chain_line(float* out, const char* name) {
  const int steps = 4000;
  const float ms = best_ms([&] { k_chain<VAR><<<256, 512>>>(out, steps, 1u); });
  // each SIMD runs two waves, each doing one iteration per step
  const double cyc = ms * 1e-3 * kClockHz / steps;
  printf("chain  %-32s %8.0f cycles/chunk/SIMD\n", name, cyc);
}

void run_chain() {
  float* out;
  CHECK(hipMalloc(&out, 256 * 512 * sizeof(float)));
  chain_line<kOwn>(out, "tile_iter (the kernel's own)");
  chain_line<0>(out, "copy");
  chain_line<kNoLds>(out, "copy, K/V from registers");
  chain_line<kNoLds | kNoBranch>(out, "... and no rescale branch");
  chain_line<kNoValu>(out, "copy, no softmax (MFMA + LDS)");
  chain_line<kNoValu | kNoLds>(out, "MFMA only");
  chain_line<kNoMfma | kNoLds>(out, "softmax only");
  chain_line<kNoMfma | kNoValu>(out, "LDS reads only");
  CHECK(hipFree(out));
}

}  // namespace

int main(int argc, char** argv) {
  const char* all[] = {"hbm", "launch", "lds", "mix", "chain"};
  const int n = argc > 1 ? argc - 1 : 5;
  for (int i = 0; i < n; ++i) {
    const char* what = argc > 1 ? argv[i + 1] : all[i];
    if (!strcmp(what, "hbm")) run_hbm();
    else if (!strcmp(what, "launch")) run_launch();
    else if (!strcmp(what, "lds")) run_lds();
    else if (!strcmp(what, "mix")) run_mix();
    else if (!strcmp(what, "chain")) run_chain();
    else {
      fprintf(stderr, "unknown measurement %s (hbm, launch, lds, mix, chain)\n", what);
      return 2;
    }
    fflush(stdout);
  }
  return 0;
}
