/*
 * msa_oracle.c -- plain fp64 CPU oracle for MiniMax-M3 block-sparse attention.
 *
 * TEST INFRASTRUCTURE. This file is the correctness reference that the GPU
 * library is compared against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code, header, table or
 * helper with the HIP library, and the HIP library never loads it.
 *
 * What it computes (fw-ai/minimax-kernels README, intro and "Quick start"):
 * every query token of every sequence, and every query head, attends only to
 * the key positions inside the 128-token blocks that the token selected for
 * the head's KV head. Keys and values are read through the sequence's
 * logical-to-physical page table from a paged cache laid out as
 * [num_pages, Hkv, page_size, 128]. The pass returns O [Tq, Hq, 128] and the
 * fp32 log-sum-exp laid out as [Hq, Tq] (README "Quick start", last
 * paragraph). The KV-outer formulation of the README intro reorganises the
 * same sum, so the oracle is the plain definition written out:
 *
 *   for each sequence s with L = used_kv_lens[s] and tokens [cu[s], cu[s+1]):
 *     pos(t) = L - Tq_s + (t - cu[s])            (bottom-right causal alignment)
 *     J(t,g)  = union over picks b = selected[t,g,k] with 0 <= b < ceil(L/128)
 *               of { j : 128b <= j < min(128b+128, L), and j <= pos(t) if causal }
 *     for every head h with h / G == g (G = Hq / Hkv):
 *       x_j = scale * <q[t,h,:], K(s,g,j)>,   scale = 1/sqrt(128)
 *       lse = max x + ln sum_j exp(x_j - max x)
 *       O   = sum_j exp(x_j - lse) * V(s,g,j)
 *   K(s,g,j) = k_cache[block_tables[s, j / P], g, j % P, :]   (same for V)
 *   An empty J gives O = 0 and lse = -inf.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): selected is [Tq, Hkv, K] token-major like q; a block id names
 * logical tokens [128b, 128b+128) whatever the page size; query head h
 * belongs to KV head h / G; causal masking is aligned bottom-right; the
 * scale is fixed at 1/sqrt(128); lse is the natural log with the scale
 * included; ids outside [0, ceil(L/128)) are ignored; a repeated id within
 * one (t, g) list and a page id outside [0, num_pages) are precondition
 * violations that the oracle reports instead of computing.
 *
 * Stored values are decoded exactly to fp64 from their bit patterns:
 *   bf16  -- the upper half of an IEEE-754 binary32;
 *   fp16  -- IEEE-754 binary16 (bias 15, subnormals, inf, NaN);
 *   e4m3fn -- OCP 8-bit float: bias 7, 3 mantissa bits, subnormals, no
 *             infinities, NaN only for the all-ones exponent and mantissa.
 *             The fp8 cache values follow the cast rule of the sglang pull
 *             request "Speed up MiniMax-M3 sparse attention on Hopper",
 *             section "Verification" (clamp to +-448, then round to e4m3fn).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC msa_oracle.c -o libmsa_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of the oracle's own interface (mirrored only by oracle/__init__.py) */
enum {
  ORC_BF16 = 0,
  ORC_FP16 = 1,
  ORC_FP8_E4M3FN = 2,
  ORC_FP32 = 3,
};

/* return codes */
enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,
  ORC_ERR_DUPLICATE_PICK = -2,
  ORC_ERR_PAGE_RANGE = -3,
  ORC_ERR_NOMEM = -4,
};

#define ORC_D 128
#define ORC_BLK 128

static double orc_decode_bf16(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double orc_decode_fp16(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 0x1F;
  int m = bits & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-10 * 2^-14 */
  } else if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  }
  return sign ? -v : v;
}

static double orc_decode_e4m3fn(uint8_t bits) {
  int sign = (bits >> 7) & 1;
  int e = (bits >> 3) & 0xF;
  int m = bits & 0x7;
  double v;
  if (e == 15 && m == 7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  } else {
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  }
  return sign ? -v : v;
}

static double orc_decode_one(int dtype, const void* base, int64_t idx) {
  switch (dtype) {
    case ORC_BF16: return orc_decode_bf16(((const uint16_t*)base)[idx]);
    case ORC_FP16: return orc_decode_fp16(((const uint16_t*)base)[idx]);
    case ORC_FP8_E4M3FN: return orc_decode_e4m3fn(((const uint8_t*)base)[idx]);
    case ORC_FP32: return (double)((const float*)base)[idx];
    default: return NAN;
  }
}

/* Decode n stored values of the given dtype into fp64 (used to pin the
 * decoders against an independent conversion routine). */
int msa_oracle_decode(int dtype, const void* src, int64_t n, double* dst) {
  if (!src || !dst || n < 0) return ORC_ERR_ARG;
  if (dtype < ORC_BF16 || dtype > ORC_FP32) return ORC_ERR_ARG;
  for (int64_t i = 0; i < n; ++i) dst[i] = orc_decode_one(dtype, src, i);
  return ORC_OK;
}

/* Sequence that owns token t, or -1 when t lies in no sequence. */
static int orc_seq_of(const int64_t* cu, int B, int64_t t) {
  for (int s = 0; s < B; ++s)
    if (cu[s] <= t && t < cu[s + 1]) return s;
  return -1;
}

/*
 * msa_oracle_attention
 *
 * q            [Tq, Hq, 128] of q_dtype (bf16 or fp16 or fp32)
 * k_cache      [num_pages, Hkv, page_size, 128] of kv_dtype
 * v_cache      same layout and dtype as k_cache
 * selected     [Tq, Hkv, topk] int32 logical block ids
 * block_tables [B, max_pages] int32 physical page per logical page
 * cu_seqlens_q [B + 1] int64
 * used_kv_lens [B] int32
 * pairs        NULL for every (t, g); otherwise n_pairs ids t*Hkv + g
 * out          [n_pairs][G][128] fp64 (n_pairs = Tq*Hkv when pairs is NULL,
 *              which is exactly the [Tq, Hq, 128] layout)
 * lse          [n_pairs][G] fp64 natural-log LSE (NULL: not returned)
 * num_threads  <= 0: OpenMP default
 *
 * Returns ORC_OK, or a negative code for a bad argument or a violated
 * precondition (repeated block id in one list, page id out of range).
 */
int msa_oracle_attention(const void* q, int q_dtype, int64_t Tq, int Hq,
                         const void* k_cache, const void* v_cache, int kv_dtype,
                         int64_t num_pages, int Hkv, int page_size,
                         const int32_t* selected, int topk,
                         const int32_t* block_tables, int B, int64_t max_pages,
                         const int64_t* cu_seqlens_q, const int32_t* used_kv_lens,
                         int causal, double scale,
                         const int64_t* pairs, int64_t n_pairs,
                         double* out, double* lse, int num_threads) {
  if (!q || !k_cache || !v_cache || !selected || !block_tables || !cu_seqlens_q ||
      !used_kv_lens || !out)
    return ORC_ERR_ARG;
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || topk <= 0 || page_size <= 0 || B < 0 ||
      Tq < 0)
    return ORC_ERR_ARG;
  if (!pairs) n_pairs = Tq * Hkv;
  const int G = Hq / Hkv;
  int64_t max_len = 0;
  for (int s = 0; s < B; ++s)
    if (used_kv_lens[s] > max_len) max_len = used_kv_lens[s];

  int status = ORC_OK;
  /* the thread count applies to this call only (a num_threads clause, not
     the process-wide setting) */
  int nthr = 1;
#ifdef _OPENMP
  nthr = num_threads > 0 ? num_threads : omp_get_max_threads();
#endif
  (void)nthr;

#pragma omp parallel num_threads(nthr)
  {
    /* per-thread scratch: the key set of one (t, g) and its scores */
    unsigned char* mark = (unsigned char*)malloc((size_t)(max_len > 0 ? max_len : 1));
    int64_t* J = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_len > 0 ? max_len : 1));
    double* x = (double*)malloc(sizeof(double) * (size_t)G * (size_t)(max_len > 0 ? max_len : 1));
    double* qd = (double*)malloc(sizeof(double) * (size_t)G * ORC_D);
    double kv[ORC_D];
    int64_t* seen = (int64_t*)malloc(sizeof(int64_t) * (size_t)topk);
    if (!mark || !J || !x || !qd || !seen) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
    }

#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < n_pairs; ++p) {
      if (!mark || !J || !x || !qd || !seen) continue;
      int64_t pid = pairs ? pairs[p] : p;
      int64_t t = pid / Hkv;
      int g = (int)(pid % Hkv);
      double* o_row = out + (size_t)p * G * ORC_D;
      double* l_row = lse ? lse + (size_t)p * G : NULL;
      if (t < 0 || t >= Tq) {
#pragma omp atomic write
        status = ORC_ERR_ARG;
        continue;
      }

      /* 1. the key set J(t, g) */
      int64_t nJ = 0;
      int s = orc_seq_of(cu_seqlens_q, B, t);
      int64_t L = 0;
      if (s >= 0) {
        L = used_kv_lens[s];
        int64_t Tq_s = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        int64_t pos = L - Tq_s + (t - cu_seqlens_q[s]);
        int64_t nblk = (L + ORC_BLK - 1) / ORC_BLK;
        memset(mark, 0, (size_t)(L > 0 ? L : 0));
        const int32_t* sel = selected + ((size_t)t * Hkv + g) * topk;
        int nseen = 0;
        for (int k = 0; k < topk; ++k) {
          int64_t b = sel[k];
          if (b < 0 || b >= nblk) continue;
          for (int i = 0; i < nseen; ++i)
            if (seen[i] == b) {
#pragma omp atomic write
              status = ORC_ERR_DUPLICATE_PICK;
            }
          seen[nseen++] = b;
          int64_t j1 = ORC_BLK * b + ORC_BLK;
          if (j1 > L) j1 = L;
          for (int64_t j = ORC_BLK * b; j < j1; ++j)
            if (!causal || j <= pos) mark[j] = 1;
        }
        for (int64_t j = 0; j < L; ++j)
          if (mark[j]) J[nJ++] = j;
      }

      if (nJ == 0) {
        memset(o_row, 0, sizeof(double) * (size_t)G * ORC_D);
        if (l_row)
          for (int r = 0; r < G; ++r) l_row[r] = -INFINITY;
        continue;
      }

      /* 2. decoded queries of the G heads of KV head g */
      for (int r = 0; r < G; ++r) {
        int64_t h = (int64_t)g * G + r;
        for (int d = 0; d < ORC_D; ++d)
          qd[r * ORC_D + d] = orc_decode_one(q_dtype, q, (t * Hq + h) * ORC_D + d);
      }

      /* 3. scores x_j = scale * <q, K_j> */
      int bad_page = 0;
      for (int64_t i = 0; i < nJ; ++i) {
        int64_t j = J[i];
        int64_t lp = j / page_size;
        int64_t page = (lp < max_pages) ? block_tables[(size_t)s * max_pages + lp] : -1;
        if (page < 0 || page >= num_pages) {
          bad_page = 1;
          break;
        }
        int64_t base = ((page * Hkv + g) * page_size + (j % page_size)) * ORC_D;
        for (int d = 0; d < ORC_D; ++d) kv[d] = orc_decode_one(kv_dtype, k_cache, base + d);
        for (int r = 0; r < G; ++r) {
          double acc = 0.0;
          for (int d = 0; d < ORC_D; ++d) acc += qd[r * ORC_D + d] * kv[d];
          x[(size_t)r * nJ + i] = scale * acc;
        }
      }
      if (bad_page) {
#pragma omp atomic write
        status = ORC_ERR_PAGE_RANGE;
        continue;
      }

      /* 4. softmax statistics per head */
      for (int r = 0; r < G; ++r) {
        const double* xr = x + (size_t)r * nJ;
        double m = -INFINITY;
        for (int64_t i = 0; i < nJ; ++i)
          if (xr[i] > m) m = xr[i];
        double l = 0.0;
        for (int64_t i = 0; i < nJ; ++i) l += exp(xr[i] - m);
        double lse_r = m + log(l);
        if (l_row) l_row[r] = lse_r;
        /* store the normalised weights in place of the scores */
        double* wr = x + (size_t)r * nJ;
        for (int64_t i = 0; i < nJ; ++i) wr[i] = exp(xr[i] - m) / l;
      }

      /* 5. O = sum_j w_j * V_j */
      memset(o_row, 0, sizeof(double) * (size_t)G * ORC_D);
      for (int64_t i = 0; i < nJ; ++i) {
        int64_t j = J[i];
        int64_t page = block_tables[(size_t)s * max_pages + j / page_size];
        int64_t base = ((page * Hkv + g) * page_size + (j % page_size)) * ORC_D;
        for (int d = 0; d < ORC_D; ++d) kv[d] = orc_decode_one(kv_dtype, v_cache, base + d);
        for (int r = 0; r < G; ++r) {
          double w = x[(size_t)r * nJ + i];
          double* o = o_row + (size_t)r * ORC_D;
          for (int d = 0; d < ORC_D; ++d) o[d] += w * kv[d];
        }
      }
    }
    free(mark);
    free(J);
    free(x);
    free(qd);
    free(seen);
  }
  return status;
}

/* Threads the OpenMP runtime would use (reported with CPU timings). */
int msa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
