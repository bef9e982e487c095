// Host-side checks of the C ABI, built together with the library under
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
// tests/test_sanitize_host.py. Every call here is refused by host validation
// or needs no device: nothing is launched. Exits 0 when every expectation
// holds; the sanitizers abort the process on any memory or UB error.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "msa_kvouter.h"

static int g_bad = 0;
#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
              msa_last_error());                                        \
      ++g_bad;                                                          \
    }                                                                   \
  } while (0)

static char g_arena[1 << 16] __attribute__((aligned(256)));  // never dereferenced by the library here

static msa_tensor T(int dtype, int ndim, long a, long b = 0, long c = 0, long d = 0, size_t off = 0) {
  msa_tensor t;
  memset(&t, 0, sizeof t);
  t.data = g_arena + off;
  t.dtype = dtype;
  t.ndim = ndim;
  t.shape[0] = a;
  t.shape[1] = b;
  t.shape[2] = c;
  t.shape[3] = d;
  return t;
}

struct Call {
  msa_tensor q, k, v, sel, bt, cu, used, out, lse;
  int page, causal;
};

static Call good(long Tq = 4, long Hq = 16, long Hkv = 2, long NP = 8, long P = 64, long K = 4, long B = 2,
                 long MP = 4) {
  Call c;
  c.q = T(MSA_BF16, 3, Tq, Hq, 128);
  c.k = T(MSA_BF16, 4, NP, Hkv, P, 128);
  c.v = T(MSA_BF16, 4, NP, Hkv, P, 128);
  c.sel = T(MSA_INT32, 3, Tq, Hkv, K);
  c.bt = T(MSA_INT32, 2, B, MP);
  c.cu = T(MSA_INT64, 1, B + 1);
  c.used = T(MSA_INT32, 1, B);
  c.out = T(MSA_BF16, 3, Tq, Hq, 128);
  c.lse = T(MSA_FP32, 2, Hq, Tq);
  c.page = (int)P;
  c.causal = 1;
  return c;
}

static int attn(Call& c) {
  return msa_kvouter_attention(&c.q, &c.k, &c.v, &c.sel, &c.bt, &c.cu, &c.used, c.page, c.causal, &c.out, &c.lse,
                               nullptr);
}

static int attn_ws(Call& c, void* ws, size_t n) {
  return msa_kvouter_attention_ws(&c.q, &c.k, &c.v, &c.sel, &c.bt, &c.cu, &c.used, c.page, c.causal, &c.out,
                                  &c.lse, ws, n, nullptr);
}

int main() {
  EXPECT(strstr(msa_version(), "gfx950") != nullptr);
  // descriptor errors, each refused before any device call
  {
    Call c = good();
    c.q = T(MSA_FP8_E4M3FN, 3, 4, 16, 128);
    EXPECT(attn(c) == MSA_ERR_UNSUPPORTED && strlen(msa_last_error()) > 0);
  }
  {
    Call c = good();
    c.q.shape[2] = 64;
    EXPECT(attn(c) == MSA_ERR_UNSUPPORTED);
  }
  {
    Call c = good();
    c.sel.shape[2] = 65;
    EXPECT(attn(c) == MSA_ERR_UNSUPPORTED);
  }
  {
    Call c = good();
    c.k.data = g_arena + 8;  // misaligned
    EXPECT(attn(c) == MSA_ERR_INVALID_ARGUMENT);
  }
  {
    Call c = good();
    c.cu = T(MSA_INT64, 1, 5);
    EXPECT(attn(c) == MSA_ERR_INVALID_ARGUMENT);
  }
  {
    Call c = good();
    EXPECT(msa_kvouter_attention(nullptr, &c.k, &c.v, &c.sel, &c.bt, &c.cu, &c.used, 64, 1, &c.out, nullptr,
                                 nullptr) == MSA_ERR_INVALID_ARGUMENT);
    EXPECT(attn_ws(c, nullptr, 1 << 20) == MSA_ERR_INVALID_ARGUMENT);
    EXPECT(attn_ws(c, g_arena + 64, 1 << 20) == MSA_ERR_INVALID_ARGUMENT);
  }
  {
    Call c = good(0);
    EXPECT(attn(c) == MSA_OK);  // nothing to do
  }
  // the size query reads shapes only: data pointers may be null
  {
    Call c = good(64, 64, 8, 64, 64, 16, 64, 512);
    c.q.data = c.k.data = c.v.data = c.sel.data = c.bt.data = c.cu.data = c.used.data = nullptr;
    size_t n = 0;
    EXPECT(msa_kvouter_workspace_bytes(&c.q, &c.k, &c.v, &c.sel, &c.bt, &c.cu, &c.used, 64, 1, &n) == MSA_OK);
    EXPECT(n > 0 && n < 200000);
    EXPECT(msa_kvouter_workspace_bytes(&c.q, &c.k, &c.v, &c.sel, &c.bt, &c.cu, &c.used, 64, 1, nullptr) ==
           MSA_ERR_INVALID_ARGUMENT);
    Call p = good(16384, 64, 8, 128, 128, 16, 1, 128);
    EXPECT(msa_kvouter_workspace_bytes(&p.q, &p.k, &p.v, &p.sel, &p.bt, &p.cu, &p.used, 128, 1, &n) == MSA_OK);
    EXPECT(n > 4000000000ull);
  }
  // the other entry points' argument checks
  {
    msa_tensor sel = T(MSA_INT32, 3, 4, 2, 4), cu = T(MSA_INT64, 1, 3), used = T(MSA_INT32, 1, 2);
    EXPECT(msa_build_index(&sel, &cu, &used, 15, 4, 0, 8, 8, 0, nullptr, nullptr) == MSA_ERR_INVALID_ARGUMENT);
    EXPECT(msa_widen_fp8(nullptr, 16, MSA_BF16, g_arena, nullptr) == MSA_ERR_INVALID_ARGUMENT);
    EXPECT(msa_widen_fp8(g_arena, 15, MSA_BF16, g_arena, nullptr) == MSA_ERR_INVALID_ARGUMENT);
    msa_tensor kn = T(MSA_FP32, 3, 8, 2, 128), loc = T(MSA_INT64, 1, 8), kc = T(MSA_FP8_E4M3FN, 4, 4, 2, 64, 128);
    EXPECT(msa_store_kv(&kn, nullptr, &loc, &kc, nullptr, 64, nullptr) == MSA_ERR_INVALID_ARGUMENT);
    msa_tensor qi = T(MSA_BF16, 3, 4, 2, 128), ki = T(MSA_FP8_E4M3FN, 4, 8, 2, 64, 128), bt = T(MSA_INT32, 2, 2, 4);
    msa_tensor s2 = T(MSA_INT32, 3, 4, 2, 4);
    EXPECT(msa_select_blocks(&qi, &ki, &bt, &cu, &used, 64, 1, 0, 1, &s2, nullptr, nullptr) ==
           MSA_ERR_INVALID_ARGUMENT);
    EXPECT(msa_set_workspace_limit(1 << 20) == MSA_OK);
    EXPECT(msa_set_workspace_limit(0) == MSA_OK);
    double ms = 0;
    long long n = 0;
    EXPECT(msa_profile_collect(99, &ms, (int64_t*)&n) == MSA_ERR_INVALID_ARGUMENT);
  }
  // a well-formed call on a host without a usable device: an error, no crash
  {
    int ndev = 0;
    if (getenv("MSA_EXPECT_NO_DEVICE")) {
      Call c = good();
      EXPECT(attn(c) == MSA_ERR_HIP);
      (void)ndev;
    }
  }
  if (g_bad) fprintf(stderr, "%d expectation(s) failed\n", g_bad);
  else printf("abi host checks passed\n");
  return g_bad ? 1 : 0;
}
