// msa_api.hip -- the C ABI: descriptor validation, workspace, launches.
//
// Entry points and their contracts are declared in include/msa_kvouter.h.
// Validation reads shapes only (no device memory), runs before anything is
// enqueued, and never falls back to another path.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/msa_kvouter.h"
#include "msa_internal.hpp"

namespace {

// message of the last failing call on this thread (a fixed buffer: no call
// path allocates host memory)
thread_local char g_err[512];

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return MSA_OK;
}

const char* dname(int32_t d) {
  switch (d) {
    case MSA_BF16: return "bf16";
    case MSA_FP16: return "fp16";
    case MSA_FP8_E4M3FN: return "fp8_e4m3fn";
    case MSA_FP32: return "fp32";
    case MSA_INT32: return "int32";
    case MSA_INT64: return "int64";
    case MSA_UINT8: return "uint8";
    default: return "unknown";
  }
}

int64_t numel(const msa_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// need_data: the buffer must be present and aligned (off for shape-only queries)
int32_t check_tensor(const msa_tensor* t, const char* name, int ndim, int32_t dtype, size_t align,
                     bool need_data = true) {
  if (!t) return fail(MSA_ERR_INVALID_ARGUMENT, "%s: null descriptor", name);
  if (t->ndim != ndim) return fail(MSA_ERR_INVALID_ARGUMENT, "%s: expected rank %d, got %d", name, ndim, t->ndim);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(MSA_ERR_INVALID_ARGUMENT, "%s: negative extent", name);
  if (dtype >= 0 && t->dtype != dtype)
    return fail(MSA_ERR_INVALID_ARGUMENT, "%s: expected %s, got %s", name, dname(dtype), dname(t->dtype));
  if (need_data && numel(t) > 0) {
    if (!t->data) return fail(MSA_ERR_INVALID_ARGUMENT, "%s: null data pointer", name);
    if (((uintptr_t)t->data) % align) return fail(MSA_ERR_INVALID_ARGUMENT, "%s: data not %zu-byte aligned", name, align);
  }
  return MSA_OK;
}

struct Dims {
  int Tq, Hq, Hkv, G, K, B, MP, P, NP, nb_max, NR, W, T, Tu;
  int q_elem, kv_elem;
};

int elem_of(int32_t d) {
  return d == MSA_BF16 ? msa::kElemBF16 : d == MSA_FP16 ? msa::kElemF16 : msa::kElemFP8;
}

int32_t validate(const msa_tensor* q, const msa_tensor* k, const msa_tensor* v, const msa_tensor* sel,
                 const msa_tensor* bt, const msa_tensor* cu, const msa_tensor* used, int32_t page_size,
                 int32_t causal, const msa_tensor* out, const msa_tensor* lse, Dims* d, bool nd = true) {
  int32_t rc;
  if ((rc = check_tensor(q, "q", 3, -1, 16, nd))) return rc;
  if (q->dtype == MSA_FP8_E4M3FN) return fail(MSA_ERR_UNSUPPORTED, "q: fp8 queries are not supported");
  if (q->dtype != MSA_BF16 && q->dtype != MSA_FP16)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q: dtype must be bf16 or fp16, got %s", dname(q->dtype));
  if (q->shape[2] != 128) return fail(MSA_ERR_UNSUPPORTED, "q: head dim %lld, only 128 is supported", (long long)q->shape[2]);
  if ((rc = check_tensor(k, "k_cache", 4, -1, 16, nd))) return rc;
  if ((rc = check_tensor(v, "v_cache", 4, -1, 16, nd))) return rc;
  if (k->dtype != q->dtype && k->dtype != MSA_FP8_E4M3FN)
    return fail(k->dtype == MSA_BF16 || k->dtype == MSA_FP16 ? MSA_ERR_UNSUPPORTED : MSA_ERR_INVALID_ARGUMENT,
                "k_cache: dtype %s must equal q's (%s) or be fp8_e4m3fn", dname(k->dtype), dname(q->dtype));
  if (v->dtype != k->dtype) return fail(MSA_ERR_INVALID_ARGUMENT, "v_cache: dtype differs from k_cache");
  for (int i = 0; i < 4; ++i)
    if (v->shape[i] != k->shape[i]) return fail(MSA_ERR_INVALID_ARGUMENT, "v_cache: shape differs from k_cache");
  if (k->shape[3] != 128) return fail(MSA_ERR_UNSUPPORTED, "k_cache: head dim %lld, only 128 is supported", (long long)k->shape[3]);
  if (page_size != 64 && page_size != 128) return fail(MSA_ERR_UNSUPPORTED, "page_size %d: only 64 and 128 are supported", page_size);
  if (k->shape[2] != page_size)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_cache: page dimension %lld != page_size %d", (long long)k->shape[2], page_size);
  if ((rc = check_tensor(sel, "selected", 3, MSA_INT32, 4, nd))) return rc;
  if ((rc = check_tensor(bt, "block_tables", 2, MSA_INT32, 4, nd))) return rc;
  if ((rc = check_tensor(cu, "cu_seqlens_q", 1, MSA_INT64, 8, nd))) return rc;
  if ((rc = check_tensor(used, "used_kv_lens", 1, MSA_INT32, 4, nd))) return rc;
  if (causal != 0 && causal != 1) return fail(MSA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  const int64_t Tq = q->shape[0], Hq = q->shape[1], Hkv = k->shape[1], NP = k->shape[0];
  const int64_t B = bt->shape[0], MP = bt->shape[1];
  if (Hkv <= 0 || Hq <= 0) return fail(MSA_ERR_INVALID_ARGUMENT, "head counts must be positive");
  if (Hq % Hkv) return fail(MSA_ERR_INVALID_ARGUMENT, "Hq (%lld) is not a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (Hq / Hkv > 128) return fail(MSA_ERR_UNSUPPORTED, "Hq/Hkv = %lld exceeds 128", (long long)(Hq / Hkv));
  if (sel->shape[0] != Tq || sel->shape[1] != Hkv)
    return fail(MSA_ERR_INVALID_ARGUMENT, "selected: shape must be [Tq=%lld, Hkv=%lld, topk]", (long long)Tq, (long long)Hkv);
  const int64_t K = sel->shape[2];
  if (K < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "selected: topk must be >= 1");
  if (K > 64) return fail(MSA_ERR_UNSUPPORTED, "selected: topk %lld exceeds 64", (long long)K);
  if (cu->shape[0] != B + 1) return fail(MSA_ERR_INVALID_ARGUMENT, "cu_seqlens_q: expected %lld entries", (long long)(B + 1));
  if (used->shape[0] != B) return fail(MSA_ERR_INVALID_ARGUMENT, "used_kv_lens: expected %lld entries", (long long)B);
  if (B > 0 && MP < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "block_tables: max_pages must be >= 1");
  if (out) {
    if ((rc = check_tensor(out, "out", 3, q->dtype, 16, nd))) return rc;
    if (out->shape[0] != Tq || out->shape[1] != Hq || out->shape[2] != 128)
      return fail(MSA_ERR_INVALID_ARGUMENT, "out: shape must equal q's");
  }
  if (lse) {
    if ((rc = check_tensor(lse, "lse", 2, MSA_FP32, 4, nd))) return rc;
    if (lse->shape[0] != Hq || lse->shape[1] != Tq) return fail(MSA_ERR_INVALID_ARGUMENT, "lse: shape must be [Hq, Tq]");
  }
  // int32 indexing limits of the kernels
  const int64_t nb_max = (MP * page_size + 127) / 128;
  if (Tq * Hkv * K >= (1ll << 31) || Tq >= (1ll << 30) || B >= (1 << 30) || NP >= (1ll << 31) ||
      nb_max * Hkv >= (1ll << 30) || MP * page_size >= (1ll << 31) || Tq * Hq >= (1ll << 31))
    return fail(MSA_ERR_UNSUPPORTED, "problem too large for 32-bit indices");
  d->Tq = (int)Tq;
  d->Hq = (int)Hq;
  d->Hkv = (int)Hkv;
  d->G = (int)(Hq / Hkv);
  d->K = (int)K;
  d->B = (int)B;
  d->MP = (int)MP;
  d->P = page_size;
  d->NP = (int)NP;
  d->nb_max = (int)std::max<int64_t>(nb_max, 1);
  d->NR = d->nb_max * d->Hkv;
  d->W = (int)((Tq + 31) / 32);
  // tiles of up to 256 query rows (the tile kernel's 8 waves x 32 rows), at
  // most 128 tokens; unit kernel pieces of up to 128 rows, windows of up to
  // 8 pieces' worth of tokens
  d->T = std::min(128, std::max(1, 256 / d->G));
  d->Tu = std::min(8 * std::max(1, 128 / d->G), msa::kUnitWindowTokens);
  d->q_elem = elem_of(q->dtype);
  d->kv_elem = elem_of(k->dtype);
  return MSA_OK;
}

// ---------------------------------------------------------------------------
// workspace
//
// A call needs three kinds of device memory besides its inputs and outputs:
//   - a counter set (work-queue heads, totals), zero when the call starts;
//   - the residual token bitmaps (one bit per (row, token)), zero when the
//     call starts; only calls that may have residual slots use them;
//   - planning arrays and, for calls that may have residual slots, the
//     KV-outer partial results (layout() below).
// Absent chunks read a page of zeros, a static device array that is never
// written.
//
// The library-owned workspace (msa_kvouter_attention) keeps two counter sets
// used on alternate calls and a bitmap that every call leaves zeroed, so no
// fill runs per call; it grows on demand (synchronising the device once).
// A caller-owned workspace (msa_kvouter_attention_ws) holds one counter set
// and the bitmap at its start, cleared by a fill kernel at the start of
// every call that uses them.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t g_zero_page[msa::kZeroPageBytes] = {};

// Scratch of msa_kvouter_attention_noalloc: one array per device, held until
// the process ends. Host code never uses the array's name as a device
// address: each device's address is resolved once with hipGetSymbolAddress
// (DeviceState::scratch) and only that address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

struct Carve {
  size_t off = 0;
  template <typename T>
  T* take(char* base, size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Lays the planning and partial arrays out in `base` (or only sizes them when
// base is null). Returns the bytes used. `residual`: the arrays of the
// residual inversion (bitmap copies and prefixes, the residual order);
// `with_partials`: the KV-outer partials and the tile tables. Calls whose
// tiles are all finished by the front kernel (front_only) need neither.
size_t layout(const Dims& d, char* base, msa::Params* p, bool residual, bool with_partials) {
  Carve c;
  const size_t nslots = (size_t)d.Tq * d.Hkv * d.K;
  const size_t TG = (size_t)d.Tq * d.Hkv;
  const size_t words = (size_t)d.NR * d.W;
  p->wordpre = c.take<uint32_t>(base, residual ? words : 0);
  p->wordbits = c.take<uint32_t>(base, residual ? words : 0);
  p->slot_flag = c.take<uint8_t>(base, nslots);
  p->tok_chain = c.take<int32_t>(base, TG);
  p->tok_nres = c.take<int32_t>(base, TG);
  p->chain_blk = c.take<int32_t>(base, nslots);
  p->tile_items = c.take<int32_t>(base, TG);
  p->row_cnt = c.take<int32_t>(base, d.NR);
  p->row_off = c.take<int32_t>(base, (size_t)d.NR + 1);
  p->unit_off = c.take<int32_t>(base, (size_t)d.NR + 1);
  p->ent = c.take<int32_t>(base, residual ? nslots : 0);
  p->slot_pos = c.take<int32_t>(base, residual ? nslots : 0);
  if (with_partials) {
    p->scratch_row = c.take<char>(base, 8192);
    p->res_list = c.take<int32_t>(base, nslots);
    p->res_rank = c.take<uint8_t>(base, nslots);
    p->win_desc = c.take<int4>(base, nslots);
    const size_t items = ((size_t)(d.Tq + d.T - 1) / d.T + d.B) * d.Hkv;  // tile items, listed or enumerated
    p->tdesc = c.take<int4>(base, 2 * items);
    p->ctab = c.take<int4>(base, items * 4 * d.K);
    p->opart = c.take<uint16_t>(base, (nslots * d.G + 31) / 32 * 32 * 128);  // whole 32-row blocks
    p->lpart = c.take<float>(base, nslots * d.G);
  } else {
    p->scratch_row = nullptr;
    p->res_list = nullptr;
    p->res_rank = nullptr;
    p->win_desc = nullptr;
    p->tdesc = nullptr;
    p->ctab = nullptr;
    p->opart = nullptr;
    p->lpart = nullptr;
  }
  return c.off + 256;
}

constexpr size_t kCntSetBytes = 256;  // one counter set, padded
static_assert(msa::kCntSlots * sizeof(int32_t) <= kCntSetBytes, "counter set");

constexpr int kMaxDevices = 64;

struct DeviceState {
  bool ready = false;           // num_cu and zero_page are known
  int num_cu = 0;
  const void* zero_page = nullptr;  // device address of g_zero_page on this device
  // the library-owned workspace
  void* ptr = nullptr;  // planning arrays and partial results
  size_t bytes = 0;
  void* zs = nullptr;   // zero-state: two counter sets, then the bitmap
  size_t zs_bytes = 0;
  int parity = 0;       // counter set of the next call
  bool dirty = false;   // zero-state must be cleared before use
  void* scratch = nullptr;  // device address of this device's `scratch` array (resolved on first use)
};

// Held by every entry point that touches a device's state, from the lease of
// its workspace through the last launch that uses it (launches are
// asynchronous, so this is short).
std::mutex g_ws_mutex;
DeviceState g_dev[kMaxDevices];

// State of the current device (g_ws_mutex held): compute-unit count and the
// zero page's address are queried once per device.
int32_t device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice failed: no usable HIP device");
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  DeviceState& w = g_dev[dev];
  if (!w.ready) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(MSA_ERR_HIP, "cannot query the compute-unit count of device %d", dev);
    void* zp = nullptr;
    if (hipGetSymbolAddress(&zp, HIP_SYMBOL(g_zero_page)) != hipSuccess || !zp) {
      (void)hipGetLastError();
      return fail(MSA_ERR_HIP, "cannot resolve the zero page on device %d", dev);
    }
    w.num_cu = n;
    w.zero_page = zp;
    w.ready = true;
  }
  *out = &w;
  return MSA_OK;
}

// cap on the library-owned workspace of every device (0: none), set by
// msa_set_workspace_limit (read and written with g_ws_mutex held)
size_t g_ws_limit = 0;

// The library-owned workspace of the device (g_ws_mutex held): scratch of
// `need` bytes and a zero-state buffer of two counter sets plus
// `bitmap_words` words. Growing either synchronises the device; a new
// zero-state buffer is zeroed.
int32_t grow_workspace(DeviceState& w, size_t need, size_t bitmap_words) {
  const size_t zs_need = 2 * kCntSetBytes + bitmap_words * 4;
  if (g_ws_limit && need + zs_need > g_ws_limit)
    return fail(MSA_ERR_OUT_OF_MEMORY, "this call needs %zu bytes of workspace, above the limit of %zu set with "
                "msa_set_workspace_limit", need + zs_need, g_ws_limit);
  if (w.bytes >= need && w.zs_bytes >= zs_need) return MSA_OK;
  if (w.ptr || w.zs) {
    if (hipDeviceSynchronize() != hipSuccess) return fail(MSA_ERR_HIP, "hipDeviceSynchronize failed while growing the workspace");
  }
  if (w.bytes < need) {
    if (w.ptr) (void)hipFree(w.ptr);
    w.ptr = nullptr;
    w.bytes = 0;
    const size_t alloc = std::max(need, (size_t)1 << 20);
    if (hipMalloc(&w.ptr, alloc) != hipSuccess) {
      (void)hipGetLastError();
      w.ptr = nullptr;
      return fail(MSA_ERR_OUT_OF_MEMORY, "workspace allocation of %zu bytes failed", alloc);
    }
    w.bytes = alloc;
  }
  if (w.zs_bytes < zs_need) {
    if (w.zs) (void)hipFree(w.zs);
    w.zs = nullptr;
    w.zs_bytes = 0;
    const size_t alloc = std::max(zs_need, (size_t)1 << 20);
    if (hipMalloc(&w.zs, alloc) != hipSuccess) {
      (void)hipGetLastError();
      w.zs = nullptr;
      return fail(MSA_ERR_OUT_OF_MEMORY, "zero-state allocation of %zu bytes failed", alloc);
    }
    w.dirty = hipMemset(w.zs, 0, alloc) != hipSuccess;
    w.zs_bytes = alloc;
    w.parity = 0;
  }
  return MSA_OK;
}

void fill_inputs(msa::Params* p, const Dims& d, const msa_tensor* sel, const msa_tensor* bt,
                 const msa_tensor* cu, const msa_tensor* used, int32_t causal) {
  p->selected = (const int32_t*)sel->data;
  p->block_tables = bt ? (const int32_t*)bt->data : nullptr;
  p->cu = (const int64_t*)cu->data;
  p->used = (const int32_t*)used->data;
  p->Tq = d.Tq;
  p->Hq = d.Hq;
  p->Hkv = d.Hkv;
  p->G = d.G;
  p->K = d.K;
  p->B = d.B;
  p->MP = d.MP;
  p->P = d.P;
  p->NP = d.NP;
  p->nb_max = d.nb_max;
  p->NR = d.NR;
  p->W = d.W;
  p->T = d.T;
  p->Tu = d.Tu;
  p->causal = causal;
  p->scale_log2 = (float)(1.0 / std::sqrt(128.0) * 1.4426950408889634);
}

// The attention launch plan. Tiles of one token each make every tile's chain
// its token's whole selection, so no slot is residual and the front kernel
// finishes every tile (at most 16 query rows per token); the index, unit and
// tile kernels are then not launched. Used for decode (one query token per
// sequence slot, Tq == B) and for small decode-shaped batches (Tq <= 4B)
// whose tokens all fit in one round of front workgroups, where launches cost
// more than the KV a sequence's tokens would otherwise share.
struct Plan {
  Dims d;
  bool narrow;      // decode-shaped: the front kernel streams residual-free tiles of <= 16 rows
  bool front_only;  // every tile is finished by the front kernel
};

Plan make_plan(const Dims& dims, int num_cu) {
  Plan pl;
  pl.d = dims;
  const bool decode_shaped = (int64_t)dims.Tq <= 4 * (int64_t)dims.B;
  const bool one_round = dims.Tq == dims.B || (int64_t)dims.Tq * dims.Hkv <= 2 * (int64_t)num_cu;
  // one-token tiles of up to 64 query rows (Hq/Hkv <= 64, e.g. MQA decode)
  // are streamed by the front kernel's row sets
  pl.front_only = decode_shaped && one_round && dims.G <= 64;
  pl.narrow = (dims.G <= 16 && decode_shaped) || pl.front_only;
  if (pl.front_only) pl.d.T = 1;
  return pl;
}

// bytes of a caller-owned workspace for plan pl: counter set, bitmap (calls
// with possible residual slots), planning arrays and partials
size_t ws_bytes_for(const Plan& pl) {
  msa::Params tmp{};
  const size_t head = kCntSetBytes + (pl.front_only ? 0 : (size_t)pl.d.NR * pl.d.W * 4);
  return ((head + 255) & ~size_t(255)) + layout(pl.d, nullptr, &tmp, !pl.front_only, !pl.front_only);
}

// Enqueues the kernels of one attention call. `counters` is zero on entry
// (or is cleared by the fill when clear_words > 0); counters_next, when not
// null, is cleared by the call's last kernel for the next call.
hipError_t enqueue_attention(msa::Params& p, const Plan& pl, int num_cu, uint32_t* clear, int64_t clear_words,
                             hipStream_t st) {
  const Dims& d = pl.d;
  // decode-shaped batches (few queries per sequence, at most 16 query rows
  // per token) finish their residual-free tiles in the front kernel, one
  // workgroup per token; otherwise the front kernel runs one workgroup per
  // tile and lists every tile for the tile kernel
  p.stream_narrow = pl.narrow ? 1 : 0;
  p.list_tiles = p.stream_narrow;  // otherwise the tile kernel enumerates every tile itself
  p.front_only = pl.front_only ? 1 : 0;
  hipError_t e = hipSuccess;
  if (clear_words > 0) e = msa::launch_fill(clear, clear_words, 0u, st);
  if (e == hipSuccess) e = msa::launch_front(p, d.q_elem, d.kv_elem, st);
  // decode-shaped batches rarely have residual slots: there the unit kernel
  // derives the residual order itself and the materialising pass (one more
  // launch) is skipped
  p.ent_ready = p.stream_narrow ? 0 : 1;
  if (!pl.front_only) {
    if (e == hipSuccess) e = msa::launch_index(p, p.ent_ready != 0, st);
    if (e == hipSuccess) e = msa::launch_units(p, d.q_elem, d.kv_elem, num_cu, st);
    if (e == hipSuccess) e = msa::launch_tiles(p, d.q_elem, d.kv_elem, num_cu, st);
  }
  return e;
}

void fill_attention_io(msa::Params* p, const msa_tensor* q, const msa_tensor* k, const msa_tensor* v,
                       msa_tensor* out, msa_tensor* lse) {
  p->q = q->data;
  p->k = k->data;
  p->v = v->data;
  p->out = out->data;
  p->lse = lse ? (float*)lse->data : nullptr;
}

// One attention call whose scratch is `base` (a caller-owned workspace or
// the no-allocation array, at least ws_bytes_for(pl) bytes): one counter set
// and the bitmap first, then the planning arrays and partials. Nothing is
// allocated and nothing waits; a front-only call uses neither the counters
// nor the bitmap (every tile is finished where it is classified), any other
// call clears both with a fill kernel first.
int32_t run_in_workspace(const Plan& pl, const DeviceState& w, char* base, const msa_tensor* q,
                         const msa_tensor* k_cache, const msa_tensor* v_cache, const msa_tensor* selected,
                         const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                         const msa_tensor* used_kv_lens, int32_t causal, msa_tensor* out, msa_tensor* lse,
                         hipStream_t st) {
  const size_t bitmap_words = pl.front_only ? 0 : (size_t)pl.d.NR * pl.d.W;
  const size_t head = (kCntSetBytes + bitmap_words * 4 + 255) & ~size_t(255);
  msa::Params p{};
  layout(pl.d, base + head, &p, !pl.front_only, !pl.front_only);
  p.slot_pos = nullptr;
  fill_inputs(&p, pl.d, selected, block_tables, cu_seqlens_q, used_kv_lens, causal);
  fill_attention_io(&p, q, k_cache, v_cache, out, lse);
  p.counters = (int32_t*)base;
  p.counters_next = nullptr;
  p.zero_page = w.zero_page;
  p.bitmap = (uint32_t*)(base + kCntSetBytes);
  const int64_t clear_words = pl.front_only ? 0 : (int64_t)((kCntSetBytes + bitmap_words * 4) / 4);
  const hipError_t e = enqueue_attention(p, pl, w.num_cu, (uint32_t*)base, clear_words, st);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

// ---------------------------------------------------------------------------
// kernel timing hooks
// ---------------------------------------------------------------------------
namespace msa {
volatile uint32_t g_profile_mask = 0;
}

namespace {
struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};
std::mutex g_prof_mutex;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

msa::ProfSpan msa::profile_begin(int kid) {
  ProfSpan sp{kid, nullptr, nullptr};
  if (!(g_profile_mask & (1u << kid))) return sp;
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  hipEvent_t a = pooled_event(), b = a ? pooled_event() : nullptr;
  if (!a || !b) {
    if (a) g_event_pool.push_back(a);
    return sp;
  }
  sp.a = a;
  sp.b = b;
  return sp;
}

void msa::profile_end(const ProfSpan& sp, bool launched) {
  if (!sp.a) return;
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  if (launched) {
    g_prof.push_back({sp.kid, sp.a, sp.b});
  } else {
    g_event_pool.push_back(sp.a);
    g_event_pool.push_back(sp.b);
  }
}

extern "C" {

int32_t msa_profile_enable(uint32_t kernel_mask) {
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  for (auto& r : g_prof) {
    (void)hipEventSynchronize(r.b);
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof.clear();
  msa::g_profile_mask = kernel_mask & ((1u << msa::kNumKernelIds) - 1u);
  return ok();
}

int32_t msa_profile_collect(int32_t kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches || kernel < 0 || kernel >= msa::kNumKernelIds) return fail(MSA_ERR_INVALID_ARGUMENT, "bad profile query");
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  double tot = 0.0;
  int64_t n = 0;
  std::vector<ProfRec> keep;
  for (auto& r : g_prof) {
    if (r.kernel != kernel) {
      keep.push_back(r);
      continue;
    }
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(MSA_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(MSA_ERR_HIP, "hipEventElapsedTime failed");
    tot += ms;
    ++n;
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof.swap(keep);
  *total_ms = tot;
  *launches = n;
  return ok();
}


const char* msa_last_error(void) { return g_err; }

int32_t msa_set_workspace_limit(size_t bytes) {
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  g_ws_limit = bytes;
  return ok();
}

const char* msa_version(void) { return "msa_kvouter 0.1.0 (gfx950)"; }

// One attention call on the library's workspace, the arguments validated
// (d). k / v are the caches' descriptors (for MXFP4 caches the codes), with
// the MXFP4 scales in k_scale / v_scale (else null).
static int32_t attention_library_ws(const Dims& d, const msa_tensor* q, const msa_tensor* k, const msa_tensor* v,
                             const uint8_t* k_scale, const uint8_t* v_scale, const msa_tensor* selected,
                             const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                             const msa_tensor* used_kv_lens, int32_t causal, msa_tensor* out, msa_tensor* lse,
                             void* stream) {
  int32_t rc;
  std::lock_guard<std::mutex> lk(g_ws_mutex);  // held through the last launch
  DeviceState* w = nullptr;
  if ((rc = device_state(&w))) return rc;
  const Plan pl = make_plan(d, w->num_cu);
  msa::Params p{};
  const size_t need = layout(pl.d, nullptr, &p, !pl.front_only, !pl.front_only);
  if ((rc = grow_workspace(*w, need, pl.front_only ? 0 : (size_t)pl.d.NR * pl.d.W))) return rc;
  layout(pl.d, (char*)w->ptr, &p, !pl.front_only, !pl.front_only);
  p.slot_pos = nullptr;  // the per-token residual lists replace it here
  fill_inputs(&p, pl.d, selected, block_tables, cu_seqlens_q, used_kv_lens, causal);
  fill_attention_io(&p, q, k, v, out, lse);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  int32_t* sets = (int32_t*)w->zs;
  p.counters = sets + w->parity * (kCntSetBytes / 4);
  p.counters_next = sets + (1 - w->parity) * (kCntSetBytes / 4);
  p.zero_page = w->zero_page;
  p.bitmap = (uint32_t*)((char*)w->zs + 2 * kCntSetBytes);
  const hipError_t e = enqueue_attention(p, pl, w->num_cu, (uint32_t*)w->zs,
                                         w->dirty ? (int64_t)(w->zs_bytes / 4) : 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    w->dirty = true;  // some kernels may not have run: clear everything next time
    return fail(MSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  w->dirty = false;
  w->parity = 1 - w->parity;
  return ok();
}

int32_t msa_kvouter_attention(const msa_tensor* q, const msa_tensor* k_cache, const msa_tensor* v_cache,
                              const msa_tensor* selected, const msa_tensor* block_tables,
                              const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens,
                              int32_t page_size, int32_t causal, msa_tensor* out, msa_tensor* lse,
                              void* stream) {
  Dims d;
  if (!out) return fail(MSA_ERR_INVALID_ARGUMENT, "out: null descriptor");
  int32_t rc = validate(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, page_size,
                        causal, out, lse, &d);
  if (rc) return rc;
  if (d.Tq == 0) return ok();
  return attention_library_ws(d, q, k_cache, v_cache, nullptr, nullptr, selected, block_tables, cu_seqlens_q,
                              used_kv_lens, causal, out, lse, stream);
}

int32_t msa_kvouter_attention_mxfp4(const msa_tensor* q, const msa_tensor* k_codes, const msa_tensor* k_scales,
                                    const msa_tensor* v_codes, const msa_tensor* v_scales,
                                    const msa_tensor* selected, const msa_tensor* block_tables,
                                    const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens,
                                    int32_t page_size, int32_t causal, msa_tensor* out, msa_tensor* lse,
                                    void* stream) {
  if (!out) return fail(MSA_ERR_INVALID_ARGUMENT, "out: null descriptor");
  int32_t rc;
  // the code and scale arrays: [num_pages, Hkv, page_size, 64] and [..., 4] bytes
  if ((rc = check_tensor(k_codes, "k_codes", 4, MSA_UINT8, 16))) return rc;
  if ((rc = check_tensor(v_codes, "v_codes", 4, MSA_UINT8, 16))) return rc;
  if ((rc = check_tensor(k_scales, "k_scales", 4, MSA_UINT8, 16))) return rc;
  if ((rc = check_tensor(v_scales, "v_scales", 4, MSA_UINT8, 16))) return rc;
  if (k_codes->shape[3] != 64)
    return fail(MSA_ERR_UNSUPPORTED, "k_codes: %lld bytes a row, only 64 (head dim 128) is supported",
                (long long)k_codes->shape[3]);
  for (int i = 0; i < 4; ++i)
    if (v_codes->shape[i] != k_codes->shape[i]) return fail(MSA_ERR_INVALID_ARGUMENT, "v_codes: shape differs from k_codes");
  for (int i = 0; i < 3; ++i)
    if (k_scales->shape[i] != k_codes->shape[i] || v_scales->shape[i] != k_codes->shape[i])
      return fail(MSA_ERR_INVALID_ARGUMENT, "k_scales / v_scales: pages, heads and rows must match the codes'");
  if (k_scales->shape[3] != 4 || v_scales->shape[3] != 4)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_scales / v_scales: 4 scales a row expected");
  // everything else: the common validation, given the caches' page geometry
  // as one-byte values, 128 a row, at the codes' addresses
  msa_tensor kg = *k_codes, vg = *v_codes;
  kg.dtype = vg.dtype = MSA_FP8_E4M3FN;
  kg.shape[3] = vg.shape[3] = 128;
  Dims d;
  if ((rc = validate(q, &kg, &vg, selected, block_tables, cu_seqlens_q, used_kv_lens, page_size, causal, out, lse,
                     &d)))
    return rc;
  if (q->dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "MXFP4 caches: q must be bf16");
  if (d.Tq == 0) return ok();
  d.kv_elem = msa::kElemFP4;
  return attention_library_ws(d, q, k_codes, v_codes, (const uint8_t*)k_scales->data, (const uint8_t*)v_scales->data,
                              selected, block_tables, cu_seqlens_q, used_kv_lens, causal, out, lse, stream);
}

int32_t msa_kvouter_workspace_bytes(const msa_tensor* q, const msa_tensor* k_cache, const msa_tensor* v_cache,
                                    const msa_tensor* selected, const msa_tensor* block_tables,
                                    const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens,
                                    int32_t page_size, int32_t causal, size_t* bytes) {
  if (!bytes) return fail(MSA_ERR_INVALID_ARGUMENT, "bytes: null pointer");
  *bytes = 0;
  Dims d;
  const int32_t rc = validate(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, page_size,
                              causal, nullptr, nullptr, &d, /*need_data=*/false);
  if (rc) return rc;
  if (d.Tq == 0) return ok();
  // the largest plan any device can choose for these shapes: a batch of
  // one token per sequence is front-only everywhere; other decode-shaped
  // batches are front-only only when they fit a device's front workgroups
  Plan pl = make_plan(d, 0);
  *bytes = ws_bytes_for(pl);
  return ok();
}

int32_t msa_kvouter_attention_ws(const msa_tensor* q, const msa_tensor* k_cache, const msa_tensor* v_cache,
                                 const msa_tensor* selected, const msa_tensor* block_tables,
                                 const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens,
                                 int32_t page_size, int32_t causal, msa_tensor* out, msa_tensor* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  if (!out) return fail(MSA_ERR_INVALID_ARGUMENT, "out: null descriptor");
  int32_t rc = validate(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, page_size,
                        causal, out, lse, &d);
  if (rc) return rc;
  if (d.Tq == 0) return ok();
  if (!workspace) return fail(MSA_ERR_INVALID_ARGUMENT, "workspace: null pointer");
  if ((uintptr_t)workspace % 256) return fail(MSA_ERR_INVALID_ARGUMENT, "workspace: not 256-byte aligned");
  DeviceState* w = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_ws_mutex);  // device facts only; the workspace is the caller's
    if ((rc = device_state(&w))) return rc;
  }
  const Plan pl = make_plan(d, w->num_cu);
  const size_t need = ws_bytes_for(pl);
  if (workspace_bytes < need)
    return fail(MSA_ERR_INVALID_ARGUMENT, "workspace: %zu bytes given, this call needs %zu", workspace_bytes, need);
  return run_in_workspace(pl, *w, (char*)workspace, q, k_cache, v_cache, selected, block_tables, cu_seqlens_q,
                          used_kv_lens, causal, out, lse, (hipStream_t)stream);
}

int32_t msa_kvouter_attention_noalloc(const msa_tensor* q, const msa_tensor* k_cache, const msa_tensor* v_cache,
                                      const msa_tensor* selected, const msa_tensor* block_tables,
                                      const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens,
                                      int32_t page_size, int32_t causal, msa_tensor* out, msa_tensor* lse,
                                      void* stream) {
  Dims d;
  if (!out) return fail(MSA_ERR_INVALID_ARGUMENT, "out: null descriptor");
  int32_t rc = validate(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, page_size,
                        causal, out, lse, &d);
  if (rc) return rc;
  if (d.Tq == 0) return ok();
  // held through the launches: calls from several host threads enqueue one
  // at a time (their kernels still share the array on the device)
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  DeviceState* w = nullptr;
  if ((rc = device_state(&w))) return rc;
  if (!w->scratch) {
    // this device's copy of the array, resolved once with the device current
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(MSA_ERR_HIP, "cannot resolve the no-allocation scratch array on this device");
    }
    w->scratch = ptr;
  }
  const Plan pl = make_plan(d, w->num_cu);
  const size_t need = ws_bytes_for(pl);
  if (need > kNoAllocScratchBytes)
    return fail(MSA_ERR_UNSUPPORTED,
                "this call needs %zu bytes of scratch; msa_kvouter_attention_noalloc holds %zu (use "
                "msa_kvouter_attention or msa_kvouter_attention_ws)",
                need, kNoAllocScratchBytes);
  return run_in_workspace(pl, *w, (char*)w->scratch, q, k_cache, v_cache, selected, block_tables, cu_seqlens_q,
                          used_kv_lens, causal, out, lse, (hipStream_t)stream);
}

int32_t msa_build_index(const msa_tensor* selected, const msa_tensor* cu_seqlens_q,
                        const msa_tensor* used_kv_lens, int32_t Hq, int32_t nb_max, int32_t causal,
                        int32_t tile_tokens, int32_t unit_tokens, int32_t list_all_tiles,
                        const msa_index_out* o, void* stream) {
  int32_t rc;
  if ((rc = check_tensor(selected, "selected", 3, MSA_INT32, 4))) return rc;
  if ((rc = check_tensor(cu_seqlens_q, "cu_seqlens_q", 1, MSA_INT64, 8))) return rc;
  if ((rc = check_tensor(used_kv_lens, "used_kv_lens", 1, MSA_INT32, 4))) return rc;
  if (!o) return fail(MSA_ERR_INVALID_ARGUMENT, "out: null descriptor");
  const int64_t Tq = selected->shape[0], Hkv = selected->shape[1], K = selected->shape[2];
  const int64_t B = used_kv_lens->shape[0];
  if (cu_seqlens_q->shape[0] != B + 1) return fail(MSA_ERR_INVALID_ARGUMENT, "cu_seqlens_q: expected B+1 entries");
  if (Hkv < 1 || Hq < 1 || Hq % Hkv) return fail(MSA_ERR_INVALID_ARGUMENT, "Hq must be a positive multiple of Hkv");
  if (K < 1 || K > 64) return fail(MSA_ERR_UNSUPPORTED, "topk must be in [1, 64]");
  if (tile_tokens < 0 || tile_tokens > 128) return fail(MSA_ERR_INVALID_ARGUMENT, "tile_tokens must be in [0, 128]");
  if (unit_tokens < 1 || unit_tokens > 128) return fail(MSA_ERR_INVALID_ARGUMENT, "unit_tokens must be in [1, 128]");
  if (nb_max < 1 || (int64_t)nb_max * Hkv >= (1ll << 30)) return fail(MSA_ERR_INVALID_ARGUMENT, "nb_max out of range");
  if (causal != 0 && causal != 1) return fail(MSA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (list_all_tiles != 0 && list_all_tiles != 1) return fail(MSA_ERR_INVALID_ARGUMENT, "list_all_tiles must be 0 or 1");
  if (Tq * Hkv * K >= (1ll << 31)) return fail(MSA_ERR_UNSUPPORTED, "problem too large for 32-bit indices");
  if (!o->slot_flag || !o->tok_chain || !o->tok_nres || !o->chain_blk || !o->row_off || !o->unit_off ||
      !o->ent || !o->slot_pos || !o->tile_items || !o->counters)
    return fail(MSA_ERR_INVALID_ARGUMENT, "msa_index_out: null buffer");
  if (Tq == 0) return ok();
  Dims d{};
  d.Tq = (int)Tq;
  d.Hq = Hq;
  d.Hkv = (int)Hkv;
  d.G = (int)(Hq / Hkv);
  d.K = (int)K;
  d.B = (int)B;
  d.nb_max = nb_max;
  d.NR = nb_max * (int)Hkv;
  d.W = (int)((Tq + 31) / 32);
  d.T = tile_tokens;
  d.Tu = unit_tokens;
  msa::Params p{};
  const size_t need = layout(d, nullptr, &p, true, false);
  std::lock_guard<std::mutex> lk(g_ws_mutex);  // held through the last launch
  DeviceState* w = nullptr;
  if ((rc = device_state(&w))) return rc;
  if ((rc = grow_workspace(*w, need, (size_t)d.NR * d.W))) return rc;
  layout(d, (char*)w->ptr, &p, true, false);
  fill_inputs(&p, d, selected, nullptr, cu_seqlens_q, used_kv_lens, causal);
  p.T = tile_tokens;
  p.Tu = unit_tokens;
  p.stream_narrow = list_all_tiles ? 0 : 1;
  p.list_tiles = 1;
  p.counters = o->counters;  // caller-visible counters; the bitmap stays internal
  p.counters_next = nullptr;
  p.zero_page = w->zero_page;
  p.bitmap = (uint32_t*)((char*)w->zs + 2 * kCntSetBytes);
  p.slot_flag = o->slot_flag;
  p.tok_chain = o->tok_chain;
  p.tok_nres = o->tok_nres;
  p.chain_blk = o->chain_blk;
  p.row_off = o->row_off;
  p.unit_off = o->unit_off;
  p.ent = o->ent;
  p.slot_pos = o->slot_pos;
  p.tile_items = o->tile_items;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (w->dirty) e = msa::launch_fill((uint32_t*)w->zs, (int64_t)(w->zs_bytes / 4), 0u, st);
  if (e == hipSuccess) e = msa::launch_fill((uint32_t*)o->counters, 8, 0u, st);
  if (e == hipSuccess) e = msa::launch_fill((uint32_t*)o->slot_pos, (int64_t)Tq * Hkv * K, 0xFFFFFFFFu, st);
  if (e == hipSuccess) e = msa::launch_front(p, -1, -1, st);
  if (e == hipSuccess) e = msa::launch_index(p, true, st);
  if (e != hipSuccess) {
    w->dirty = true;
    return fail(MSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  w->dirty = false;
  return ok();
}

int32_t msa_widen_fp8(const void* in, int64_t n, int32_t out_dtype, void* out, void* stream) {
  if (!in || !out) return fail(MSA_ERR_INVALID_ARGUMENT, "null buffer");
  if (n < 0 || n % 16) return fail(MSA_ERR_INVALID_ARGUMENT, "n must be a non-negative multiple of 16");
  if (((uintptr_t)in) % 16 || ((uintptr_t)out) % 16) return fail(MSA_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
  if (out_dtype != MSA_BF16 && out_dtype != MSA_FP16) return fail(MSA_ERR_INVALID_ARGUMENT, "out dtype must be bf16 or fp16");
  hipError_t e = msa::launch_widen_fp8(in, n, elem_of(out_dtype), out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t msa_store_kv(const msa_tensor* k_new, const msa_tensor* v_new, const msa_tensor* loc,
                     msa_tensor* k_cache, msa_tensor* v_cache, int32_t page_size, void* stream) {
  int32_t rc;
  if ((rc = check_tensor(k_new, "k_new", 3, -1, 16))) return rc;
  if (k_new->dtype != MSA_BF16 && k_new->dtype != MSA_FP16)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_new: dtype must be bf16 or fp16, got %s", dname(k_new->dtype));
  if (!v_new != !v_cache) return fail(MSA_ERR_INVALID_ARGUMENT, "v_new and v_cache: pass both or neither");
  const bool has_v = v_new != nullptr;
  if (has_v && (rc = check_tensor(v_new, "v_new", 3, k_new->dtype, 16))) return rc;
  if ((rc = check_tensor(loc, "loc", 1, MSA_INT64, 8))) return rc;
  if ((rc = check_tensor(k_cache, "k_cache", 4, -1, 16))) return rc;
  if (has_v && (rc = check_tensor(v_cache, "v_cache", 4, k_cache->dtype, 16))) return rc;
  if (k_cache->dtype != k_new->dtype && k_cache->dtype != MSA_FP8_E4M3FN)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_cache: dtype %s must equal k_new's (%s) or be fp8_e4m3fn",
                dname(k_cache->dtype), dname(k_new->dtype));
  if (page_size != 64 && page_size != 128)
    return fail(MSA_ERR_UNSUPPORTED, "page_size %d: only 64 and 128 are supported", page_size);
  for (int i = 0; has_v && i < 3; ++i)
    if (v_new->shape[i] != k_new->shape[i]) return fail(MSA_ERR_INVALID_ARGUMENT, "v_new: shape differs from k_new");
  for (int i = 0; has_v && i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i])
      return fail(MSA_ERR_INVALID_ARGUMENT, "v_cache: shape differs from k_cache");
  if (k_new->shape[2] != 128 || k_cache->shape[3] != 128)
    return fail(MSA_ERR_UNSUPPORTED, "head dim must be 128");
  if (k_cache->shape[2] != page_size)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_cache: page dimension %lld != page_size %d",
                (long long)k_cache->shape[2], page_size);
  if (k_cache->shape[1] != k_new->shape[1])
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_cache: %lld KV heads, k_new has %lld", (long long)k_cache->shape[1],
                (long long)k_new->shape[1]);
  if (loc->shape[0] != k_new->shape[0])
    return fail(MSA_ERR_INVALID_ARGUMENT, "loc: %lld slots for %lld new tokens", (long long)loc->shape[0],
                (long long)k_new->shape[0]);
  const int64_t N = k_new->shape[0], Hkv = k_new->shape[1], NP = k_cache->shape[0];
  if (N * Hkv * 32 >= (1ll << 31) || NP * Hkv * page_size >= (1ll << 40))
    return fail(MSA_ERR_UNSUPPORTED, "problem too large");
  if (N == 0) return ok();
  hipError_t e = msa::launch_store_kv(k_new->data, has_v ? v_new->data : nullptr, (const int64_t*)loc->data,
                                      k_cache->data, has_v ? v_cache->data : nullptr, (int)N, (int)Hkv, page_size,
                                      NP, elem_of(k_new->dtype),
                                      k_cache->dtype == MSA_FP8_E4M3FN, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t msa_select_blocks(const msa_tensor* q_idx, const msa_tensor* k_idx_cache, const msa_tensor* block_tables,
                          const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens, int32_t page_size,
                          int32_t causal, int32_t topk, int32_t force_local, msa_tensor* selected,
                          msa_tensor* scores, void* stream) {
  int32_t rc;
  if ((rc = check_tensor(q_idx, "q_idx", 3, -1, 16))) return rc;
  if (q_idx->dtype != MSA_BF16 && q_idx->dtype != MSA_FP16)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q_idx: dtype must be bf16 or fp16, got %s", dname(q_idx->dtype));
  if ((rc = check_tensor(k_idx_cache, "k_idx_cache", 4, -1, 16))) return rc;
  if (k_idx_cache->dtype != q_idx->dtype && k_idx_cache->dtype != MSA_FP8_E4M3FN)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_idx_cache: dtype %s must equal q_idx's (%s) or be fp8_e4m3fn",
                dname(k_idx_cache->dtype), dname(q_idx->dtype));
  if ((rc = check_tensor(block_tables, "block_tables", 2, MSA_INT32, 4))) return rc;
  if ((rc = check_tensor(cu_seqlens_q, "cu_seqlens_q", 1, MSA_INT64, 8))) return rc;
  if ((rc = check_tensor(used_kv_lens, "used_kv_lens", 1, MSA_INT32, 4))) return rc;
  if ((rc = check_tensor(selected, "selected", 3, MSA_INT32, 4))) return rc;
  if (scores && (rc = check_tensor(scores, "scores", 3, MSA_FP32, 4))) return rc;
  if (page_size != 64 && page_size != 128)
    return fail(MSA_ERR_UNSUPPORTED, "page_size %d: only 64 and 128 are supported", page_size);
  if ((causal != 0 && causal != 1) || (force_local != 0 && force_local != 1))
    return fail(MSA_ERR_INVALID_ARGUMENT, "causal and force_local must be 0 or 1");
  const int64_t Tq = q_idx->shape[0], Hkv = q_idx->shape[1], B = used_kv_lens->shape[0];
  const int64_t NP = k_idx_cache->shape[0], MP = block_tables->shape[1];
  if (q_idx->shape[2] != 128 || k_idx_cache->shape[3] != 128) return fail(MSA_ERR_UNSUPPORTED, "head dim must be 128");
  if (k_idx_cache->shape[1] != Hkv)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_idx_cache: %lld KV heads, q_idx has %lld",
                (long long)k_idx_cache->shape[1], (long long)Hkv);
  if (k_idx_cache->shape[2] != page_size)
    return fail(MSA_ERR_INVALID_ARGUMENT, "k_idx_cache: page dimension %lld != page_size %d",
                (long long)k_idx_cache->shape[2], page_size);
  if (block_tables->shape[0] != B || cu_seqlens_q->shape[0] != B + 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "block_tables, cu_seqlens_q and used_kv_lens disagree on the batch size");
  if (topk < 1 || topk > msa::kSelMaxBlocks)
    return fail(MSA_ERR_INVALID_ARGUMENT, "topk %d outside [1, %d]", topk, msa::kSelMaxBlocks);
  if (selected->shape[0] != Tq || selected->shape[1] != Hkv || selected->shape[2] != topk)
    return fail(MSA_ERR_INVALID_ARGUMENT, "selected: expected [%lld, %lld, %d]", (long long)Tq, (long long)Hkv, topk);
  const int64_t nb_cap = (MP * page_size + 127) / 128;
  if (nb_cap > msa::kSelMaxBlocks)
    return fail(MSA_ERR_UNSUPPORTED, "page tables reach %lld blocks; the selection scores at most %d per sequence",
                (long long)nb_cap, msa::kSelMaxBlocks);
  if (scores && (scores->shape[0] != Tq || scores->shape[1] != Hkv || scores->shape[2] != nb_cap))
    return fail(MSA_ERR_INVALID_ARGUMENT, "scores: expected [%lld, %lld, %lld]", (long long)Tq, (long long)Hkv,
                (long long)nb_cap);
  if (Tq >= (1ll << 31) / 16 || Hkv > 65535 || NP >= (1ll << 31) || B >= (1ll << 30) ||
      Tq * Hkv * (int64_t)topk >= (1ll << 40) ||
      (Tq / 16 + B + 1) * Hkv * ((nb_cap + msa::kSelSplitBlocks - 1) / msa::kSelSplitBlocks) >= (1ll << 31))
    return fail(MSA_ERR_UNSUPPORTED, "problem too large");
  if (Tq == 0 || Hkv == 0) return ok();
  if (B == 0) return fail(MSA_ERR_INVALID_ARGUMENT, "Tq > 0 with an empty batch");
  msa::SelectParams p{};
  p.q = q_idx->data;
  p.k = k_idx_cache->data;
  p.bt = (const int32_t*)block_tables->data;
  p.cu = (const int64_t*)cu_seqlens_q->data;
  p.used = (const int32_t*)used_kv_lens->data;
  p.selected = (int32_t*)selected->data;
  p.scores = scores ? (float*)scores->data : nullptr;
  p.Tq = (int)Tq;
  p.Hkv = (int)Hkv;
  p.B = (int)B;
  p.MP = (int)MP;
  p.P = page_size;
  p.num_pages = (int)NP;
  p.nb_cap = (int)nb_cap;
  p.topk = topk;
  p.causal = causal;
  p.force_local = force_local;
  // Prefill-shaped batches: 256-token tiles share each block's keys through
  // LDS. Decode-shaped batches (a few queries per long sequence): 16-token
  // tiles whose blocks are split over slices. Both write the score table --
  // the caller's `scores` or the library workspace -- and list it.
  const bool tiled = Tq > 4 * B;
  float* table = nullptr;
  std::unique_lock<std::mutex> lk(g_ws_mutex, std::defer_lock);
  if (scores) {
    table = (float*)scores->data;
  } else {
    lk.lock();  // held through the launches that use the library's workspace
    DeviceState* w = nullptr;
    if ((rc = device_state(&w))) return rc;
    if ((rc = grow_workspace(*w, (size_t)Tq * Hkv * nb_cap * sizeof(float), 0))) return rc;
    table = (float*)w->ptr;
  }
  hipError_t e = msa::launch_select(p, elem_of(q_idx->dtype), k_idx_cache->dtype == MSA_FP8_E4M3FN, table, tiled,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int32_t msa_validate_inputs(const msa_tensor* q, const msa_tensor* k_cache, const msa_tensor* v_cache,
                            const msa_tensor* selected, const msa_tensor* block_tables,
                            const msa_tensor* cu_seqlens_q, const msa_tensor* used_kv_lens, int32_t page_size,
                            int32_t causal, void* stream) {
  Dims d;
  int32_t rc = validate(q, k_cache, v_cache, selected, block_tables, cu_seqlens_q, used_kv_lens, page_size,
                        causal, nullptr, nullptr, &d);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return fail(MSA_ERR_HIP, "hipStreamSynchronize failed");
  std::vector<int64_t> cu(d.B + 1);
  std::vector<int32_t> used(d.B), bt((size_t)d.B * d.MP), sel((size_t)d.Tq * d.Hkv * d.K);
  auto cp = [](void* dst, const void* src, size_t bytes) {
    return bytes == 0 || hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost) == hipSuccess;
  };
  if (!cp(cu.data(), cu_seqlens_q->data, cu.size() * 8) || !cp(used.data(), used_kv_lens->data, used.size() * 4) ||
      !cp(bt.data(), block_tables->data, bt.size() * 4) || !cp(sel.data(), selected->data, sel.size() * 4))
    return fail(MSA_ERR_HIP, "device-to-host copy failed");
  if (cu[0] != 0) return fail(MSA_ERR_PRECONDITION, "cu_seqlens_q[0] = %lld, expected 0", (long long)cu[0]);
  for (int s = 0; s < d.B; ++s) {
    if (cu[s + 1] < cu[s]) return fail(MSA_ERR_PRECONDITION, "cu_seqlens_q decreases at %d", s);
    if (used[s] < 0 || (int64_t)used[s] > (int64_t)d.MP * d.P)
      return fail(MSA_ERR_PRECONDITION, "used_kv_lens[%d] = %d outside [0, max_pages*page_size]", s, used[s]);
    if (causal && used[s] < cu[s + 1] - cu[s])
      return fail(MSA_ERR_PRECONDITION, "sequence %d: used_kv_lens < query count under causal masking", s);
  }
  if (cu[d.B] != d.Tq) return fail(MSA_ERR_PRECONDITION, "cu_seqlens_q[B] = %lld, expected Tq = %d", (long long)cu[d.B], d.Tq);
  for (int s = 0; s < d.B; ++s) {
    const int L = used[s];
    const int nblk = (L + 127) / 128;
    for (int64_t t = cu[s]; t < cu[s + 1]; ++t)
      for (int g = 0; g < d.Hkv; ++g) {
        const int32_t* row = &sel[((size_t)t * d.Hkv + g) * d.K];
        for (int k = 0; k < d.K; ++k) {
          const int b = row[k];
          if (b < 0 || b >= nblk) continue;
          for (int k2 = 0; k2 < k; ++k2)
            if (row[k2] == b)
              return fail(MSA_ERR_PRECONDITION, "selected[%lld, %d]: block %d appears twice", (long long)t, g, b);
          const int lp0 = (128 * b) / d.P, lp1 = (std::min(128 * b + 128, L) + d.P - 1) / d.P;
          for (int lp = lp0; lp < lp1; ++lp) {
            const int page = bt[(size_t)s * d.MP + lp];
            if (page < 0 || page >= d.NP)
              return fail(MSA_ERR_PRECONDITION, "block_tables[%d, %d] = %d outside [0, %d)", s, lp, page, d.NP);
          }
        }
      }
  }
  return ok();
}

}  // extern "C"
