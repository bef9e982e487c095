// msa_internal.hpp -- host/device shared parameter block and launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// counters[] slots in the workspace
enum Counter {
  kCntResidual = 0,   // residual slots in the batch (the front kernel sets it to 1 if
                      // there are any; the index kernel replaces that with the total)
  kCntTiles = 1,      // tile items (tiles the front kernel does not finish itself)
  kCntUnits = 2,      // KV-outer units
  kCntDoneR = 5,      // finished row groups of the index kernel
  kCntXcd = 8,        // 8 per-XCD work queue heads of the tile kernel (8..15)
  kCntXcdU = 16,      // 8 per-XCD work queue heads of the unit kernel (16..23)
  kCntSlots = 64,     // counters per set
};

// A page of zeros that absent chunks are read from (a static device array,
// never written). The counter sets and the residual token bitmaps are zero
// when a call starts: the library-owned zero-state buffer is left that way
// by every call (the bitmap words are cleared by the kernel that consumes
// them, and the call's last kernel clears the counter set of the next call);
// a caller-owned workspace is cleared by a fill kernel instead.
constexpr size_t kZeroPageBytes = 16384;

enum ElemCode { kElemBF16 = 0, kElemF16 = 1, kElemFP8 = 2, kElemFP4 = 3 };

// tokens of one KV-outer work item (the unit kernel's LDS token list)
constexpr int kUnitWindowTokens = 512;

struct Params {
  // inputs
  const void* q;
  const void* k;
  const void* v;
  const int32_t* selected;
  const int32_t* block_tables;
  const int64_t* cu;
  const int32_t* used;
  // outputs
  void* out;
  float* lse;  // may be null
  // sizes
  int Tq, Hq, Hkv, G, K, B, MP, P, NP;
  int nb_max;   // ceil(MP*P/128)
  int NR;       // nb_max * Hkv rows of the residual inversion
  int W;        // 32-bit words per row bitmap: ceil(Tq/32)
  int T;        // tile tokens of chains (0: chains off)
  int Tu;       // tokens per KV-outer unit
  int causal;
  int stream_narrow;  // front kernel finishes residual-free tiles of <= 16 rows (decode mode)
  int list_tiles;     // front kernel appends the tiles it does not finish to tile_items
  int ent_ready;      // the index step materialised ent and res_list (else the unit kernel derives them)
  int front_only;     // one-token tiles, all finished by the front kernel: no later kernel runs, and
                      // the front kernel clears counters_next (otherwise the tile kernel does)
  float scale_log2;   // softmax scale * log2(e)
  // planning arrays
  int32_t* counters;       // this call's counter set (zero on entry)
  int32_t* counters_next;  // the next call's set, cleared by the tile kernel (may be null)
  const void* zero_page;   // kZeroPageBytes of zeros
  uint8_t* slot_flag;
  int32_t* tok_chain;
  int32_t* tok_nres;
  int32_t* chain_blk;
  int32_t* tile_items;  // t_leader * Hkv + g of each listed tile
  uint32_t* bitmap;    // residual bits, zero outside a call
  uint32_t* wordpre;   // per word: residual slots of the row before it
  uint32_t* wordbits;  // copy of the bitmap words taken before they are cleared
  int32_t* row_cnt;
  int32_t* row_off;
  int32_t* unit_off;
  int32_t* ent;
  int32_t* slot_pos;   // staged index entry: residual order of each slot
  int32_t* res_list;   // attention: per (t, g), the residual order of its residual slots, in slot order
  uint8_t* res_rank;   // attention: rank of a residual slot among the residual slots of its (t, g)
  int4* win_desc;      // attention: per unit-kernel window (row, first rank, first entry, entries)
  int4* tdesc;         // attention: per tile item, 2 x int4 (see write_tile_desc)
  int4* ctab;          // attention: per tile item, 4 topk chunk entries
  void* scratch_row;  // 8 KB that stores of rows outside a tile may land in
  // partial results of the KV-outer units
  void* opart;   // normalised O per (residual slot, head) row, in q's 16-bit type, in blocks of
                 // 32 rows: row r's 16-byte chunk k at byte (r >> 5) * 8192 + k * 512 + (r & 31) * 16
  float* lpart;  // [residual slots, G] LSE (log2 units)
  // MXFP4 caches: e8m0 scales [num_pages, Hkv, P, 4] (else null)
  const uint8_t* k_scale;
  const uint8_t* v_scale;
};

// Kernel timing (msa_api.hip), off unless msa_profile_enable set the bit of
// a kernel id. A span covers the kernels of one launcher call: while its id
// is profiled it holds a pair of pooled HIP events that the dispatches
// themselves record (hipExtLaunchKernel), the first kernel's start and the
// last kernel's end, so it measures the kernels' execution and nothing the
// host or the stream does around them.
enum KernelId { kKIndex = 0, kKFront = 1, kKUnits = 2, kKTiles = 3, kKStore = 4, kKSelect = 5 };
constexpr int kNumKernelIds = 6;
extern volatile uint32_t g_profile_mask;
struct ProfSpan {
  int kid;
  hipEvent_t a, b;  // null when the kernel id is not profiled
};
ProfSpan profile_begin(int kid);
void profile_end(const ProfSpan& sp, bool launched);

// launch of one kernel of a span (first: its dispatch records the span's
// start event; last: its end event)
template <typename F, typename... Args>
inline hipError_t launch_k(const ProfSpan& sp, bool first, bool last, F kernel, dim3 grid, dim3 block,
                           uint32_t shm, hipStream_t st, Args... args) {
  if (sp.a)
    hipExtLaunchKernelGGL(kernel, grid, block, shm, st, first ? sp.a : nullptr, last ? sp.b : nullptr, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, st, args...);
  return hipGetLastError();
}

hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t value, hipStream_t st);
// residual inversion: row counts and row scan; `materialise` also writes the
// residual order (ent, and slot_pos or the per-token residual lists) (msa_index.hip)
hipError_t launch_index(const Params& p, bool materialise, hipStream_t st);
// front kernel: classification, plus the residual-free narrow tiles when
// attention is requested (msa_forward.hip); q_elem < 0 classifies only
hipError_t launch_front(const Params& p, int q_elem, int kv_elem, hipStream_t st);
// KV-outer units, then the listed tiles with their merges (msa_tiles.hip)
hipError_t launch_units(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st);
hipError_t launch_tiles(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st);
hipError_t launch_widen_fp8(const void* in, int64_t n, int out_elem, void* out, hipStream_t st);
hipError_t launch_store_kv(const void* kn, const void* vn, const int64_t* loc, void* kc, void* vc, int N, int Hkv,
                           int P, int64_t num_pages, int in_elem, bool fp8_cache, hipStream_t st);

// block selection (msa_select.hip)
constexpr int kSelMaxBlocks = 2048;  // blocks per sequence the selection can score (262144 tokens)
struct SelectParams {
  const void* q;          // [Tq, Hkv, 128] index queries, 16-bit
  const void* k;          // [num_pages, Hkv, P, 128] index keys, q's type or e4m3fn
  const int32_t* bt;      // [B, MP]
  const int64_t* cu;      // [B + 1]
  const int32_t* used;    // [B]
  int32_t* selected;      // [Tq, Hkv, topk]
  float* scores;          // [Tq, Hkv, nb_cap] or null
  int Tq, Hkv, B, MP, P, num_pages, nb_cap, topk, causal, force_local;
};
constexpr int kSelSplitBlocks = 16;  // blocks per workgroup of the split (decode-shaped) path
constexpr int kSelSplitWaves = 4;
// scores into the table [Tq, Hkv, nb_cap] fp32 (`table`), by 256-token tiles
// (tiled: prefill-shaped batches) or by 16-token tiles split over block
// slices (decode-shaped batches), then the lists from the table
hipError_t launch_select(const SelectParams& p, int q_elem, bool fp8_keys, float* table, bool tiled, hipStream_t st);

}  // namespace msa
