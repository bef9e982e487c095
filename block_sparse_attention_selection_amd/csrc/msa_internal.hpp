// msa_internal.hpp -- host/device shared parameter block and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// counters[] slots in the workspace
enum Counter {
  kCntResidual = 0,   // residual slots in the batch
  kCntCombine = 1,    // (token, KV head) pairs whose output the combine writes
  kCntWide = 2,       // chain items with more than 16 rows
  kCntUnits = 3,      // KV-outer units
  kCntTask = 4,       // work queue head of the work kernel
  kCntDoneR = 5,      // finished row groups of the index kernel
  kCntSlots = 64,     // counters per set
};

// zero-state buffer: two counter sets used on alternate calls, a page of
// zeros that absent chunks are read from, and the residual token bitmaps.
// Every call leaves it as it found it: the bitmap words are cleared by the
// kernel that consumes them and the combine kernel clears the counter set of
// the next call.
constexpr size_t kZeroPageBytes = 16384;
constexpr size_t kZsHeaderBytes = 2 * kCntSlots * sizeof(int32_t) + kZeroPageBytes;

enum ElemCode { kElemBF16 = 0, kElemF16 = 1, kElemFP8 = 2 };

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
  int stream_narrow;  // front kernel streams tiles of <= 16 rows itself (decode mode)
  float scale_log2;   // softmax scale * log2(e)
  // planning arrays
  int32_t* counters;       // this call's counter set (zero on entry)
  int32_t* counters_next;  // the next call's set, cleared by the combine kernel (may be null)
  const void* zero_page;   // kZeroPageBytes of zeros
  uint8_t* slot_flag;
  int32_t* tok_chain;
  int32_t* tok_nres;
  int32_t* chain_blk;
  int32_t* combine_items;
  int32_t* wide_items;
  uint32_t* bitmap;    // residual bits, zero outside a call
  uint32_t* wordpre;   // per word: residual slots of the row before it
  uint32_t* wordbits;  // copy of the bitmap words taken before they are cleared
  int32_t* row_cnt;
  int32_t* row_off;
  int32_t* unit_off;
  int32_t* ent;
  int32_t* slot_pos;
  // partial results
  float* cpart;  // [Tq, Hq, 128] chain partial (normalised O)
  float* clse;   // [Tq, Hq] chain partial LSE (log2 units)
  float* opart;  // [residual slots, G, 128] KV-outer partial (normalised O)
  float* lpart;  // [residual slots, G] KV-outer partial LSE (log2 units)
};

// kernel timing hooks (msa_api.hip): no-ops unless msa_profile_enable set the bit
enum KernelId { kKIndex = 0, kKFront = 1, kKWork = 2, kKMerge = 3 };
extern volatile uint32_t g_profile_mask;
void profile_mark(int kernel, bool begin, hipStream_t st);

hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t value, hipStream_t st);
// residual inversion: row counts and row scan; `materialise` also writes
// ent / slot_pos (staged entry point only) (msa_index.hip)
hipError_t launch_index(const Params& p, bool materialise, hipStream_t st);
// front kernel: classification, plus the streaming of narrow chains when
// attention is requested (msa_forward.hip); q_elem < 0 classifies only
hipError_t launch_front(const Params& p, int q_elem, int kv_elem, hipStream_t st);
// wide chains and KV-outer units, then the merges (msa_forward.hip)
hipError_t launch_work(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st);
hipError_t launch_merge(const Params& p, int q_elem, int num_cu, hipStream_t st);
hipError_t launch_widen_fp8(const void* in, int64_t n, int out_elem, void* out, hipStream_t st);

}  // namespace msa
