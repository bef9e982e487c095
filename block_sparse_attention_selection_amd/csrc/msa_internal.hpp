// msa_internal.hpp -- host/device shared parameter block and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// counters[] slots in the workspace
enum Counter {
  kCntResidual = 0,   // residual slots in the batch
  kCntNarrow = 1,     // chain items with at most 16 rows
  kCntWide = 2,       // chain items with more than 16 rows
  kCntUnits = 3,      // KV-outer units
  kCntWideNext = 4,   // dynamic work counter of the wide kernel
  kCntSlots = 8,
};

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
  float scale_log2;  // softmax scale * log2(e)
  // planning arrays
  int32_t* counters;
  uint8_t* slot_flag;
  int32_t* tok_chain;
  int32_t* tok_nres;
  int32_t* chain_blk;
  int32_t* narrow_items;
  int32_t* wide_items;
  uint32_t* bitmap;
  uint32_t* wordpre;
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

// planning kernels (msa_index.hip)
hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t value, hipStream_t st);
hipError_t launch_plan(const Params& p, hipStream_t st);
// attention kernels (msa_forward.hip)
hipError_t launch_forward(const Params& p, int q_elem, int kv_elem, int num_cu, hipStream_t st);
hipError_t launch_widen_fp8(const void* in, int64_t n, int out_elem, void* out, hipStream_t st);

}  // namespace msa
