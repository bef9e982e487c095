// msa_index.hip -- selection inversion and work split on gfx950.
//
// The pages name an index builder and a load-balancing scheduler as kernels
// of the KV-outer pass (fw-ai/minimax-kernels README, "Tests") and describe
// the aim: load each selected KV block once and serve every query that
// picked it (README, intro). Their rules are this library's own:
//
//   classify  (the front kernel in msa_forward.hip) one workgroup per (tile
//             leader, KV head): the tile's chain (blocks picked by every
//             token of the tile), per-slot covered/residual flags, residual
//             bits in the per-row token bitmaps, work lists
//   index     one workgroup per group of rows (block b, KV head g): popcount
//             prefix of each row's token bitmap (the words are copied and
//             cleared); the last workgroup scans the row counts
// A residual slot's place in the residual order is then a pure function of
// the row data (residual_pos), so no scatter pass is needed: KV-outer units
// enumerate their tokens from the bitmap copy and merges compute positions
// directly. The staged index entry point materialises the order (emit).
//
// Every output is a deterministic function of the inputs; the atomics only
// set bits (order-free) or append to item lists whose order is not part of
// the result.
#include "msa_device.hpp"
#include "msa_index_dev.hpp"
#include "msa_internal.hpp"

namespace msa {

__global__ void k_fill(uint32_t* __restrict__ p, int64_t n, uint32_t value) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = value;
}

hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

// rows: each workgroup counts a group of rows (its four waves one row each at
// a time, copying and clearing the rows' bitmap words) and publishes the row
// counts with atomic stores; the last
// workgroup to finish, found with an atomic counter, scans them. Only
// atomics carry data between workgroups of this kernel.
__global__ __launch_bounds__(256) void k_index(Params p, int rows_per_task, int ntasks) {
  __shared__ int smem[8];
  __shared__ int s_last;
  if (p.counters[kCntResidual] == 0) return;  // nothing to place (every decode batch)
  const int r0 = blockIdx.x * rows_per_task, r1 = min(r0 + rows_per_task, p.NR);
  // one row per wave at a time
  for (int r = r0 + (int)(threadIdx.x >> 6); r < r1; r += 4) {
    const int total = rowcount_row_wave(p, r);
    if ((threadIdx.x & 63) == 0) __hip_atomic_store(&p.row_cnt[r], total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(&p.counters[kCntDoneR], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (done == ntasks - 1);
  }
  __syncthreads();
  if (s_last) rowscan_all<256>(p, smem);
}

// materialise the residual order (ent, and slot_pos or the per-token lists)
__global__ __launch_bounds__(256) void k_emit(Params p) {
  if (p.counters[kCntResidual] == 0) return;
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (slot < (int64_t)p.Tq * p.Hkv * p.K) emit_slot(p, slot);
}

hipError_t launch_index(const Params& p, bool materialise, hipStream_t st) {
  const ProfSpan sp = profile_begin(kKIndex);
  const int rows_per_task = max(1, 2048 / max(p.W, 1));
  const int ntasks = (p.NR + rows_per_task - 1) / rows_per_task;
  hipError_t e = launch_k(sp, true, !materialise, k_index, dim3(ntasks), dim3(256), 0, st, p, rows_per_task, ntasks);
  if (e == hipSuccess && materialise) {
    const int64_t nslots = (int64_t)p.Tq * p.Hkv * p.K;
    e = launch_k(sp, false, true, k_emit, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st, p);
  }
  profile_end(sp, e == hipSuccess);
  return e;
}

}  // namespace msa
