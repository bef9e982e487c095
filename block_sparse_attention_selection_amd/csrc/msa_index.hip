// msa_index.hip -- selection inversion and work split on gfx950.
//
// The pages name an index builder and a load-balancing scheduler as kernels
// of the KV-outer pass (fw-ai/minimax-kernels README, "Tests") and describe
// the aim: load each selected KV block once and serve every query that
// picked it (README, intro). Their rules are this library's own:
//
//   classify  one wave per (tile leader, KV head): the tile's chain (blocks
//             picked by every token of the tile), per-slot covered/residual
//             flags, residual bits in the per-row token bitmaps, chain items
//   rowcount  one workgroup per row (block b, KV head g): popcount prefix of
//             the row's token bitmap
//   rowscan   one workgroup: exclusive scans of row counts and unit counts
//   emit      one thread per slot: position of each residual slot in its
//             row (bitmap rank), giving rows sorted by token without a sort
//
// Every output is a deterministic function of the inputs; the atomics only
// set bits (order-free) or append to item lists whose order is not part of
// the result.
#include "msa_device.hpp"
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

// exclusive scan across a workgroup of NT threads (NT a multiple of 64)
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int* total, int* smem) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) smem[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int v = (lane < NW) ? smem[lane] : 0;
    int vi = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(vi, off, 64);
      if (lane >= off) vi += y;
    }
    if (lane < NW) smem[lane] = vi - v;
    if (lane == NW - 1) smem[NW] = vi;
  }
  __syncthreads();
  const int res = smem[wid] + incl - x;
  *total = smem[NW];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// classify: one wave per candidate leader token t and KV head g
// dynamic LDS: picks of the tile, T_eff * K ints
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_classify(Params p) {
  extern __shared__ int s_sel[];  // [nt][K], -1 for invalid slots
  __shared__ int s_chain[64];
  __shared__ int s_nres[128];
  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int K = p.K, Hkv = p.Hkv;
  const size_t tg = (size_t)t * Hkv + g;

  const int s = seq_of(p.cu, p.B, t);
  if (s < 0) {  // outside every sequence: nothing valid
    for (int k = lane; k < K; k += 64) p.slot_flag[tg * K + k] = 0;
    if (lane == 0) {
      p.tok_chain[tg] = 0;
      p.tok_nres[tg] = 0;
    }
    return;
  }
  const int64_t q0 = p.cu[s], q1 = min(p.cu[s + 1], (int64_t)p.Tq);
  const int i0 = (int)(t - q0);
  const int Teff = p.T > 0 ? p.T : 1;
  if (i0 % Teff != 0) return;  // the tile's leader handles this token
  const int nt = (int)min((int64_t)Teff, q1 - t);
  const int L = p.used[s];
  const int Tq_s = (int)(p.cu[s + 1] - q0);
  const int nblk = L > 0 ? min((L + kBlk - 1) / kBlk, p.nb_max) : 0;

  for (int idx = lane; idx < nt * K; idx += 64) {
    const int tau = idx / K, k = idx - tau * K;
    const int b = p.selected[((size_t)(t + tau) * Hkv + g) * K + k];
    const int64_t pos = (int64_t)L - Tq_s + i0 + tau;
    const bool valid = b >= 0 && b < nblk && (!p.causal || (int64_t)kBlk * b <= pos);
    s_sel[idx] = valid ? b : -1;
  }
  for (int tau = lane; tau < nt; tau += 64) s_nres[tau] = 0;
  __syncthreads();

  // the chain: leader picks present in every token of the tile
  bool in_chain = false;
  int b_lead = -1;
  if (p.T > 0 && lane < K) {
    b_lead = s_sel[lane];
    in_chain = b_lead >= 0;
    for (int k2 = 0; k2 < lane && in_chain; ++k2) in_chain = s_sel[k2] != b_lead;
    for (int tau = 1; tau < nt && in_chain; ++tau) {
      bool found = false;
      for (int k2 = 0; k2 < K; ++k2) found |= (s_sel[tau * K + k2] == b_lead);
      in_chain = found;
    }
  }
  const uint64_t mask = __ballot(in_chain);
  const int n_ch = __popcll(mask);
  if (in_chain) {
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    s_chain[rank] = b_lead;
    p.chain_blk[tg * K + rank] = b_lead;
  }
  __syncthreads();

  // flags, residual bits, residual counts
  for (int idx = lane; idx < nt * K; idx += 64) {
    const int tau = idx / K;
    const int b = s_sel[idx];
    uint8_t flag = 0;
    if (b >= 0) {
      bool cov = false;
      for (int c = 0; c < n_ch; ++c) cov |= (s_chain[c] == b);
      flag = cov ? 1 : 2;
      if (!cov) {
        const int tt = t + tau;
        atomicOr(&p.bitmap[((size_t)b * Hkv + g) * p.W + (tt >> 5)], 1u << (tt & 31));
        atomicAdd(&s_nres[tau], 1);
      }
    }
    p.slot_flag[((size_t)(t + tau) * Hkv + g) * K + (idx - tau * K)] = flag;
  }
  __syncthreads();

  int tile_res = 0;
  for (int tau = lane; tau < nt; tau += 64) {
    const size_t tg2 = (size_t)(t + tau) * Hkv + g;
    p.tok_chain[tg2] = n_ch;
    p.tok_nres[tg2] = s_nres[tau];
    tile_res += s_nres[tau];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) tile_res += __shfl_xor(tile_res, off, 64);
  if (lane == 0) {
    if (tile_res > 0) atomicAdd(&p.counters[kCntResidual], tile_res);
    if (n_ch > 0) {
      const bool narrow = nt * p.G <= 16;
      const int slot = atomicAdd(&p.counters[narrow ? kCntNarrow : kCntWide], 1);
      (narrow ? p.narrow_items : p.wide_items)[slot] = (int)tg;
    }
  }
}

// ---------------------------------------------------------------------------
// rowcount: popcount prefix of each row's token bitmap
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rowcount(Params p) {
  __shared__ int smem[8];
  const int r = blockIdx.x;
  if (p.counters[kCntResidual] == 0) {
    if (threadIdx.x == 0) p.row_cnt[r] = 0;
    return;
  }
  const uint32_t* bm = p.bitmap + (size_t)r * p.W;
  uint32_t* pre = p.wordpre + (size_t)r * p.W;
  const int per = (p.W + 255) / 256;
  const int w0 = min((int)threadIdx.x * per, p.W);
  const int w1 = min(w0 + per, p.W);
  int sum = 0;
  for (int w = w0; w < w1; ++w) sum += __popc(bm[w]);
  int total;
  int run = block_excl_scan<256>(sum, &total, smem);
  for (int w = w0; w < w1; ++w) {
    pre[w] = (uint32_t)run;
    run += __popc(bm[w]);
  }
  if (threadIdx.x == 0) p.row_cnt[r] = total;
}

// ---------------------------------------------------------------------------
// rowscan: row offsets and unit offsets (single workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_rowscan(Params p) {
  __shared__ int smem[20];
  const int NR = p.NR;
  const int per = (NR + 1023) / 1024;
  const int r0 = min((int)threadIdx.x * per, NR);
  const int r1 = min(r0 + per, NR);
  int cnt = 0, units = 0;
  for (int r = r0; r < r1; ++r) {
    const int c = p.row_cnt[r];
    cnt += c;
    units += (c + p.Tu - 1) / p.Tu;
  }
  int tot_cnt, tot_units;
  int run_c = block_excl_scan<1024>(cnt, &tot_cnt, smem);
  int run_u = block_excl_scan<1024>(units, &tot_units, smem);
  for (int r = r0; r < r1; ++r) {
    const int c = p.row_cnt[r];
    p.row_off[r] = run_c;
    p.unit_off[r] = run_u;
    run_c += c;
    run_u += (c + p.Tu - 1) / p.Tu;
  }
  if (threadIdx.x == 0) {
    p.row_off[NR] = tot_cnt;
    p.unit_off[NR] = tot_units;
    p.counters[kCntUnits] = tot_units;
  }
}

// ---------------------------------------------------------------------------
// emit: place every residual slot at its rank within its row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_emit(Params p) {
  const int64_t nslots = (int64_t)p.Tq * p.Hkv * p.K;
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (slot >= nslots) return;
  if (p.slot_flag[slot] != 2) {
    p.slot_pos[slot] = -1;
    return;
  }
  const int t = (int)(slot / ((int64_t)p.Hkv * p.K));
  const int g = (int)((slot / p.K) % p.Hkv);
  const int b = p.selected[slot];
  const size_t r = (size_t)b * p.Hkv + g;
  const size_t w = r * p.W + (t >> 5);
  const uint32_t below = p.bitmap[w] & ((1u << (t & 31)) - 1u);
  const int pos = p.row_off[r] + (int)p.wordpre[w] + __popc(below);
  p.ent[pos] = (int)slot;
  p.slot_pos[slot] = pos;
}

hipError_t launch_plan(const Params& p, hipStream_t st) {
  const int Teff = p.T > 0 ? p.T : 1;
  const size_t lds = (size_t)Teff * p.K * sizeof(int);
  hipLaunchKernelGGL(k_classify, dim3(p.Tq, p.Hkv), dim3(64), lds, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowcount, dim3(p.NR), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowscan, dim3(1), dim3(1024), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nslots = (int64_t)p.Tq * p.Hkv * p.K;
  hipLaunchKernelGGL(k_emit, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace msa
