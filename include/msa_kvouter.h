/*
 * msa_kvouter.h -- C ABI of the MI355X (gfx950) MiniMax-M3 block-sparse
 * attention forward pass.
 *
 * The operation (fw-ai/minimax-kernels README, intro and "Quick start"):
 * every query token and query head attends only to the keys of the 128-token
 * blocks that the token selected for the head's KV head. Keys and values are
 * read through a logical-to-physical page table from a paged cache; the pass
 * returns O [Tq, Hq, 128] and, on request, the fp32 log-sum-exp [Hq, Tq].
 * The KV-outer organisation of that README's intro (load a selected block
 * once, serve every query that picked it) is how the work is scheduled; the
 * result is the plain definition:
 *
 *   for token t of sequence s (cu_seqlens_q[s] <= t < cu_seqlens_q[s+1]),
 *   L = used_kv_lens[s], Tq_s = cu_seqlens_q[s+1] - cu_seqlens_q[s],
 *   pos = L - Tq_s + (t - cu_seqlens_q[s])      (bottom-right causal alignment)
 *   J = union over k of the positions j with 128*b <= j < min(128*b+128, L),
 *       b = selected[t, g, k], 0 <= b < ceil(L/128), and j <= pos if causal
 *   for head h with g = h / (Hq/Hkv):
 *       x_j = <q[t,h,:], K_j> / sqrt(128)
 *       lse[h,t] = ln sum_j exp(x_j),   out[t,h,:] = sum_j exp(x_j - lse) V_j
 *   K_j = k_cache[block_tables[s, j / page_size], g, j % page_size, :]
 *   An empty J gives out = 0 and lse = -inf.
 *
 * Conventions for every entry point
 *   - Buffers are dense, row-major, contiguous DEVICE memory owned by the
 *     caller; the library keeps no pointer after it returns. Buffers must stay
 *     valid until the stream reaches the enqueued work (usual HIP rules).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without waiting for it, except where stated.
 *   - Return 0 (MSA_OK) or a negative MSA_ERR_* code; msa_last_error() then
 *     holds a message (thread-local). Nothing throws or aborts across the
 *     ABI, and an invalid call enqueues nothing. There is no fallback path:
 *     an unsupported request is an error, never silently served another way
 *     (the README's "Backends" section states the same rule for its backends).
 */
#ifndef MSA_KVOUTER_H
#define MSA_KVOUTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 1

typedef enum msa_dtype {
  MSA_BF16 = 0,
  MSA_FP16 = 1,
  MSA_FP8_E4M3FN = 2, /* OCP e4m3fn: bias 7, max 448, NaN = 0x7F/0xFF, no inf */
  MSA_FP32 = 3,
  MSA_INT32 = 4,
  MSA_INT64 = 5,
  MSA_UINT8 = 6,
} msa_dtype;

enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = -1, /* null pointer, wrong rank/shape/dtype, misalignment */
  MSA_ERR_UNSUPPORTED = -2,      /* head_dim != 128, fp8 q, page_size not 64/128, ... */
  MSA_ERR_OUT_OF_MEMORY = -3,    /* workspace allocation failed */
  MSA_ERR_HIP = -4,              /* a HIP runtime call failed (no device, launch error) */
  MSA_ERR_PRECONDITION = -5,     /* msa_validate_inputs found a data violation */
};

/* Descriptor of a dense row-major device buffer. Unused shape entries are
 * ignored. `data` must be 16-byte aligned for q, caches, out. */
typedef struct msa_tensor {
  void* data;
  int32_t dtype; /* msa_dtype */
  int32_t ndim;
  int64_t shape[4];
} msa_tensor;

/*
 * msa_kvouter_attention -- the block-sparse attention forward pass.
 *
 *   q            [Tq, Hq, 128]                 bf16 or fp16
 *   k_cache      [num_pages, Hkv, page_size, 128]  q's dtype, or fp8 e4m3fn
 *   v_cache      same shape and dtype as k_cache
 *   selected     [Tq, Hkv, topk] int32, logical 128-token block ids; ids
 *                outside [0, ceil(L/128)) are ignored (use -1 as padding)
 *   block_tables [B, max_pages] int32, physical page of each logical page
 *   cu_seqlens_q [B + 1] int64, query offsets of the B sequences
 *   used_kv_lens [B] int32, keys of each sequence
 *   page_size    64 or 128
 *   causal       0 or 1 (bottom-right aligned)
 *   out          [Tq, Hq, 128] in q's dtype (written for every token)
 *   lse          [Hq, Tq] fp32, natural log, softmax scale included; NULL
 *                when not wanted
 *   stream       hipStream_t
 *
 * Sizes: Hq % Hkv == 0, Hq/Hkv <= 128, 1 <= topk <= 64. The softmax scale is
 * 1/sqrt(128). fp8 caches hold unscaled e4m3fn values (the cast rule of the
 * sglang pull request "Speed up MiniMax-M3 sparse attention on Hopper",
 * section "Verification"); they are widened exactly before use.
 *
 * Data-dependent preconditions that are not checked here (checking them
 * needs a device-to-host copy; msa_validate_inputs reports them): ids in one
 * (t, g) list are distinct, cu_seqlens_q is non-decreasing with
 * cu_seqlens_q[0] == 0 and cu_seqlens_q[B] == Tq, used_kv_lens[s] <=
 * max_pages*page_size, and every page id reached by a selected key lies in
 * [0, num_pages). A violation gives unspecified output values (tokens outside
 * every sequence may be left unwritten) but the kernels stay within the
 * buffers given: a page id outside the pool is treated as holding no keys,
 * and every wait inside the kernels is bounded. Tq == 0 returns MSA_OK and
 * enqueues nothing.
 *
 * Scratch memory: the library keeps one growable workspace per device
 * (allocated with hipMalloc on first use or when a larger problem arrives;
 * growing synchronises the device, so the first call at a new size is neither
 * asynchronous nor capturable into a graph). Calls into one device are
 * serialised on the host while they enqueue (the library holds a lock from
 * the workspace lease through the last launch), so several host threads may
 * call it; but the workspace is one buffer, so calls on different streams of
 * one device must not overlap in time on the device. Callers that need
 * either, or that capture the call into a graph, pass their own workspace to
 * msa_kvouter_attention_ws instead.
 *
 * Stages. The pass runs as up to five kernels on `stream`: classification of
 * every query tile (chains of shared picks, residual picks), the residual
 * inversion (per-(block, KV head) token lists, the index builder), the
 * KV-outer units (partial O and LSE per residual pick, split into windows of
 * bounded rows: the load-balancing split), and the tile kernel, which runs the
 * chains and merges each row's residual partials by LSE before writing out
 * and lse. The combine of the pages' design is fused into that last kernel's
 * epilogue, so no partial of a chain ever leaves registers; that is why there
 * are no separate split, forward-partials or combine entry points. The index
 * builder is exposed for bit-exact tests (msa_build_index).
 */
int32_t msa_kvouter_attention(const msa_tensor* q, const msa_tensor* k_cache,
                              const msa_tensor* v_cache, const msa_tensor* selected,
                              const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                              const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                              msa_tensor* out, msa_tensor* lse, void* stream);

/*
 * msa_kvouter_attention_mxfp4 -- the forward pass over MXFP4 K/V caches.
 *
 * The MSA summary page ("Highlighted Details") lists FP4 and NVFP4 among the
 * kernels' formats without defining a scale format. Read here as the OCP
 * microscaling format MXFP4: every 32 consecutive values of a K or V row
 * (dims 32 j .. 32 j + 31) share one e8m0 scale byte s, the value 2^(s - 127)
 * (s = 255, the format's NaN, is not supported, nor are s > 252, whose
 * largest values overflow the bf16 the kernels widen to); each value is an e2m1 code
 * (sign, two exponent bits with bias 1, one mantissa bit: magnitudes 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6), two codes a byte, value 2 i in the low nibble of byte
 * i. A cached value is code x scale, exactly.
 *
 *   k_codes      [num_pages, Hkv, page_size, 64]  uint8, 16-byte aligned
 *   k_scales     [num_pages, Hkv, page_size, 4]   uint8 (e8m0), 16-byte aligned
 *   v_codes, v_scales  the same shapes
 *   q            [Tq, Hq, 128] bf16
 *   other arguments as msa_kvouter_attention
 *
 * Every shape msa_kvouter_attention accepts, with bf16 queries (fp16
 * queries return MSA_ERR_UNSUPPORTED). The codes are widened to bf16, scale
 * applied, right before the products: in registers by the decode kernel, on
 * their way into LDS by the KV-outer and tile kernels. Errors, preconditions,
 * scratch and threading as msa_kvouter_attention (the library's workspace;
 * there is no caller-workspace variant).
 */
int32_t msa_kvouter_attention_mxfp4(const msa_tensor* q, const msa_tensor* k_codes,
                                    const msa_tensor* k_scales, const msa_tensor* v_codes,
                                    const msa_tensor* v_scales, const msa_tensor* selected,
                                    const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                                    const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                                    msa_tensor* out, msa_tensor* lse, void* stream);

/*
 * msa_kvouter_workspace_bytes -- bytes of the caller-owned workspace that
 * msa_kvouter_attention_ws needs for these shapes (the same descriptors as
 * msa_kvouter_attention without out / lse; only shapes and dtypes are read,
 * data pointers may be NULL). Writes 0 for Tq == 0. The size depends on
 * shapes only, and it is the largest any device needs for them:
 *
 *   - a batch with one query token per sequence (Tq == B) and Hq/Hkv <= 64
 *     (decode): planning arrays only, Tq*Hkv*(5*topk + 12) +
 *     12*Hkv*ceil(max_pages*page_size/128) bytes plus 256-byte alignment
 *     per array (about 72 KB for 64 sequences, Hkv = 8, top-16);
 *   - any other call: in addition the residual token bitmaps
 *     (ceil(max_pages*page_size/128) * Hkv * ceil(Tq/32) words), the
 *     residual order and tile tables, and the KV-outer partial results sized
 *     for every slot being residual: Tq*Hkv*topk*(Hq/Hkv) rows of 256 bytes
 *     (O in q's type) plus 4 bytes (LSE). This worst case is reached when no
 *     two consecutive tokens share a pick; which slots are residual is only
 *     known on the device. A 16384-token prefill with Hq = 64, Hkv = 8 and
 *     top-16 needs about 4.45 GB.
 *
 * Errors as for msa_kvouter_attention (descriptor errors only).
 */
int32_t msa_kvouter_workspace_bytes(const msa_tensor* q, const msa_tensor* k_cache,
                                    const msa_tensor* v_cache, const msa_tensor* selected,
                                    const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                                    const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                                    size_t* bytes);

/*
 * msa_kvouter_attention_ws -- msa_kvouter_attention with a caller-owned
 * workspace: `workspace` is device memory of `workspace_bytes` bytes (at
 * least msa_kvouter_workspace_bytes for these shapes, 256-byte aligned) that
 * the call uses as scratch until the stream reaches the end of its work; its
 * contents need not be initialised and are unspecified afterwards. The call
 * allocates nothing, synchronises nothing and issues no memset: it validates
 * on the host, then enqueues its kernels on `stream` (the first of them
 * clears the counters and bitmaps it needs, except for decode batches, which
 * use neither), so it can be captured into a HIP graph. Calls with distinct
 * workspaces may run concurrently on different streams; calls that share a
 * workspace must not overlap in time. Arguments, results and errors are
 * otherwise those of msa_kvouter_attention; a workspace that is too small or
 * misaligned is MSA_ERR_INVALID_ARGUMENT.
 */
int32_t msa_kvouter_attention_ws(const msa_tensor* q, const msa_tensor* k_cache,
                                 const msa_tensor* v_cache, const msa_tensor* selected,
                                 const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                                 const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                                 msa_tensor* out, msa_tensor* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * msa_kvouter_attention_noalloc -- msa_kvouter_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, results and
 * errors; the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine): its scratch is a fixed array of 32 MiB in the library's
 * device code, one per device, which each device holds until the process
 * ends. A call that needs more scratch than that (msa_kvouter_workspace_bytes
 * reports the need; decode batches need kilobytes, a prefill's KV-outer
 * partials take about Tq*Hkv*topk*(Hq/Hkv)*260 bytes) is refused with
 * MSA_ERR_UNSUPPORTED and enqueues nothing. Every call on a device uses that
 * device's one array, and each call clears what must start at zero itself:
 * calls that overlap in time on one device (different streams, or graphs
 * replayed concurrently) race on it and must be ordered by the caller.
 */
int32_t msa_kvouter_attention_noalloc(const msa_tensor* q, const msa_tensor* k_cache,
                                      const msa_tensor* v_cache, const msa_tensor* selected,
                                      const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                                      const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                                      msa_tensor* out, msa_tensor* lse, void* stream);

/*
 * msa_build_index -- the selection inversion and work split, exposed so that
 * their integer outputs can be compared bit for bit with a CPU reference.
 * (The pages name an index builder and a load-balancing scheduler among the
 * kernels of this pass: fw-ai/minimax-kernels README, "Tests".)
 *
 * Rules. Slot (t, g, k) holds b = selected[t, g, k]; it is valid when t lies
 * in a sequence s, 0 <= b < min(ceil(L/128), nb_max), and 128*b <= pos(t)
 * if causal. Each sequence's tokens are cut into tiles of `tile_tokens`
 * consecutive tokens (the first is the tile's leader). A tile's chain, per
 * KV head g, is the list of blocks that every token of the tile selected
 * validly, ordered as in the leader's list; tile_tokens == 0 disables chains.
 * Valid slots whose block is in the chain are "covered" (flag 1), other
 * valid slots are "residual" (flag 2), invalid slots have flag 0. Residual
 * slots are inverted into rows r = b*Hkv + g: row_off is the exclusive scan
 * of the row counts, ent lists each row's slot ids in ascending order, and
 * slot_pos[slot] is the slot's index in ent (-1 if not residual). unit_off is
 * the exclusive scan of ceil(row count / unit_tokens). A tile is listed in
 * tile_items as t_leader*Hkv + g, per KV head g, unless list_all_tiles is 0,
 * the tile has at most 16 query rows (tokens in the tile * Hq/Hkv) and none
 * of its slots is residual: such tiles are finished by the classifier itself
 * in the attention pass (the two settings are the classifier's two launch
 * shapes: one workgroup per token, or one per tile). With tile_tokens == 0
 * tiles are single tokens. The list is in unspecified order.
 *
 * All output buffers are caller-owned device memory of the sizes given;
 * chain_blk holds valid entries only at leader tokens (first tok_chain
 * entries). counters[0..2] = residual slots, tile items, units.
 * Inputs as in msa_kvouter_attention; nb_max = ceil(max_pages*page_size/128).
 */
typedef struct msa_index_out {
  uint8_t* slot_flag;    /* [Tq*Hkv*topk] */
  int32_t* tok_chain;    /* [Tq*Hkv] chain length of the token's tile */
  int32_t* tok_nres;     /* [Tq*Hkv] residual slots of (t, g) */
  int32_t* chain_blk;    /* [Tq*Hkv*topk] */
  int32_t* row_off;      /* [nb_max*Hkv + 1] */
  int32_t* unit_off;     /* [nb_max*Hkv + 1] */
  int32_t* ent;          /* [Tq*Hkv*topk] capacity */
  int32_t* slot_pos;     /* [Tq*Hkv*topk] */
  int32_t* tile_items;   /* [Tq*Hkv] capacity */
  int32_t* counters;     /* [8] */
} msa_index_out;

int32_t msa_build_index(const msa_tensor* selected, const msa_tensor* cu_seqlens_q,
                        const msa_tensor* used_kv_lens, int32_t Hq, int32_t nb_max,
                        int32_t causal, int32_t tile_tokens, int32_t unit_tokens,
                        int32_t list_all_tiles, const msa_index_out* out, void* stream);

/*
 * msa_widen_fp8 -- widen n e4m3fn values (device bytes `in`) to bf16 or fp16
 * (`out_dtype`, device buffer `out` of n elements) with the same conversion
 * the attention kernels apply to fp8 caches. Exposed for exhaustive tests of
 * that conversion. in and out must be 16-byte aligned; n % 16 == 0.
 */
int32_t msa_widen_fp8(const void* in, int64_t n, int32_t out_dtype, void* out, void* stream);

/*
 * msa_store_kv -- the paged K/V store, the step before the attention pass
 * (sglang pull request "Speed up MiniMax-M3 sparse attention on Hopper",
 * summary and "Verification": the fused K/V store with an unscaled cast of
 * 16-bit values to fp8 e4m3fn, bit-exact with
 * x.float().clamp(-448, 448).to(float8_e4m3fn)).
 *
 *   k_new, v_new  [N, Hkv, 128] bf16 or fp16 (the same dtype), the new
 *                 tokens' keys and values
 *   loc           [N] int64, the flat cache slot of each new token:
 *                 page * page_size + offset. A negative slot, or one at or
 *                 beyond num_pages * page_size, stores nothing.
 *   k_cache, v_cache  [num_pages, Hkv, page_size, 128], the layout the
 *                 attention pass reads, in the new values' dtype (copied
 *                 unchanged) or fp8_e4m3fn (each value clamped to [-448, 448]
 *                 and rounded to nearest even; NaN keeps its sign and becomes
 *                 the NaN code)
 *   page_size     64 or 128
 *
 * Row (i, g) of k_new / v_new goes to cache[loc[i] / page_size, g,
 * loc[i] % page_size, :]. v_new and v_cache may both be NULL: then only the
 * K rows are stored, which is how the sparse index K cache read by
 * msa_select_blocks (same layout) is written. Two new tokens with the same slot race (the result
 * is one of them). All buffers are caller-owned device memory, 16-byte
 * aligned; the call enqueues one kernel on `stream` and returns; the caches
 * are modified in place. Errors as for msa_kvouter_attention; N == 0
 * enqueues nothing.
 */
int32_t msa_store_kv(const msa_tensor* k_new, const msa_tensor* v_new, const msa_tensor* loc,
                     msa_tensor* k_cache, msa_tensor* v_cache, int32_t page_size, void* stream);

/*
 * msa_select_blocks -- block selection, the step that produces `selected`
 * (the MSA README, "How It Works" and "Highlighted Details": sparse top-k
 * selection; sglang pull request "Speed up MiniMax-M3 sparse attention on
 * Hopper", "Changes to existing code": the sparse index K cache, fp8 with an
 * fp8 KV cache). The pages do not give the scoring; this call implements:
 *
 *   score(t, g, b) = max over visible tokens j of block b (tokens
 *                    [128 b, 128 b + 128)) of q_idx[t, g, :] . k_idx(s, g, j, :)
 *
 * with j visible when j < used_kv_lens[s] and, when causal,
 * j <= pos(t) = used_kv_lens[s] - Tq_s + (t - cu_seqlens_q[s]) (the
 * attention pass's alignment). selected[t, g, :] lists the token's own block
 * first when force_local is 1 (the block of pos(t) when causal, the last
 * block when not), then the other blocks by descending score, equal scores by
 * ascending block id; -1 pads the rest. Blocks without a visible token and
 * NaN scores are never selected. Scores are accumulated in fp32 by MFMA.
 *
 *   q_idx         [Tq, Hkv, 128] bf16 or fp16, one index query per (token,
 *                 KV head)
 *   k_idx_cache   [num_pages, Hkv, page_size, 128] index keys in q_idx's
 *                 dtype or fp8_e4m3fn (scale 1), read through block_tables
 *   block_tables, cu_seqlens_q, used_kv_lens, page_size, causal: as for
 *                 msa_kvouter_attention (the same preconditions)
 *   topk          1 .. 2048, the width of `selected`
 *   selected      [Tq, Hkv, topk] int32, written
 *   scores        NULL, or [Tq, Hkv, nb] fp32 with nb = ceil(max_pages *
 *                 page_size / 128): written with every block's score (-inf
 *                 for blocks without a visible token)
 *
 * Sequences may reach at most 2048 blocks (nb <= 2048, else
 * MSA_ERR_UNSUPPORTED). All buffers are caller-owned device memory; the call
 * validates descriptors on the host, enqueues two kernels on `stream` (the
 * scores, then the lists) and returns. The fp32 score table of Tq * Hkv * nb
 * entries is `scores` when given, else the library's per-device workspace
 * (shared with msa_kvouter_attention: calls on different streams of one
 * device must not overlap in time). Errors as for msa_kvouter_attention; Tq
 * == 0 enqueues nothing.
 */
int32_t msa_select_blocks(const msa_tensor* q_idx, const msa_tensor* k_idx_cache,
                          const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                          const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                          int32_t topk, int32_t force_local, msa_tensor* selected,
                          msa_tensor* scores, void* stream);

/*
 * msa_validate_inputs -- synchronous check of the data-dependent
 * preconditions of msa_kvouter_attention (copies the small index arrays to
 * the host and waits for `stream`). Returns MSA_OK or MSA_ERR_PRECONDITION
 * with the first violation in msa_last_error(); descriptor errors are
 * reported as by msa_kvouter_attention.
 */
int32_t msa_validate_inputs(const msa_tensor* q, const msa_tensor* k_cache,
                            const msa_tensor* v_cache, const msa_tensor* selected,
                            const msa_tensor* block_tables, const msa_tensor* cu_seqlens_q,
                            const msa_tensor* used_kv_lens, int32_t page_size, int32_t causal,
                            void* stream);

/*
 * Kernel timing for benchmarks. msa_profile_enable(mask) makes every later
 * call time the kernels whose bit is set in `mask` (1 << MSA_KERNEL_*);
 * mask 0 turns timing off. Enabling discards earlier records. For each timed
 * launch of a kernel family the dispatches themselves record a pair of HIP
 * events (hipExtLaunchKernel): the start of the family's first kernel and
 * the end of its last, so a record measures kernel execution only, not the
 * host or the stream around it. msa_profile_collect waits for the recorded
 * events of one family and returns their summed duration (ms) and the
 * number of timed launches, then forgets them.
 */
enum {
  MSA_KERNEL_INDEX = 0, /* residual inversion: row counts and scan */
  MSA_KERNEL_FRONT = 1, /* classification + residual-free tiles of <= 16 rows */
  MSA_KERNEL_UNITS = 2, /* KV-outer units: partial O and LSE per residual slot */
  MSA_KERNEL_TILES = 3, /* listed tiles: chain blocks, LSE merge of the partials */
  MSA_KERNEL_STORE = 4, /* msa_store_kv */
  MSA_KERNEL_SELECT = 5, /* msa_select_blocks */
};
int32_t msa_profile_enable(uint32_t kernel_mask);
int32_t msa_profile_collect(int32_t kernel, double* total_ms, int64_t* launches);

/*
 * msa_set_workspace_limit -- cap the library-owned workspace of every device
 * at `bytes` (0: no cap, the default). A call whose workspace (planning
 * arrays, partial results, counters and bitmaps; msa_kvouter_workspace_bytes
 * reports about the same figure) would exceed the cap returns
 * MSA_ERR_OUT_OF_MEMORY and enqueues nothing; memory already held is kept.
 * Calls with a caller-owned workspace are not affected. Lets a caller bound
 * the library's memory, and lets tests force the out-of-memory path.
 */
int32_t msa_set_workspace_limit(size_t bytes);

/* Message of the last failing call on this thread ("" if none). */
const char* msa_last_error(void);

/* Library version string. */
const char* msa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_KVOUTER_H */
