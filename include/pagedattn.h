/*
 * pagedattn.h -- C ABI of libpagedattn.so: exact causal attention over a
 * KV cache split into fixed-size blocks, reached through per-sequence block
 * tables, on one AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *  - "Stateful Large Language Model Serving with Pensieve" (papercache.org
 *    summary), sections on attention (LLM与注意力机制), the multi-token
 *    kernel over non-contiguous KV (多Token注意力内核运算原理, 融合因果掩码与
 *    内核实现) and unified prefill/decode batches (统一Prefill和Generation
 *    阶段的执行过程).
 *  - "vLLM-SOSP23" (papers.lqhl.me), sections 核心方法 (block tables,
 *    copy-on-write) and Kernel 层实现 (block write, paged attention, block
 *    copy).
 *  - the devpress.csdn.net article on vLLM, sections 1 (block table worked
 *    example) and 2.1 (copy-on-write under parallel sampling).
 *  - "PagedAttention" (lib.yinfer.top), section 数学表述.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Memory.  Every pointer argument marked "device" is device memory on the
 *  current HIP device; "host" pointers are host memory.  The caller allocates
 *  and owns all buffers.  The library keeps no state between calls and never
 *  allocates device memory.
 *  Streams.  All GPU work is enqueued on `stream` (0 = the null stream) and
 *  every call returns without waiting for it; buffers must stay alive until
 *  that work completes.  Host pointers are read during the call only.
 *  Errors.  Every call returns a pa_status.  Argument errors are found on the
 *  host before anything is enqueued; then nothing is enqueued.
 *  pa_last_error() gives a thread-local message for the last non-OK status.
 *  Launch failures give PA_ERR_HIP.
 *
 *  Element types: PA_F32 (binary32), PA_F16 (binary16), PA_BF16 (bfloat16).
 *  Attention accumulates in fp32 and rounds its output once, to nearest even.
 *
 *  KV pools (one per layer, K and V separate; num_blocks physical blocks):
 *    k_cache[num_blocks][num_kv_heads][block_size][head_dim]
 *    v_cache[num_blocks][num_kv_heads][head_dim][block_size]
 *  i.e. inside a block and head, K is token-major and V is head-dim-major.
 *  A slot is block * block_size + offset.
 *
 *  Supported shapes: head_dim 64 or 128; block_size 4, 8, 16, 32 or 64 for
 *  every dtype, and 128 for fp16 / bf16 (the MFMA decode and multi-token
 *  paths take block_size 16..128 and a 16-bit dtype; other cases take a
 *  vector-ALU path with the same results within tolerance, which has no
 *  128-token blocks); num_q_heads a multiple of num_kv_heads with a group of
 *  1, 2, 4, 8 or 16 query heads per KV head.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, bad count, n > context, ... */
  PA_ERR_UNSUPPORTED = -2, /* dtype / head_dim / block_size / group not built */
  PA_ERR_WORKSPACE = -3,   /* workspace null or smaller than required */
  PA_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
  PA_ERR_BOUNDS = -5       /* PA_VALIDATE=1 found an id or slot out of range */
} pa_status;

/* Shape and element type of a KV pool pair. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pa_dtype */
} pa_cache_desc;

/* Optional tuning knobs; pass NULL for the defaults.  Results do not depend
 * on them beyond floating-point rounding order. */
typedef struct {
  /* Tokens per split of a single-token (decode) row's context; 0 = auto.
   * Rounded up to a multiple of 64.  Each split yields a partial softmax
   * state that a combine kernel merges. */
  int32_t decode_split_tokens;
  /* Keys per split of a multi-token request's context, rounded up to a
   * multiple of 128; 0 = auto.  Each (tile of rows, split) is a separate
   * work item; a new token whose causal range spans several splits gets one
   * partial softmax state per split, merged by the combine kernel (more
   * parallelism for few, long requests).  Auto cuts the longest work item
   * into equal splits of about half a workgroup's share of the batch's
   * multi-token work (at least 1024 keys, or 256 when the unsplit items fill
   * under a quarter of the GPU's workgroup slots), and only when that makes
   * two splits or more; PA_FLAG_NO_PREFILL_SPLIT turns it off.  The
   * workspace size depends on it. */
  int32_t prefill_split_tokens;
  /* Bit 0 (PA_FLAG_VECTOR_ALU): route every row through the vector-ALU row
   * kernel (the MFMA kernels are skipped).
   * Bit 1 (PA_FLAG_KV_UNSHARED): the caller asserts that no physical block
   * is read by two sequences of this call (no reference-count sharing, no
   * sub-requests over one table row).  Decode then streams K/V with
   * non-temporal loads, and its work items are listed longest first and
   * dealt round-robin over the XCDs (each XCD's L2 then serves an even share
   * of the work instead of the neighbouring rows that would share blocks);
   * faster when nothing is re-read, slower when blocks are shared; results
   * are identical either way.
   * Bit 2 (PA_FLAG_NO_PREFILL_SPLIT): with prefill_split_tokens = 0, never
   * split multi-token contexts.
   * Other bits must be 0. */
  int32_t flags;
  /* Profiling hook: when timed_kernel is one of PA_TIME_* and that kernel is
   * launched, timing_start / timing_end (caller-created hipEvent_t, may be
   * NULL) are recorded on `stream` immediately before and after it. */
  int32_t timed_kernel;
  hipEvent_t timing_start;
  hipEvent_t timing_end;
  /* Rows of (token, head) pairs per multi-token MFMA work item: 128 (4
   * waves) or 256 (8 waves sharing each staged K/V tile); 0 = auto (256 when
   * the batch has enough work items to fill the GPU). */
  int32_t prefill_tile_rows;
} pa_options;

enum { PA_TIME_NONE = 0, PA_TIME_TILE = 1, PA_TIME_ROWS = 2, PA_TIME_COMBINE = 3 };
enum { PA_FLAG_VECTOR_ALU = 1, PA_FLAG_KV_UNSHARED = 2, PA_FLAG_NO_PREFILL_SPLIT = 4 };

/*
 * pa_write_kv -- slot-mapping scatter of new K/V into the pools.
 *
 * Pensieve page (统一Prefill和Generation阶段的执行过程): newly computed K and
 * V of every batched token are stored into the cache slots allocated for them
 * before attention runs.  vLLM-SOSP23 page (Kernel 层实现): the reshape and
 * the block write are one fused kernel.
 *
 *  k_new, v_new   device, [num_tokens][num_kv_heads][head_dim], c->dtype.
 *  slot_mapping   device int64 [num_tokens]; token t goes to block
 *                 slot / block_size, offset slot % block_size.  A negative
 *                 slot skips the token.  Slots >= num_blocks * block_size are
 *                 skipped too (PA_VALIDATE=1 reports them as PA_ERR_BOUNDS).
 *  k_cache, v_cache  device pools (layout above), written in place.
 *  Precondition: slots within one call are distinct.  The copy is bit-exact.
 *  num_tokens == 0 is valid and enqueues nothing.  A call moves at most
 *  2^31 - 1 16-byte chunks of K (num_tokens rounded up to 32, times
 *  num_kv_heads times head_dim * elt / 16); beyond that it returns
 *  PA_ERR_UNSUPPORTED (split the call).  pa_write_kv_attention has the same
 *  limit for its total_q new tokens.
 */
pa_status pa_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache,
                      const pa_cache_desc* c, hipStream_t stream);

/*
 * pa_copy_blocks -- batched whole-block copy for copy-on-write.
 *
 * devpress.csdn.net vLLM article, section 2.1: a writer that finds its block
 * shared (reference count > 1) gets a new physical block into which the old
 * block is copied; vLLM-SOSP23 page (Kernel 层实现) names the batched block
 * copy kernel.
 *
 *  block_pairs  device int32 [num_pairs][2] = (src, dst); for every pair both
 *               K and V of all heads of block src are copied to block dst.
 *               Pairs with an id outside [0, num_blocks) are skipped
 *               (PA_VALIDATE=1 reports PA_ERR_BOUNDS).
 *  Precondition: destinations are distinct and no destination is a source in
 *  the same call, so pairs may run in any order.  Bit-exact.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* c,
                         const int32_t* block_pairs, int32_t num_pairs, hipStream_t stream);

/*
 * pa_copy_blocks_layers -- the copies of pa_copy_blocks on every layer's pools
 * in one launch.
 *
 * vLLM-SOSP23 page (Kernel 层实现): the copy-on-write block copies are
 * batched into one kernel; a model keeps one pool pair per layer and the same
 * block ids in each, so one launch serves all layers.
 *
 *  k_caches, v_caches  HOST arrays of num_layers device pool pointers (read
 *                      during the call, may be freed after it); every layer's
 *                      pools have the shape and dtype of *c.
 *  num_layers          0..PA_MAX_LAYERS; more layers take several calls.
 *  block_pairs, num_pairs, precondition, bounds and exactness as for
 *  pa_copy_blocks, applied to each layer.
 */
#define PA_MAX_LAYERS 128
pa_status pa_copy_blocks_layers(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                                const pa_cache_desc* c, const int32_t* block_pairs,
                                int32_t num_pairs, hipStream_t stream);

/*
 * pa_swap_blocks -- move whole blocks between the device pool and a host pool.
 *
 * Pensieve page (流水线KV缓存恢复, 提前交换, 实现细节与优化): K/V tokens evicted
 * from GPU memory live in a CPU cache and are copied back before the layer
 * that needs them runs; vLLM-SOSP23 page (调度与抢占): preempted sequences'
 * blocks are swapped to CPU memory and back.  Runs of consecutive block
 * pairs are merged; up to 8 runs go to the DMA engines (hipMemcpyAsync on
 * `stream`, leaving the compute units free), more runs to a copy kernel on
 * `stream` that addresses the pinned host pool directly (each DMA transfer
 * has a fixed submission cost).
 *
 *  dev_k, dev_v     device pools, layout and shape of *c.
 *  host_k, host_v   host pools with the same per-block layout and
 *                   host_num_blocks blocks; pinned (hipHostMalloc, or torch
 *                   pin_memory=True).  Unpinned memory takes the DMA path
 *                   with synchronous copies.
 *  block_pairs      HOST int32 [num_pairs][2] = (src, dst), read during the
 *                   call: PA_SWAP_OUT copies device block src to host block
 *                   dst, PA_SWAP_IN host block src to device block dst.  Ids
 *                   outside their pool give PA_ERR_BOUNDS and nothing is
 *                   enqueued.  Destinations must be distinct.  Bit-exact.
 *  direction        PA_SWAP_OUT or PA_SWAP_IN.
 * The caller orders swaps against attention with events (the page gates each
 * layer's attention on the event that ends its swap-in).
 */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };
pa_status pa_swap_blocks(void* dev_k, void* dev_v, const pa_cache_desc* c, void* host_k,
                         void* host_v, int32_t host_num_blocks, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t direction, hipStream_t stream);

/*
 * pa_attention_workspace_size -- bytes of device workspace pa_attention needs
 * for a batch of num_seqs sequences, total_q query rows, and no context longer
 * than max_context_len, with the given options (NULL = defaults).
 */
size_t pa_attention_workspace_size(const pa_cache_desc* c, int32_t num_q_heads,
                                   int32_t num_seqs, int32_t total_q,
                                   int32_t max_context_len, const pa_options* opt);

/*
 * pa_attention_plan -- the plan pa_attention would make for a batch, on the
 * host only (no GPU work, no device memory touched).
 *
 * Pensieve page (实验结果, multi-token kernel): the per-request auxiliary data
 * that lets the paged kernel run like a contiguous one is derived on the CPU
 * side; this call exposes what the library derives from the host mirrors.
 *
 *  Arguments as for pa_attention; workspace_bytes is the workspace the call
 *  would be given (the automatic multi-token split is lengthened until its
 *  partial states fit it).  info (may be NULL) receives the work counts, the
 *  chosen split lengths and tile rows, and the workspace bytes the plan
 *  occupies.  Returns PA_OK when the plan fits workspace_bytes,
 *  PA_ERR_WORKSPACE when it does not (info is still filled), or the argument
 *  error pa_attention would return.
 */
typedef struct {
  int64_t row_items;             /* single-row work items (row, key split) */
  int64_t tile_items;            /* multi-token work items (row tile, key split) */
  int64_t combine_items;         /* rows whose key splits are merged */
  int64_t partial_slots;         /* partial softmax states of split rows */
  int32_t decode_split_tokens;   /* keys per split of a single row */
  int32_t prefill_split_tokens;  /* keys per split of a multi-token context, 0 = none */
  int32_t prefill_tile_rows;     /* (token, head) rows per multi-token work item */
  int32_t reserved;              /* 0 */
  size_t workspace_bytes;        /* workspace the plan occupies */
} pa_plan_info;
pa_status pa_attention_plan(const pa_cache_desc* c, int32_t num_q_heads,
                            int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_q,
                            const int32_t* context_lens_host, const int32_t* query_start_loc_host,
                            size_t workspace_bytes, const pa_options* opt, pa_plan_info* info);

/*
 * pa_attention -- causal attention of a ragged batch over the paged cache.
 *
 * Pensieve page (LLM与注意力机制): A = Q K^T * scale, O = softmax(A) V per
 * head.  "PagedAttention" page (数学表述): query i attends to keys up to its
 * own position.  vLLM-SOSP23 page (核心方法): K/V are read by indirection
 * through the block table, exactly, with no approximation.  Pensieve page
 * (多Token注意力内核运算原理, 统一Prefill和Generation阶段的执行过程): a batch
 * concatenates each request's new tokens -- one for a decode, many for a
 * prefill -- and per-request auxiliary data delimits them; the causal mask is
 * fused into the kernel.
 *
 *  out             device [total_q][num_q_heads][head_dim], c->dtype.
 *  q               device [total_q][num_q_heads][head_dim], c->dtype.
 *  k_cache,v_cache device pools (layout above); not modified.
 *  num_q_heads     query heads; query head h reads KV head h / (num_q_heads /
 *                  num_kv_heads).
 *  block_tables    device int32 [num_seqs][max_blocks_per_seq]; entry j of
 *                  row s is the physical block of tokens [j*bs, (j+1)*bs) of
 *                  sequence s.  Entries at or beyond ceil(L_s / bs) are never
 *                  read.  Ids must lie in [0, num_blocks).
 *  context_lens    device int32 [num_seqs]: L_s, the context length including
 *                  the sequence's new tokens (which pa_write_kv must already
 *                  have stored).
 *  query_start_loc device int32 [num_seqs + 1]: rows of sequence s are
 *                  [qsl[s], qsl[s+1]); n_s = qsl[s+1] - qsl[s] new tokens,
 *                  which are the last n_s context positions: row i of s
 *                  attends to positions 0 .. L_s - n_s + i.  n_s = 0 is
 *                  allowed.  qsl[0] must be 0 and qsl[num_seqs] = total_q.
 *  context_lens_host, query_start_loc_host
 *                  host mirrors of the two arrays above, with identical
 *                  contents; used on the host for validation and launch
 *                  sizing.
 *  scale           multiplies q.k (usually 1/sqrt(head_dim)).
 *  workspace       device, 256-byte aligned, at least the bytes the batch's
 *                  plan occupies (pa_attention_plan); a workspace of
 *                  pa_attention_workspace_size(...) bytes always suffices.
 *                  Contents on entry are ignored; on return it holds the
 *                  plan and its status (pa_attention_check).
 *  opt             NULL or tuning options (same as given to the size query).
 *  Errors: PA_ERR_INVALID_ARG if num_q_heads % num_kv_heads != 0, n_s > L_s,
 *  qsl is not non-decreasing from 0 to total_q, or L_s > max_blocks_per_seq*bs;
 *  PA_ERR_WORKSPACE if the workspace is too small.  Device data that
 *  disagree with the host mirrors are reported by pa_attention_check.
 *  Sub-requests (two query ranges over one context) are expressed by giving
 *  two sequences the same block-table row with different context_lens and
 *  query ranges.
 */
pa_status pa_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const pa_cache_desc* c, int32_t num_q_heads,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* query_start_loc,
                       int32_t num_seqs, int32_t total_q,
                       const int32_t* context_lens_host, const int32_t* query_start_loc_host,
                       float scale, void* workspace, size_t workspace_bytes,
                       const pa_options* opt, hipStream_t stream);

/*
 * pa_write_kv_attention -- the new tokens' K/V written into the pools, then
 * attention over them: the result of pa_write_kv(k_new, v_new, slot_mapping,
 * total_q, ...) followed by pa_attention(...), in one call.
 *
 * vLLM-SOSP23 page (Kernel 层实现): the block write of new K/V is fused with
 * the work around it to save launches.  Pensieve page
 * (统一Prefill和Generation阶段的执行过程): each batched token's new K/V is
 * stored into its slot before attention reads it.
 *
 * The write shares one launch with the attention planner (neither reads what
 * the other writes), so the call has one launch fewer than the two calls it
 * replaces; the attention kernels then read the new tokens from the pools.
 *
 *  k_new, v_new    device [total_q][num_kv_heads][head_dim], c->dtype, 16-byte
 *                  aligned: row t is the K/V of query row t (the new tokens
 *                  are the queries).
 *  slot_mapping    device int64 [total_q]; the slot of query row t's token,
 *                  as for pa_write_kv (its PA_VALIDATE=1 checks included).
 *  k_cache,v_cache device pools, modified at the new tokens' slots.
 *  Other arguments, errors and options as for pa_attention.
 */
pa_status pa_write_kv_attention(void* out, const void* q, const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                const pa_cache_desc* c, int32_t num_q_heads,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int32_t total_q,
                                const int32_t* context_lens_host,
                                const int32_t* query_start_loc_host, float scale,
                                void* workspace, size_t workspace_bytes, const pa_options* opt,
                                hipStream_t stream);

/*
 * pa_write_kv_attention_static -- pa_write_kv_attention without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The plan, split states and status live in a static device array of
 * PA_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends.  The call allocates nothing: its first call on a device
 * looks up that device's copy of the array, later calls reuse it.
 *  Arguments, results, options and errors as for pa_write_kv_attention, with
 *  the workspace replaced by the static scratch.  A batch whose plan needs
 *  more than PA_STATIC_SCRATCH_BYTES (pa_attention_plan with that size
 *  reports it) returns PA_ERR_WORKSPACE and enqueues nothing.  Under
 *  PA_VALIDATE=1 only the final status check runs (the other checks copy
 *  into host buffers).
 *  Every call on one GPU shares that GPU's scratch, which keeps the last
 *  call's contents (each call writes what it reads first, so nothing needs
 *  clearing): calls that overlap on one GPU -- on two streams, or from two
 *  host threads -- race and must be serialized by the caller.
 */
#define PA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_write_kv_attention_static(void* out, const void* q, const void* k_new,
                                       const void* v_new, const int64_t* slot_mapping,
                                       void* k_cache, void* v_cache, const pa_cache_desc* c,
                                       int32_t num_q_heads, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       const int32_t* query_start_loc, int32_t num_seqs,
                                       int32_t total_q, const int32_t* context_lens_host,
                                       const int32_t* query_start_loc_host, float scale,
                                       const pa_options* opt, hipStream_t stream);

/*
 * pa_attention_check -- wait for `stream`, then report whether the last
 * pa_attention / pa_write_kv_attention call that used `workspace` ran every
 * work item it was sized for.
 *
 * The grids of a call are sized on the host from the host mirrors, and the
 * device plans from context_lens / query_start_loc.  If the two disagree, or
 * a kernel meets an index outside the batch or the workspace, work is skipped
 * (never read or written out of bounds) and the call's first kernel records
 * it in the workspace.  PA_OK: every item ran.  PA_ERR_BOUNDS: the
 * descriptions differed or work was skipped; the output is not valid.
 * PA_ERR_HIP: the stream or the read failed.  Under PA_VALIDATE=1 every
 * attention call ends with this check (and so synchronizes).
 */
pa_status pa_attention_check(const void* workspace, hipStream_t stream);

/* Thread-local text of the last non-OK status returned on this thread. */
const char* pa_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
