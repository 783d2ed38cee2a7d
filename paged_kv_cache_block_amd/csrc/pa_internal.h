// Host-side declarations shared by the C ABI (pa_api.cpp) and the kernel
// launch wrappers of libpagedattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Rows of packed (token, head) pairs per MFMA workgroup: 4 waves x 32 rows,
// or 8 waves x 32 rows for batches with enough tiles to fill the GPU.
constexpr int kTileRows = 128;
constexpr int kTileRowsWide = 256;
// 256-row workgroups (8 waves sharing each staged K/V tile) issue half the
// tile loads and LDS stores per MFMA; they pay off once a batch has enough of
// them to keep every CU busy.
constexpr int kWideTileMinGroups = 1024;
// Automatic split length of single-row work: about kAutoTargetWaves * 2 /
// (G + 1) wavefronts over the whole batch (G query heads per KV head: every
// split of a row writes G partial states for the combine, so larger groups
// take fewer, longer splits), clamped to [kMinAutoSplit, kMaxAutoSplit] keys
// and rounded to a multiple of 64.
constexpr int kAutoTargetWaves = 8192;
// Multi-token key splits are whole numbers of this many keys (the largest
// MFMA tile), so no tile straddles two splits.
constexpr int kPrefillSplitQuantum = 128;
constexpr int kMinAutoSplit = 64;
// (The cap matters for large GQA batches: the long mixed bf16 batch's 128
// decode rows take 1472-key splits, 4.6% faster than 1024 once its row items
// are dealt evenly over the XCDs.)
constexpr int kMaxAutoSplit = 2048;

struct PoolArgs {
  int num_blocks, block_size, num_kv_heads, head_dim, dtype;
};

// Byte offsets of the plan inside the workspace and the capacities behind them.
struct WorkspaceLayout {
  size_t counts, rows, tiles, combs, part_ml, part_o, total;
  int64_t cap_rows, cap_tiles, cap_combs, cap_partials;
};

struct PlanParams {
  int num_seqs;
  int split_tokens;   // keys per split of a row-kernel row
  int group;          // query heads per KV head
  int vector_all;     // 1: every row goes to the row kernel
  int tile_rows;      // rows per MFMA multi-token work item
  int prefill_split;  // keys per split of a multi-token sequence (0: none)
  int rows_dealt;     // 1: list row items longest first, for dealing over the XCDs
  int row_shift;      // row items' length buckets: (split - keys) >> row_shift
  int64_t cap_rows, cap_tiles, cap_combs, cap_partials;
  // The counts the host derived from its mirrors (the launch sizes).
  int64_t want_rows, want_tiles, want_combs, want_partials;
  // Multi-token items are listed longest first, bucketed by their key count
  // >> lpt_shift (chosen so the longest context fits kLptBuckets buckets).
  int lpt_shift;
};
constexpr int kLptBuckets = 512;
// Row items listed longest first go in this many buckets of split length.
constexpr int kRowBuckets = 64;

// A kernel that must skip work it was handed (an index outside the batch or
// the workspace: the device batch disagrees with the host mirrors) records it
// here for pa_attention_check.  Every writer stores the same value.
__device__ __forceinline__ void mark_dropped(const void* ws, const WorkspaceLayout& lay) {
  volatile int32_t* d = &reinterpret_cast<PlanCounts*>(static_cast<uint8_t*>(const_cast<void*>(ws)) + lay.counts)->dropped;
  *d = 1;
}

hipError_t launch_write_kv(const void* k_new, const void* v_new, const int64_t* slots,
                           int num_tokens, void* k_cache, void* v_cache, const PoolArgs& p,
                           hipStream_t s);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const PoolArgs& p,
                              const int32_t* pairs, int num_pairs, hipStream_t s);
// Pool pointers of every layer, passed by value to the multi-layer copy.
constexpr int kMaxLayers = 128;
struct LayerPools {
  void* k[kMaxLayers];
  void* v[kMaxLayers];
};
hipError_t launch_copy_blocks_layers(const LayerPools& lp, int num_layers, const PoolArgs& p,
                                     const int32_t* pairs, int num_pairs, hipStream_t s);
// Block copies between a device pool and a host pool the device can address
// (pinned, mapped): the pairs travel in the kernel arguments.
constexpr int kSwapPairsPerLaunch = 448;
// Swaps with more runs of consecutive blocks than this use the copy kernel.
constexpr int kSwapDmaMaxRuns = 8;
struct SwapPairs {
  int32_t p[2 * kSwapPairsPerLaunch];
};
hipError_t launch_swap_kernel(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const PoolArgs& p, const SwapPairs& pairs, int n, hipStream_t s);
hipError_t launch_plan(const int32_t* context_lens, const int32_t* qsl, const PlanParams& pp,
                       void* ws, const WorkspaceLayout& lay, hipStream_t s);
// The plan and the slot-mapping write of num_tokens new tokens in one launch
// (the plan reads no pool, the write no plan).
hipError_t launch_plan_write(const int32_t* context_lens, const int32_t* qsl, const PlanParams& pp,
                             void* ws, const WorkspaceLayout& lay, const void* k_new,
                             const void* v_new, const int64_t* slots, int num_tokens,
                             void* k_cache, void* v_cache, const PoolArgs& p, hipStream_t s);

struct AttnArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* qsl;
  int max_blocks;
  int num_q_heads;
  int total_q;
  float scale_log2;   // scale * log2(e)
  void* ws;
  int prefill_split;  // keys per split of a multi-token sequence (0: none)
  int rows_dealt;     // 1: row items are listed longest first and dealt over the XCDs
};

hipError_t launch_row_attention(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                                int num_items, int split_tokens, hipStream_t s);
bool decode_mfma_supported(const PoolArgs& p, int group);
hipError_t launch_decode_mfma(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                              int num_items, int split_tokens, bool stream_kv, hipStream_t s);
// Workgroups of the decode kernel's grid: one per (row item, KV head), or,
// with row items dealt over the XCDs, whole rounds of 8 items.
int64_t decode_mfma_groups(int64_t num_items, int num_kv_heads, bool dealt);
hipError_t launch_combine(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                          int num_combs, hipStream_t s);
hipError_t launch_tile_attention(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                                 int num_tiles, int tile_rows, hipStream_t s);
bool tile_path_supported(const PoolArgs& p);

}  // namespace pa
