// C ABI of libpagedattn: argument checks, workspace layout, launch sizing.
// Declarations and contracts are in include/pagedattn.h.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "pa_write.h"
#include "pagedattn.h"

using namespace pa;

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool validate_mode() {
  const char* v = getenv("PA_VALIDATE");
  return v && v[0] == '1';
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

pa_status check_desc(const pa_cache_desc* c, PoolArgs* p) {
  if (!c) return fail(PA_ERR_INVALID_ARG, "cache descriptor is null");
  if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "dtype %d not supported", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", c->head_dim);
  if (c->block_size != 4 && c->block_size != 8 && c->block_size != 16 && c->block_size != 32 &&
      c->block_size != 64 && c->block_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (4, 8, 16, 32, 64, 128)", c->block_size);
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_blocks and num_kv_heads must be positive");
  *p = PoolArgs{c->num_blocks, c->block_size, c->num_kv_heads, c->head_dim, c->dtype};
  return PA_OK;
}

// Copy a small device array to the host (used only under PA_VALIDATE=1).
template <typename T>
pa_status fetch(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "PA_VALIDATE copy");
  return PA_OK;
}

// Split length of row work.  `total_keys` is the sum over rows of the keys
// each row attends to (only known at call time; -1 in size queries).
int choose_split(const pa_options* opt, int64_t total_keys, int num_kv_heads, int group) {
  if (opt && opt->decode_split_tokens > 0) return (opt->decode_split_tokens + 63) / 64 * 64;
  if (total_keys < 0) return kMinAutoSplit;
  const int64_t target = (int64_t)kAutoTargetWaves * 2 / (group + 1);
  int64_t want = (total_keys * num_kv_heads + target - 1) / target;
  want = (want + 63) / 64 * 64;
  return (int)std::min<int64_t>(kMaxAutoSplit, std::max<int64_t>(kMinAutoSplit, want));
}

// Keys per split of a multi-token sequence given by the option, rounded up to
// a whole number of 128-key MFMA tiles; 0 = none given.
int prefill_split(const pa_options* opt) {
  if (!opt || opt->prefill_split_tokens <= 0) return 0;
  return (opt->prefill_split_tokens + kPrefillSplitQuantum - 1) / kPrefillSplitQuantum * kPrefillSplitQuantum;
}

// Automatic multi-token key split: with W keys of tile work over P resident
// workgroups, a target of w = max(W / (2P), floor) keys per split.  The
// longest item is cut into floor(longest / w) equal splits (rounded up to the
// quantum), and nothing is split when that is fewer than two: a split that
// only trims an item costs its partial states and their combine without
// shortening the launch.  Nor is an item cut into more pieces than make the
// batch's items fill the workgroup slots once (two pieces are always
// allowed).  The floor is kMinAutoPrefillSplit, or kMinAutoPrefillSplitSparse
// when the unsplit items fill less than a quarter of the slots (then
// parallelism outweighs the partial states).  When the unsplit items fill
// every slot already, nothing is split either while the longest item is
// under twice a slot's fair share W / P: the planner lists items longest
// first, so such an item starts first and ends within the launch's length
// (on the unified fp16 batch, 640 items over 512 slots with a longest item
// of 1.5 shares, splitting gained nothing and cost 36 MB of partial-state
// writes).
constexpr int kMinAutoPrefillSplit = 1024;
constexpr int kMinAutoPrefillSplitSparse = 256;

bool auto_prefill_split(const pa_options* opt) {
  return prefill_split(opt) == 0 && !(opt && (opt->flags & PA_FLAG_NO_PREFILL_SPLIT));
}

// Compute units of the current device (cached per device).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Automatic key split of a batch's multi-token work (see kMinAutoPrefillSplit):
// 0 when the longest item is shorter than two target splits.
int choose_prefill_split(const int32_t* lens, const int32_t* qsl, int num_seqs, int group,
                         int tile_rows, int num_kv_heads) {
  int64_t work = 0, items = 0;
  int longest = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = qsl[s + 1] - qsl[s];
    const SeqWork w = seq_work(n, 0, group, tile_rows);
    items += w.tiles;
    for (int t = 0; t < w.tiles; ++t) {
      const int k = tile_key_end(n, lens[s], group, tile_rows, t);
      work += k;
      longest = std::max(longest, k);
    }
  }
  if (work == 0) return 0;
  const int64_t slots = (int64_t)cu_count() * (tile_rows == kTileRowsWide ? 1 : 2);
  if (items * num_kv_heads >= slots && (int64_t)longest * slots < 2 * work * num_kv_heads) return 0;
  const bool sparse = items * num_kv_heads * 4 < slots;
  const int64_t want = std::max<int64_t>(work * num_kv_heads / (2 * slots),
                                         sparse ? kMinAutoPrefillSplitSparse : kMinAutoPrefillSplit);
  // Split up to filling the slots once, not beyond (more items than slots
  // add a round and more partial states to combine), but at least in two
  // where the longest item is that much longer than the target.
  const int64_t pieces =
      std::min<int64_t>(longest / want, std::max<int64_t>(2, slots / (items * num_kv_heads)));
  if (pieces < 2) return 0;
  const int64_t split = (longest + pieces - 1) / pieces;
  return (int)((split + kPrefillSplitQuantum - 1) / kPrefillSplitQuantum * kPrefillSplitQuantum);
}

bool vector_all(const PoolArgs& p, const pa_options* opt) {
  return (opt && (opt->flags & PA_FLAG_VECTOR_ALU)) || !tile_path_supported(p);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WorkspaceLayout make_layout(const PoolArgs& p, int hq, int num_seqs, int total_q, int max_len,
                            const pa_options* opt) {
  WorkspaceLayout w{};
  const bool va = vector_all(p, opt);
  const int64_t row_rows = va ? total_q : std::min(num_seqs, total_q);
  const int group = hq / p.num_kv_heads;
  if (opt && opt->decode_split_tokens > 0) {
    const int split = choose_split(opt, -1, p.num_kv_heads, group);
    w.cap_rows = row_rows * row_splits(std::max(max_len, 1), split);
  } else {
    // Every row has at most keys/split + 1 splits.  With the automatic split,
    // sum(keys)/split <= kAutoTargetWaves / H_kv unless the split is clamped at
    // kMaxAutoSplit, where sum(keys)/split <= rows * max_len / kMaxAutoSplit.
    w.cap_rows = row_rows + (kAutoTargetWaves + p.num_kv_heads - 1) / p.num_kv_heads +
                 row_rows * ((std::max(max_len, 1) + kMaxAutoSplit - 1) / kMaxAutoSplit);
  }
  w.cap_combs = row_rows;
  w.cap_partials = w.cap_rows;
  w.cap_tiles = va ? 0 : ((int64_t)total_q * group + kTileRows - 1) / kTileRows + num_seqs;
  // Room for automatic splits of kMinAutoPrefillSplit keys; shorter ones are
  // lengthened at call time until they fit.
  const int ps = auto_prefill_split(opt) ? kMinAutoPrefillSplit : prefill_split(opt);
  if (!va && ps > 0) {
    // Every tile has at most key_splits(max_len) splits; every new token at
    // most that many partial slots and one combine item.
    const int64_t ks = key_splits(std::max(max_len, 1), ps);
    w.cap_tiles *= ks;
    w.cap_partials += (int64_t)total_q * ks;
    w.cap_combs += total_q;
  }
  size_t off = 0;
  w.counts = off; off = align256(off + sizeof(PlanCounts));
  w.rows = off;   off = align256(off + sizeof(RowItem) * (size_t)w.cap_rows);
  w.tiles = off;  off = align256(off + sizeof(TileItem) * (size_t)w.cap_tiles);
  w.combs = off;  off = align256(off + sizeof(CombItem) * (size_t)w.cap_combs);
  w.part_ml = off; off = align256(off + 8ull * (size_t)w.cap_partials * hq);
  w.part_o = off;  off = align256(off + 4ull * (size_t)w.cap_partials * hq * p.head_dim);
  w.total = off;
  return w;
}

// The layout of one call's plan, sized by its exact work counts (never more
// than make_layout's bound for a batch within that bound's arguments).
WorkspaceLayout exact_layout(const PoolArgs& p, int hq, int64_t rows, int64_t tiles, int64_t combs,
                             int64_t partials) {
  WorkspaceLayout w{};
  w.cap_rows = rows;
  w.cap_tiles = tiles;
  w.cap_combs = combs;
  w.cap_partials = partials;
  size_t off = 0;
  w.counts = off; off = align256(off + sizeof(PlanCounts));
  w.rows = off;   off = align256(off + sizeof(RowItem) * (size_t)rows);
  w.tiles = off;  off = align256(off + sizeof(TileItem) * (size_t)tiles);
  w.combs = off;  off = align256(off + sizeof(CombItem) * (size_t)combs);
  w.part_ml = off; off = align256(off + 8ull * (size_t)partials * hq);
  w.part_o = off;  off = align256(off + 4ull * (size_t)partials * hq * p.head_dim);
  w.total = off;
  return w;
}

// Everything the host decides about one attention call: checked shapes, the
// split and tile choices, the exact work counts and the workspace layout.
struct CallPlan {
  PoolArgs p;
  int group = 0, max_len = 0, split = 0, tile_rows = kTileRows, psplit = 0;
  bool va = false, rows_on_mfma = false;
  // Row items listed longest first and dealt round-robin over the XCDs (each
  // gets an even share of the work).  Only where no block is read by two
  // sequences: sharers of a prompt then no longer meet in one L2.
  bool rows_dealt = false;
  int64_t n_rows = 0, n_tiles = 0, n_combs = 0, n_partials = 0;
  WorkspaceLayout lay{};
};

pa_status plan_call(const pa_cache_desc* c, int32_t num_q_heads, int32_t max_blocks_per_seq,
                    int32_t num_seqs, int32_t total_q, const int32_t* context_lens_host,
                    const int32_t* query_start_loc_host, size_t workspace_bytes,
                    const pa_options* opt, CallPlan* cp);
pa_status read_status(const void* workspace, hipStream_t stream);

// PA_VALIDATE checks of a slot mapping: every slot inside the pool, no slot
// twice.  The mapping is left in `slots`.
pa_status check_slots(std::vector<int64_t>& slots, const int64_t* slot_mapping, int num_tokens,
                      const PoolArgs& p, hipStream_t stream) {
  pa_status st = fetch(slots, slot_mapping, (size_t)num_tokens, stream);
  if (st != PA_OK) return st;
  const int64_t total = (int64_t)p.num_blocks * p.block_size;
  std::vector<int64_t> seen;
  for (int64_t sl : slots) {
    if (sl >= total) return fail(PA_ERR_BOUNDS, "slot %lld out of range", (long long)sl);
    if (sl >= 0) seen.push_back(sl);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(PA_ERR_BOUNDS, "duplicate slot in slot_mapping");
  return PA_OK;
}

// New tokens written by the fused entry point (null: plain attention).
struct FusedWrite {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
};

pa_status attention_impl(void* out, const void* q, void* k_cache, void* v_cache,
                         const pa_cache_desc* c, int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
                         const int32_t* context_lens_host, const int32_t* query_start_loc_host,
                         float scale, void* workspace, size_t workspace_bytes,
                         const pa_options* opt, const FusedWrite* fw, hipStream_t stream,
                         bool static_scratch);

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_version(void) { return 100; }

pa_status pa_write_kv(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache, const pa_cache_desc* c,
                      hipStream_t stream) {
  PoolArgs p;
  pa_status st = check_desc(c, &p);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  if (write_geom(num_tokens, p).chunks > 0x7fffffff)
    return fail(PA_ERR_UNSUPPORTED, "too many new tokens for one write (at most 2^31 - 1 16-byte chunks)");
  if (validate_mode()) {
    std::vector<int64_t> slots;
    if ((st = check_slots(slots, slot_mapping, num_tokens, p, stream)) != PA_OK) return st;
  }
  hipError_t e = launch_write_kv(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, p, stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "write_kv launch");
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const pa_cache_desc* c,
                         const int32_t* block_pairs, int32_t num_pairs, hipStream_t stream) {
  PoolArgs p;
  pa_status st = check_desc(c, &p);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs < 0");
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "K/V pools must be 16-byte aligned");
  if (validate_mode()) {
    std::vector<int32_t> pr;
    if ((st = fetch(pr, block_pairs, 2 * (size_t)num_pairs, stream)) != PA_OK) return st;
    std::vector<int32_t> dsts, srcs;
    for (int i = 0; i < num_pairs; ++i) {
      const int32_t a = pr[2 * i], b = pr[2 * i + 1];
      if (a < 0 || a >= p.num_blocks || b < 0 || b >= p.num_blocks)
        return fail(PA_ERR_BOUNDS, "block pair (%d, %d) out of range", a, b);
      srcs.push_back(a);
      dsts.push_back(b);
    }
    std::sort(dsts.begin(), dsts.end());
    std::sort(srcs.begin(), srcs.end());
    if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end())
      return fail(PA_ERR_BOUNDS, "duplicate destination block");
    for (int32_t d : dsts)
      if (std::binary_search(srcs.begin(), srcs.end(), d))
        return fail(PA_ERR_BOUNDS, "block %d is both a source and a destination", d);
  }
  hipError_t e = launch_copy_blocks(k_cache, v_cache, p, block_pairs, num_pairs, stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "copy_blocks launch");
}

pa_status pa_swap_blocks(void* dev_k, void* dev_v, const pa_cache_desc* c, void* host_k,
                         void* host_v, int32_t host_num_blocks, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t direction, hipStream_t stream) {
  PoolArgs p;
  pa_status st = check_desc(c, &p);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || host_num_blocks < 0) return fail(PA_ERR_INVALID_ARG, "negative count");
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID_ARG, "direction must be PA_SWAP_OUT or PA_SWAP_IN");
  if (num_pairs == 0) return PA_OK;
  if (!dev_k || !dev_v || !host_k || !host_v || !block_pairs)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  const bool out = direction == PA_SWAP_OUT;
  const int64_t src_n = out ? p.num_blocks : host_num_blocks;
  const int64_t dst_n = out ? host_num_blocks : p.num_blocks;
  std::vector<int32_t> dsts;
  dsts.reserve(num_pairs);
  for (int i = 0; i < num_pairs; ++i) {
    const int32_t a = block_pairs[2 * i], b = block_pairs[2 * i + 1];
    if (a < 0 || a >= src_n || b < 0 || b >= dst_n)
      return fail(PA_ERR_BOUNDS, "swap pair (%d, %d) out of range", a, b);
    dsts.push_back(b);
  }
  std::sort(dsts.begin(), dsts.end());
  if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end())
    return fail(PA_ERR_BOUNDS, "duplicate destination block");
  const size_t blk = (size_t)p.num_kv_heads * p.block_size * p.head_dim * (p.dtype == DT_F32 ? 4 : 2);
  char* sk = static_cast<char*>(out ? dev_k : host_k);
  char* sv = static_cast<char*>(out ? dev_v : host_v);
  char* dk = static_cast<char*>(out ? host_k : dev_k);
  char* dv = static_cast<char*>(out ? host_v : dev_v);
  const hipMemcpyKind kind = out ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  // Runs of pairs whose sources and destinations both advance by one block
  // become one DMA transfer each for K and for V.  Many short runs instead go
  // through a copy kernel that addresses the (pinned, mapped) host pool
  // directly, since each DMA transfer costs a fixed submission time.
  int runs = 0;
  for (int i = 0; i < num_pairs; ++runs) {
    int run = 1;
    while (i + run < num_pairs && block_pairs[2 * (i + run)] == block_pairs[2 * i] + run &&
           block_pairs[2 * (i + run) + 1] == block_pairs[2 * i + 1] + run)
      ++run;
    i += run;
  }
  void* hk_dev = nullptr;
  void* hv_dev = nullptr;
  if (runs > kSwapDmaMaxRuns && hipHostGetDevicePointer(&hk_dev, host_k, 0) == hipSuccess &&
      hipHostGetDevicePointer(&hv_dev, host_v, 0) == hipSuccess) {
    const void* s_k = out ? dev_k : hk_dev;
    const void* s_v = out ? dev_v : hv_dev;
    void* d_k = out ? hk_dev : dev_k;
    void* d_v = out ? hv_dev : dev_v;
    for (int i0 = 0; i0 < num_pairs; i0 += kSwapPairsPerLaunch) {
      const int n = std::min(kSwapPairsPerLaunch, num_pairs - i0);
      SwapPairs sp;
      memcpy(sp.p, block_pairs + 2 * i0, sizeof(int32_t) * 2 * n);
      const hipError_t e = launch_swap_kernel(s_k, s_v, d_k, d_v, p, sp, n, stream);
      if (e != hipSuccess) return hip_fail(e, "swap kernel launch");
    }
    return PA_OK;
  }
  (void)hipGetLastError();   // clear a failed pointer query (memory not mapped)
  for (int i = 0; i < num_pairs;) {
    const int32_t a = block_pairs[2 * i], b = block_pairs[2 * i + 1];
    int run = 1;
    while (i + run < num_pairs && block_pairs[2 * (i + run)] == a + run &&
           block_pairs[2 * (i + run) + 1] == b + run)
      ++run;
    hipError_t e = hipMemcpyAsync(dk + (size_t)b * blk, sk + (size_t)a * blk, run * blk, kind, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(dv + (size_t)b * blk, sv + (size_t)a * blk, run * blk, kind, stream);
    if (e != hipSuccess) return hip_fail(e, "swap copy");
    i += run;
  }
  return PA_OK;
}

static_assert(kMaxLayers == PA_MAX_LAYERS, "layer limit of the ABI and the kernel arguments");

pa_status pa_copy_blocks_layers(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                                const pa_cache_desc* c, const int32_t* block_pairs,
                                int32_t num_pairs, hipStream_t stream) {
  PoolArgs p;
  pa_status st = check_desc(c, &p);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_layers < 0) return fail(PA_ERR_INVALID_ARG, "negative count");
  if (num_layers > PA_MAX_LAYERS)
    return fail(PA_ERR_INVALID_ARG, "%d layers in one call, at most %d", num_layers, PA_MAX_LAYERS);
  if (num_pairs == 0 || num_layers == 0) return PA_OK;
  if (!k_caches || !v_caches || !block_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  LayerPools lp{};
  for (int l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return fail(PA_ERR_INVALID_ARG, "null pool of layer %d", l);
    if (!aligned16(k_caches[l]) || !aligned16(v_caches[l]))
      return fail(PA_ERR_INVALID_ARG, "pools of layer %d must be 16-byte aligned", l);
    lp.k[l] = k_caches[l];
    lp.v[l] = v_caches[l];
  }
  if (validate_mode()) {
    std::vector<int32_t> pr;
    if ((st = fetch(pr, block_pairs, 2 * (size_t)num_pairs, stream)) != PA_OK) return st;
    for (int i = 0; i < num_pairs; ++i)
      if (pr[2 * i] < 0 || pr[2 * i] >= p.num_blocks || pr[2 * i + 1] < 0 || pr[2 * i + 1] >= p.num_blocks)
        return fail(PA_ERR_BOUNDS, "block pair (%d, %d) out of range", pr[2 * i], pr[2 * i + 1]);
  }
  hipError_t e = launch_copy_blocks_layers(lp, num_layers, p, block_pairs, num_pairs, stream);
  return e == hipSuccess ? PA_OK : hip_fail(e, "copy_blocks_layers launch");
}

size_t pa_attention_workspace_size(const pa_cache_desc* c, int32_t num_q_heads, int32_t num_seqs,
                                   int32_t total_q, int32_t max_context_len,
                                   const pa_options* opt) {
  PoolArgs p;
  if (check_desc(c, &p) != PA_OK || num_q_heads <= 0 || num_seqs < 0 || total_q < 0 ||
      num_q_heads % p.num_kv_heads != 0)
    return 0;
  return make_layout(p, num_q_heads, num_seqs, total_q, max_context_len, opt).total;
}

pa_status pa_attention_plan(const pa_cache_desc* c, int32_t num_q_heads,
                            int32_t max_blocks_per_seq, int32_t num_seqs, int32_t total_q,
                            const int32_t* context_lens_host, const int32_t* query_start_loc_host,
                            size_t workspace_bytes, const pa_options* opt, pa_plan_info* info) {
  CallPlan cp;
  const pa_status st = plan_call(c, num_q_heads, max_blocks_per_seq, num_seqs, total_q,
                                 context_lens_host, query_start_loc_host, workspace_bytes, opt, &cp);
  if (info && (st == PA_OK || st == PA_ERR_WORKSPACE)) {
    info->row_items = cp.n_rows;
    info->tile_items = cp.n_tiles;
    info->combine_items = cp.n_combs;
    info->partial_slots = cp.n_partials;
    info->decode_split_tokens = cp.split;
    info->prefill_split_tokens = cp.psplit;
    info->prefill_tile_rows = cp.tile_rows;
    info->reserved = 0;
    info->workspace_bytes = cp.lay.total;
  }
  return st;
}

pa_status pa_attention_check(const void* workspace, hipStream_t stream) {
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "workspace is null");
  return read_status(workspace, stream);
}

pa_status pa_attention(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const pa_cache_desc* c, int32_t num_q_heads, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
                       const int32_t* context_lens_host, const int32_t* query_start_loc_host,
                       float scale, void* workspace, size_t workspace_bytes,
                       const pa_options* opt, hipStream_t stream) {
  return attention_impl(out, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), c,
                        num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, context_lens_host,
                        query_start_loc_host, scale, workspace, workspace_bytes, opt, nullptr,
                        stream, false);
}

pa_status pa_write_kv_attention(void* out, const void* q, const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                const pa_cache_desc* c, int32_t num_q_heads,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int32_t total_q,
                                const int32_t* context_lens_host,
                                const int32_t* query_start_loc_host, float scale,
                                void* workspace, size_t workspace_bytes, const pa_options* opt,
                                hipStream_t stream) {
  const FusedWrite fw{k_new, v_new, slot_mapping};
  return attention_impl(out, q, k_cache, v_cache, c, num_q_heads, block_tables,
                        max_blocks_per_seq, context_lens, query_start_loc, num_seqs, total_q,
                        context_lens_host, query_start_loc_host, scale, workspace,
                        workspace_bytes, opt, &fw, stream, false);
}

}  // extern "C"

namespace {

pa_status plan_call(const pa_cache_desc* c, int32_t num_q_heads, int32_t max_blocks_per_seq,
                    int32_t num_seqs, int32_t total_q, const int32_t* context_lens_host,
                    const int32_t* query_start_loc_host, size_t workspace_bytes,
                    const pa_options* opt, CallPlan* cp) {
  PoolArgs& p = cp->p;
  pa_status st = check_desc(c, &p);
  if (st != PA_OK) return st;
  if (num_q_heads <= 0 || num_q_heads % p.num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, p.num_kv_heads);
  const int group = num_q_heads / p.num_kv_heads;
  cp->group = group;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return fail(PA_ERR_UNSUPPORTED, "query heads per KV head %d not supported", group);
  if (num_seqs < 0 || total_q < 0) return fail(PA_ERR_INVALID_ARG, "negative num_seqs or total_q");
  if (opt && (opt->flags & ~(PA_FLAG_VECTOR_ALU | PA_FLAG_KV_UNSHARED | PA_FLAG_NO_PREFILL_SPLIT)))
    return fail(PA_ERR_INVALID_ARG, "unknown option flags");
  if (opt && (opt->decode_split_tokens < 0 || opt->prefill_split_tokens < 0))
    return fail(PA_ERR_INVALID_ARG, "negative split length");
  if (opt && opt->prefill_tile_rows != 0 && opt->prefill_tile_rows != kTileRows &&
      opt->prefill_tile_rows != kTileRowsWide)
    return fail(PA_ERR_INVALID_ARG, "prefill_tile_rows must be 0, %d or %d", kTileRows, kTileRowsWide);
  if (opt && (opt->timed_kernel < 0 || opt->timed_kernel > PA_TIME_COMBINE))
    return fail(PA_ERR_INVALID_ARG, "unknown timed_kernel %d", opt->timed_kernel);
  if (num_seqs > 0 && (!context_lens_host || !query_start_loc_host))
    return fail(PA_ERR_INVALID_ARG, "host mirrors are required");
  if (num_seqs > 0 && max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");

  // Host-side checks of the ragged batch.
  int max_len = 0;
  if (num_seqs > 0 && query_start_loc_host[0] != 0)
    return fail(PA_ERR_INVALID_ARG, "query_start_loc[0] must be 0");
  for (int s = 0; s < num_seqs; ++s) {
    const int n = query_start_loc_host[s + 1] - query_start_loc_host[s];
    const int L = context_lens_host[s];
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "query_start_loc decreases at sequence %d", s);
    if (L < 0) return fail(PA_ERR_INVALID_ARG, "negative context length at sequence %d", s);
    if (n > L) return fail(PA_ERR_INVALID_ARG, "sequence %d has %d new tokens but context %d", s, n, L);
    if ((int64_t)L > (int64_t)max_blocks_per_seq * p.block_size)
      return fail(PA_ERR_INVALID_ARG, "sequence %d context %d exceeds its block table", s, L);
    max_len = std::max(max_len, L);
  }
  cp->max_len = max_len;
  if ((num_seqs > 0 && query_start_loc_host[num_seqs] != total_q) || (num_seqs == 0 && total_q != 0))
    return fail(PA_ERR_INVALID_ARG, "query_start_loc[num_seqs] != total_q");

  // Work counts: the same functions the plan kernel runs on the device.
  const bool va = vector_all(p, opt);
  cp->va = va;
  int64_t total_keys = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = query_start_loc_host[s + 1] - query_start_loc_host[s];
    const int L = context_lens_host[s];
    const SeqWork w = seq_work(n, va ? 1 : 0, group, kTileRows);
    for (int i = w.row_first; i < w.row_first + w.rows; ++i) total_keys += L - n + i + 1;
  }
  const int split = choose_split(opt, total_keys, p.num_kv_heads, group);
  cp->split = split;
  // Wide (256-row) multi-token work items when there are enough of them.
  int tile_rows = kTileRows;
  if (opt && opt->prefill_tile_rows) {
    tile_rows = opt->prefill_tile_rows;
  } else if (!va) {
    int64_t wide = 0;
    for (int s = 0; s < num_seqs; ++s)
      wide += seq_work(query_start_loc_host[s + 1] - query_start_loc_host[s], 0, group,
                       kTileRowsWide).tiles;
    if (wide * p.num_kv_heads >= kWideTileMinGroups) tile_rows = kTileRowsWide;
  }
  cp->tile_rows = tile_rows;
  int psplit = va ? 0
               : auto_prefill_split(opt)
                   ? choose_prefill_split(context_lens_host, query_start_loc_host, num_seqs,
                                          group, tile_rows, p.num_kv_heads)
                   : prefill_split(opt);
  auto count = [&]() {
    cp->n_rows = cp->n_tiles = cp->n_combs = cp->n_partials = 0;
    for (int s = 0; s < num_seqs; ++s) {
      const int n = query_start_loc_host[s + 1] - query_start_loc_host[s];
      const int L = context_lens_host[s];
      const SeqWork w = seq_work(n, va ? 1 : 0, group, tile_rows);
      for (int i = w.row_first; i < w.row_first + w.rows; ++i) {
        const int ns = row_splits(L - n + i + 1, split);
        cp->n_rows += ns;
        if (ns > 1) {
          cp->n_combs += 1;
          cp->n_partials += ns;
        }
      }
      const TileWork tw = tile_work(n, L, group, tile_rows, w.tiles, psplit);
      cp->n_tiles += tw.items;
      cp->n_combs += tw.combs;
      cp->n_partials += tw.slots;
    }
    cp->lay = exact_layout(p, num_q_heads, cp->n_rows, cp->n_tiles, cp->n_combs, cp->n_partials);
    return cp->lay.total <= workspace_bytes;
  };
  bool fits = count();
  // An automatic multi-token split whose partial states do not fit the
  // workspace is lengthened until they do (pa_attention_workspace_size
  // reserves room for kMinAutoPrefillSplit-key splits).
  while (!fits && psplit > 0 && auto_prefill_split(opt)) {
    const int longer = (psplit + psplit / 4 + kPrefillSplitQuantum - 1) / kPrefillSplitQuantum *
                       kPrefillSplitQuantum;
    psplit = psplit >= max_len ? 0 : std::max(longer, psplit + kPrefillSplitQuantum);
    fits = count();
  }
  cp->psplit = psplit;
  if (cp->n_rows > 0x7fffffff || cp->n_tiles > 0x7fffffff || cp->n_partials > 0x7fffffff ||
      decode_mfma_groups(cp->n_rows, p.num_kv_heads, true) > 0x7fffffff)
    return fail(PA_ERR_UNSUPPORTED, "batch too large for one launch");
  cp->rows_on_mfma = !va && decode_mfma_supported(p, group);
  cp->rows_dealt = cp->rows_on_mfma && opt && (opt->flags & PA_FLAG_KV_UNSHARED);
  if (cp->n_rows > 0 && !cp->rows_on_mfma && p.block_size > 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d needs the fp16/bf16 MFMA kernels", p.block_size);
  if (!fits)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                cp->lay.total);
  return PA_OK;
}

// Status of the last call that used `workspace`, once `stream` is idle.
pa_status read_status(const void* workspace, hipStream_t stream) {
  PlanCounts pc{};
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(&pc, workspace, sizeof pc, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the plan status");
  if (pc.mismatch)
    return fail(PA_ERR_BOUNDS, "context_lens / query_start_loc on the device differ from the host mirrors");
  if (pc.dropped)
    return fail(PA_ERR_BOUNDS, "work items were skipped: an index left the batch or the workspace");
  return PA_OK;
}

pa_status attention_impl(void* out, const void* q, void* k_cache, void* v_cache,
                         const pa_cache_desc* c, int32_t num_q_heads, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
                         const int32_t* context_lens_host, const int32_t* query_start_loc_host,
                         float scale, void* workspace, size_t workspace_bytes,
                         const pa_options* opt, const FusedWrite* fw, hipStream_t stream,
                         bool static_scratch) {
  CallPlan cp;
  pa_status st = plan_call(c, num_q_heads, max_blocks_per_seq, num_seqs, total_q,
                           context_lens_host, query_start_loc_host,
                           workspace ? workspace_bytes : 0, opt, &cp);
  if (st == PA_ERR_WORKSPACE && total_q > 0 && static_scratch)
    return fail(PA_ERR_WORKSPACE,
                "the batch's plan needs %zu bytes of workspace; the static scratch holds %zu "
                "(give pa_write_kv_attention a workspace instead)", cp.lay.total, workspace_bytes);
  if (st != PA_OK && !(st == PA_ERR_WORKSPACE && total_q == 0)) return st;
  if (total_q == 0) return PA_OK;
  const PoolArgs& p = cp.p;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "q, out and the pools must be 16-byte aligned");
  if (fw && (!fw->k_new || !fw->v_new || !fw->slots))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (fw && (!aligned16(fw->k_new) || !aligned16(fw->v_new)))
    return fail(PA_ERR_INVALID_ARG, "K/V buffers must be 16-byte aligned");
  if (fw && write_geom(total_q, p).chunks > 0x7fffffff)
    return fail(PA_ERR_UNSUPPORTED, "too many new tokens for one write (at most 2^31 - 1 16-byte chunks)");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  if (validate_mode() && !static_scratch) {   // (these copies use host buffers)
    std::vector<int32_t> bt, lens, qsl;
    if ((st = fetch(bt, block_tables, (size_t)num_seqs * max_blocks_per_seq, stream)) != PA_OK) return st;
    if ((st = fetch(lens, context_lens, (size_t)num_seqs, stream)) != PA_OK) return st;
    if ((st = fetch(qsl, query_start_loc, (size_t)num_seqs + 1, stream)) != PA_OK) return st;
    for (int s = 0; s < num_seqs; ++s) {
      if (lens[s] != context_lens_host[s] || qsl[s + 1] != query_start_loc_host[s + 1])
        return fail(PA_ERR_BOUNDS, "device and host batch descriptions differ at sequence %d", s);
      const int nb = (lens[s] + p.block_size - 1) / p.block_size;
      for (int j = 0; j < nb; ++j) {
        const int32_t b = bt[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= p.num_blocks)
          return fail(PA_ERR_BOUNDS, "block_tables[%d][%d] = %d out of range", s, j, b);
      }
    }
    if (fw) {
      std::vector<int64_t> slots;   // the pa_write_kv rules for the fused write
      if ((st = check_slots(slots, fw->slots, total_q, p, stream)) != PA_OK) return st;
    }
  }

  // The plan, and with the fused write the new tokens' K/V stores too, in one
  // launch ahead of every kernel that reads the pools.
  const WorkspaceLayout& lay = cp.lay;
  int lpt_shift = 0;   // buckets of 2^lpt_shift keys, the longest context in the last
  while (((cp.max_len - 1) >> lpt_shift) >= kLptBuckets) ++lpt_shift;
  int row_shift = 0;   // (split - 1) >> row_shift < kRowBuckets
  while (((cp.split - 1) >> row_shift) >= kRowBuckets) ++row_shift;
  PlanParams pp{num_seqs, cp.split, cp.group, cp.va ? 1 : 0, cp.tile_rows, cp.psplit,
                cp.rows_dealt ? 1 : 0, row_shift, lay.cap_rows, lay.cap_tiles, lay.cap_combs, lay.cap_partials,
                cp.n_rows, cp.n_tiles, cp.n_combs, cp.n_partials, lpt_shift};
  hipError_t e =
      fw ? launch_plan_write(context_lens, query_start_loc, pp, workspace, lay, fw->k_new,
                             fw->v_new, fw->slots, total_q, k_cache, v_cache, p, stream)
         : launch_plan(context_lens, query_start_loc, pp, workspace, lay, stream);
  if (e != hipSuccess) return hip_fail(e, "plan launch");

  AttnArgs a{out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
             max_blocks_per_seq, num_q_heads, total_q, scale * kLog2e, workspace, cp.psplit,
             cp.rows_dealt ? 1 : 0};
  // Optional events around one kernel, recorded on `stream` (profiling hook).
  const int timed = opt ? opt->timed_kernel : 0;
  auto mark = [&](int which, hipEvent_t ev) {
    if (timed == which && ev) (void)hipEventRecord(ev, stream);
  };
  if (cp.n_tiles > 0) {
    mark(PA_TIME_TILE, opt ? opt->timing_start : nullptr);
    if ((e = launch_tile_attention(a, p, lay, (int)cp.n_tiles, cp.tile_rows, stream)) != hipSuccess)
      return hip_fail(e, "multi-token attention launch");
    mark(PA_TIME_TILE, opt ? opt->timing_end : nullptr);
  }
  if (cp.n_rows > 0) {
    mark(PA_TIME_ROWS, opt ? opt->timing_start : nullptr);
    e = cp.rows_on_mfma
            ? launch_decode_mfma(a, p, lay, (int)cp.n_rows, cp.split,
                                 opt && (opt->flags & PA_FLAG_KV_UNSHARED), stream)
            : launch_row_attention(a, p, lay, (int)cp.n_rows, cp.split, stream);
    if (e != hipSuccess) return hip_fail(e, "row attention launch");
    mark(PA_TIME_ROWS, opt ? opt->timing_end : nullptr);
  }
  if (cp.n_combs > 0) {
    mark(PA_TIME_COMBINE, opt ? opt->timing_start : nullptr);
    if ((e = launch_combine(a, p, lay, (int)cp.n_combs, stream)) != hipSuccess)
      return hip_fail(e, "split combine launch");
    mark(PA_TIME_COMBINE, opt ? opt->timing_end : nullptr);
  }
  if (validate_mode()) return read_status(workspace, stream);
  return PA_OK;
}

}  // namespace

// ---- the no-allocation entry point --------------------------------------
// A file-scope device array serves as the workspace of
// pa_write_kv_attention_static.  Host code never uses the array's name as an
// address: on each device, with that device current, its address is looked up
// once with hipGetSymbolAddress and kept.

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

pa_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_write_kv_attention_static(
    void* out, const void* q, const void* k_new, const void* v_new, const int64_t* slot_mapping,
    void* k_cache, void* v_cache, const pa_cache_desc* c, int32_t num_q_heads,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
    const int32_t* context_lens_host, const int32_t* query_start_loc_host, float scale,
    const pa_options* opt, hipStream_t stream) {
  static_assert(PA_STATIC_SCRATCH_BYTES == kScratchBytes, "scratch size of the ABI and the array");
  void* ws = nullptr;
  const pa_status st = scratch_of_current_device(&ws);
  if (st != PA_OK) return st;
  const FusedWrite fw{k_new, v_new, slot_mapping};
  return attention_impl(out, q, k_cache, v_cache, c, num_q_heads, block_tables,
                        max_blocks_per_seq, context_lens, query_start_loc, num_seqs, total_q,
                        context_lens_host, query_start_loc_host, scale, ws, kScratchBytes, opt, &fw,
                        stream, true);
}
