// Work planning on the device.
//
// Pensieve page (实验结果, multi-token kernel): computing the per-request
// auxiliary data outside the attention kernel is what let its kernel match an
// ideal contiguous one.  Here one small workgroup turns context_lens and
// query_start_loc into flat work lists inside the caller's workspace, so the
// attention kernels launch compact grids and read one record each; the host
// derives the same list sizes from the host mirrors to size those grids.
// With the fused write (pa_write_kv_attention), the same launch also carries
// the slot-mapping write: the plan reads no pool and the write no plan.

#include "pa_write.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kSplitList = 256;   // split multi-token sequences whose combine items are written by all threads

// Keys of split k of a tile whose causal range ends at kend (split length S;
// S = 0: the whole range).
__device__ __forceinline__ int item_keys(int kend, int k, int S) {
  return S > 0 ? min(kend, (k + 1) * S) - k * S : kend;
}
// Bucket of an item with `keys` keys: longer items get lower buckets.
__device__ __forceinline__ int lpt_bucket(int keys, int shift) {
  const int b = min(max(keys - 1, 0) >> shift, kLptBuckets - 1);
  return kLptBuckets - 1 - b;
}

// Bucket of a row item with `keys` (1..split) of a `split`-key split: full
// splits in bucket 0, shorter ones later (longest first); `shift` makes
// (split - 1) >> shift < kRowBuckets.
__device__ __forceinline__ int row_bucket(int keys, int split, int shift) {
  return (split - keys) >> shift;
}

struct SplitSeq {
  int32_t seq, comb_base, pbase, i0, n, L, q0, ns;
};

__device__ __forceinline__ void plan_block(const int32_t* __restrict__ lens,
                                           const int32_t* __restrict__ qsl, const PlanParams& pp,
                                           uint8_t* ws, const WorkspaceLayout& lay) {
  __shared__ int32_t scan[4][kPlanThreads];
  __shared__ SplitSeq split_list[kSplitList];
  __shared__ int32_t split_count;
  __shared__ int32_t lpt_start[kLptBuckets];   // first list position of each bucket
  __shared__ int32_t lpt_fill[kLptBuckets];    // items counted / placed per bucket
  __shared__ int32_t row_start[kRowBuckets];   // the same for row items listed longest first
  __shared__ int32_t row_fill[kRowBuckets];
  const int tid = threadIdx.x;
  if (tid == 0) split_count = 0;
  for (int b = tid; b < kLptBuckets; b += kPlanThreads) lpt_fill[b] = 0;
  for (int b = tid; b < kRowBuckets; b += kPlanThreads) row_fill[b] = 0;
  __syncthreads();   // (row_fill is counted in the first pass)
  const int S = pp.num_seqs;
  const int per = (S + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(S, tid * per);
  const int s1 = min(S, s0 + per);

  int32_t c[4] = {0, 0, 0, 0};  // rows, tiles, combs, partials
  for (int s = s0; s < s1; ++s) {
    const int n = qsl[s + 1] - qsl[s];
    const int L = lens[s];
    const SeqWork w = seq_work(n, pp.vector_all, pp.group, pp.tile_rows);
    for (int i = w.row_first; i < w.row_first + w.rows; ++i) {
      const int keys = L - n + i + 1;
      const int ns = row_splits(keys, pp.split_tokens);
      c[0] += ns;
      if (ns > 1) {
        c[2] += 1;
        c[3] += ns;
      }
      if (pp.rows_dealt) {
        if (ns > 1) atomicAdd(&row_fill[0], ns - 1);
        atomicAdd(&row_fill[row_bucket(keys - (ns - 1) * pp.split_tokens, pp.split_tokens, pp.row_shift)], 1);
      }
    }
    const TileWork tw = tile_work(n, L, pp.group, pp.tile_rows, w.tiles, pp.prefill_split);
    c[1] += tw.items;
    c[2] += tw.combs;
    c[3] += tw.slots;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) scan[k][tid] = c[k];
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    int32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = tid >= off ? scan[k][tid - off] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) scan[k][tid] += v[k];
    __syncthreads();
  }
  if (pp.rows_dealt) {
    // Bucket starts of the row items: an exclusive scan by the first wave, one
    // bucket a lane (the scan above ordered the counts).
    static_assert(kRowBuckets == 64, "one wave scans the row buckets");
    if (tid < kRowBuckets) {
      const int cnt = row_fill[tid];
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (tid >= off) incl += v;
      }
      row_start[tid] = incl - cnt;
      row_fill[tid] = 0;
    }
    __syncthreads();
  }
  int32_t base[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) base[k] = scan[k][tid] - c[k];
  const int32_t part0 = base[3];   // this thread's first partial slot
  int32_t total[4];                // the batch's counts (scan[0] is reused below)
#pragma unroll
  for (int k = 0; k < 4; ++k) total[k] = scan[k][kPlanThreads - 1];

  RowItem* rows = reinterpret_cast<RowItem*>(ws + lay.rows);
  TileItem* tiles = reinterpret_cast<TileItem*>(ws + lay.tiles);
  CombItem* combs = reinterpret_cast<CombItem*>(ws + lay.combs);
  for (int s = s0; s < s1; ++s) {
    const int n = qsl[s + 1] - qsl[s];
    const int L = lens[s];
    const SeqWork w = seq_work(n, pp.vector_all, pp.group, pp.tile_rows);
    for (int i = w.row_first; i < w.row_first + w.rows; ++i) {
      const int ns = row_splits(L - n + i + 1, pp.split_tokens);
      int32_t pslot = -1;
      if (ns > 1) {
        pslot = base[3];
        if (base[2] < pp.cap_combs) combs[base[2]] = CombItem{qsl[s] + i, pslot, ns, s};
        base[2] += 1;
        base[3] += ns;
      }
      if (pp.rows_dealt) {
        // Longest first: the full splits as one run of bucket 0, the last
        // split in its length's bucket.
        const int keys = L - n + i + 1;
        if (ns > 1) {
          const int at = row_start[0] + atomicAdd(&row_fill[0], ns - 1);
          for (int k = 0; k < ns - 1; ++k)
            if (at + k < pp.cap_rows) rows[at + k] = RowItem{s, i, k, pslot};
        }
        const int b = row_bucket(keys - (ns - 1) * pp.split_tokens, pp.split_tokens, pp.row_shift);
        const int at = row_start[b] + atomicAdd(&row_fill[b], 1);
        if (at < pp.cap_rows) rows[at] = RowItem{s, i, ns - 1, pslot};
      } else {
        for (int k = 0; k < ns; ++k) {
          if (base[0] < pp.cap_rows) rows[base[0]] = RowItem{s, i, k, pslot};
          base[0] += 1;
        }
      }
    }
    if (w.tiles == 0) continue;
    // A split multi-token sequence: partial slots token-major, a combine
    // item for every token that sees more than one split.
    const TileWork tw = tile_work(n, L, pp.group, pp.tile_rows, w.tiles, pp.prefill_split);
    const int ns = key_splits(L, pp.prefill_split);
    int32_t pbase = -1;
    if (ns > 1) {
      pbase = base[3];
      // The combine items of the sequence's tokens: listed for all threads
      // to write below, or written here if the list is full.
      const int i0 = n - tw.combs;
      const int at = atomicAdd(&split_count, 1);
      if (at < kSplitList) {
        split_list[at] = SplitSeq{s, base[2], pbase, i0, n, L, qsl[s], ns};
      } else {
        for (int i = i0; i < n; ++i)
          if (base[2] + i - i0 < pp.cap_combs)
            combs[base[2] + i - i0] = CombItem{qsl[s] + i, pbase + i * ns, key_splits(L - n + i + 1, pp.prefill_split), s};
      }
      base[2] += tw.combs;
      base[3] += tw.slots;
    }
    // Items are listed longest first.  A sequence whose keys are not split
    // goes in as one contiguous run (its tiles re-read the same K/V, which
    // then meet in one L2), placed by its longest item (the last tile); the
    // items of a split sequence go in one by one (those of one key split read
    // the same keys and have the same length, so they stay together).
    if (ns > 1) {
      // Every split of a tile but its last holds exactly prefill_split keys.
      for (int t = 0; t < w.tiles; ++t) {
        const int kend = tile_key_end(n, L, pp.group, pp.tile_rows, t);
        const int nk = key_splits(kend, pp.prefill_split);
        if (nk > 1) atomicAdd(&lpt_fill[lpt_bucket(pp.prefill_split, pp.lpt_shift)], nk - 1);
        atomicAdd(&lpt_fill[lpt_bucket(item_keys(kend, nk - 1, pp.prefill_split), pp.lpt_shift)], 1);
      }
    } else {
      atomicAdd(&lpt_fill[lpt_bucket(tile_key_end(n, L, pp.group, pp.tile_rows, w.tiles - 1), pp.lpt_shift)],
                w.tiles);
    }
  }
  __syncthreads();
  // Bucket starts: an exclusive scan of the histogram (two buckets a thread).
  // (A batch without multi-token items skips this and the placement.)
  static_assert(kLptBuckets == 2 * kPlanThreads, "two buckets per planner thread");
  if (total[1] > 0) {
    const int b0 = lpt_fill[2 * tid], b1 = lpt_fill[2 * tid + 1];
    __syncthreads();
    scan[0][tid] = b0 + b1;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int v = tid >= off ? scan[0][tid - off] : 0;
      __syncthreads();
      scan[0][tid] += v;
      __syncthreads();
    }
    const int ex = scan[0][tid] - b0 - b1;
    lpt_start[2 * tid] = ex;
    lpt_start[2 * tid + 1] = ex + b0;
    lpt_fill[2 * tid] = 0;
    lpt_fill[2 * tid + 1] = 0;
    __syncthreads();
  }
  // Place every item (or run) at its bucket's next free position.  The
  // order inside a bucket is arbitrary: each item computes outputs of its own.
  int32_t part = part0;   // partial slots handed out as in the first pass
  for (int s = s0; s < s1 && total[1] > 0; ++s) {
    const int n = qsl[s + 1] - qsl[s];
    const int L = lens[s];
    const SeqWork w = seq_work(n, pp.vector_all, pp.group, pp.tile_rows);
    for (int i = w.row_first; i < w.row_first + w.rows; ++i) {
      const int nr = row_splits(L - n + i + 1, pp.split_tokens);
      if (nr > 1) part += nr;
    }
    if (w.tiles == 0) continue;
    const int ns = key_splits(L, pp.prefill_split);
    const int32_t pbase = ns > 1 ? part : -1;
    if (ns > 1) {
      part += tile_work(n, L, pp.group, pp.tile_rows, w.tiles, pp.prefill_split).slots;
      for (int t = 0; t < w.tiles; ++t) {
        const int kend = tile_key_end(n, L, pp.group, pp.tile_rows, t);
        const int nk = key_splits(kend, pp.prefill_split);
        // The full splits as one run of a bucket, then the last split.
        if (nk > 1) {
          const int b = lpt_bucket(pp.prefill_split, pp.lpt_shift);
          const int at = lpt_start[b] + atomicAdd(&lpt_fill[b], nk - 1);
          for (int k = 0; k < nk - 1; ++k)
            if (at + k < pp.cap_tiles) tiles[at + k] = TileItem{s, t, k, pbase};
        }
        const int b = lpt_bucket(item_keys(kend, nk - 1, pp.prefill_split), pp.lpt_shift);
        const int at = lpt_start[b] + atomicAdd(&lpt_fill[b], 1);
        if (at < pp.cap_tiles) tiles[at] = TileItem{s, t, nk - 1, pbase};
      }
    } else {
      // The run, last tile (the most keys) first.
      const int b = lpt_bucket(tile_key_end(n, L, pp.group, pp.tile_rows, w.tiles - 1), pp.lpt_shift);
      int at = lpt_start[b] + atomicAdd(&lpt_fill[b], w.tiles);
      for (int t = w.tiles - 1; t >= 0; --t, ++at)
        if (at < pp.cap_tiles) tiles[at] = TileItem{s, t, 0, pbase};
    }
  }
  const int nl = min(split_count, kSplitList);
  for (int e = 0; e < nl; ++e) {
    const SplitSeq q = split_list[e];
    for (int i = q.i0 + tid; i < q.n; i += kPlanThreads) {
      const int64_t at = (int64_t)q.comb_base + i - q.i0;
      if (at < pp.cap_combs)
        combs[at] = CombItem{q.q0 + i, q.pbase + i * q.ns, key_splits(q.L - q.n + i + 1, pp.prefill_split), q.seq};
    }
  }
  if (tid == kPlanThreads - 1) {
    PlanCounts* pc = reinterpret_cast<PlanCounts*>(ws + lay.counts);
    pc->rows = (int32_t)min<int64_t>(total[0], pp.cap_rows);
    pc->tiles = (int32_t)min<int64_t>(total[1], pp.cap_tiles);
    pc->combs = (int32_t)min<int64_t>(total[2], pp.cap_combs);
    pc->partials = (int32_t)min<int64_t>(total[3], pp.cap_partials);
    pc->mismatch = total[0] != pp.want_rows || total[1] != pp.want_tiles ||
                   total[2] != pp.want_combs || total[3] != pp.want_partials;
    pc->dropped = 0;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ lens,
                                                           const int32_t* __restrict__ qsl,
                                                           PlanParams pp, uint8_t* ws,
                                                           WorkspaceLayout lay) {
  plan_block(lens, qsl, pp, ws, lay);
}

// Workgroup 0 plans; the others write the new tokens' K/V.
struct WriteArgs {
  const uint4* k_new;
  const uint4* v_new;
  const int64_t* slots;
  int64_t num_tokens, chunks, total_slots;
  int k_blocks, cpr, H, D, bs;
  uint8_t* k_cache;
  void* v_cache;
};
template <int EB>
__global__ __launch_bounds__(kPlanThreads) void plan_write_kernel(const int32_t* __restrict__ lens,
                                                                 const int32_t* __restrict__ qsl,
                                                                 PlanParams pp, uint8_t* ws,
                                                                 WorkspaceLayout lay, WriteArgs w) {
  static_assert(kPlanThreads == 256, "the write runs 256-thread workgroups");
  if (blockIdx.x == 0) {
    plan_block(lens, qsl, pp, ws, lay);
    return;
  }
  write_kv_block<EB>((int)blockIdx.x - 1, w.k_new, w.v_new, w.slots, w.num_tokens, w.chunks,
                     w.k_blocks, w.cpr, w.H, w.D, w.bs, w.total_slots, w.k_cache, w.v_cache);
}

}  // namespace

hipError_t launch_plan_write(const int32_t* context_lens, const int32_t* qsl, const PlanParams& pp,
                             void* ws, const WorkspaceLayout& lay, const void* k_new,
                             const void* v_new, const int64_t* slots, int num_tokens,
                             void* k_cache, void* v_cache, const PoolArgs& p, hipStream_t s) {
  const WriteGeom g = write_geom(num_tokens, p);
  if (g.chunks > 0x7fffffff) return hipErrorInvalidValue;   // 32-bit index arithmetic
  const WriteArgs w{(const uint4*)k_new, (const uint4*)v_new, slots, (int64_t)num_tokens, g.chunks,
                    g.total_slots, (int)g.blocks, g.cpr, p.num_kv_heads, p.head_dim, p.block_size,
                    (uint8_t*)k_cache, v_cache};
  const dim3 grid((unsigned)(1 + 2 * g.blocks));
  if (g.eb == 4)
    hipLaunchKernelGGL(plan_write_kernel<4>, grid, dim3(kPlanThreads), 0, s, context_lens, qsl, pp,
                       (uint8_t*)ws, lay, w);
  else
    hipLaunchKernelGGL(plan_write_kernel<2>, grid, dim3(kPlanThreads), 0, s, context_lens, qsl, pp,
                       (uint8_t*)ws, lay, w);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* context_lens, const int32_t* qsl, const PlanParams& pp,
                       void* ws, const WorkspaceLayout& lay, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, context_lens, qsl, pp,
                     (uint8_t*)ws, lay);
  return hipGetLastError();
}

}  // namespace pa
