// Work planning on the device.
//
// Pensieve page (实验结果, multi-token kernel): computing the per-request
// auxiliary data outside the attention kernel is what let its kernel match an
// ideal contiguous one.  Here one small workgroup turns context_lens and
// query_start_loc into flat work lists inside the caller's workspace, so the
// attention kernels launch compact grids and read one record each; the host
// derives the same list sizes from the host mirrors to size those grids.

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ lens,
                                                           const int32_t* __restrict__ qsl,
                                                           PlanParams pp, uint8_t* ws,
                                                           WorkspaceLayout lay) {
  __shared__ int32_t scan[4][kPlanThreads];
  const int tid = threadIdx.x;
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
      const int ns = row_splits(L - n + i + 1, pp.split_tokens);
      c[0] += ns;
      if (ns > 1) {
        c[2] += 1;
        c[3] += ns;
      }
    }
    c[1] += w.tiles;
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
  int32_t base[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) base[k] = scan[k][tid] - c[k];

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
      for (int k = 0; k < ns; ++k) {
        if (base[0] < pp.cap_rows) rows[base[0]] = RowItem{s, i, k, pslot};
        base[0] += 1;
      }
    }
    // Last tile first: later rows see the longest causal key range.
    for (int t = w.tiles - 1; t >= 0; --t) {
      if (base[1] < pp.cap_tiles) tiles[base[1]] = TileItem{s, t};
      base[1] += 1;
    }
  }
  if (tid == kPlanThreads - 1) {
    PlanCounts* pc = reinterpret_cast<PlanCounts*>(ws + lay.counts);
    pc->rows = (int32_t)min<int64_t>(scan[0][tid], pp.cap_rows);
    pc->tiles = (int32_t)min<int64_t>(scan[1][tid], pp.cap_tiles);
    pc->combs = (int32_t)min<int64_t>(scan[2][tid], pp.cap_combs);
    pc->partials = (int32_t)min<int64_t>(scan[3][tid], pp.cap_partials);
  }
}

}  // namespace

hipError_t launch_plan(const int32_t* context_lens, const int32_t* qsl, const PlanParams& pp,
                       void* ws, const WorkspaceLayout& lay, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, context_lens, qsl, pp,
                     (uint8_t*)ws, lay);
  return hipGetLastError();
}

}  // namespace pa
