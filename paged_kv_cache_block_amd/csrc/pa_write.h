// The slot-mapping write of new K/V, as a per-workgroup device function:
// the write kernel runs it on every workgroup, and the combined plan + write
// launch on all but its first.
#pragma once

#include "pa_internal.h"

namespace pa {

// One launch, two kinds of workgroup, each with the thread order that makes
// its stores contiguous.  The first k_blocks workgroups copy K: one thread per
// 16-byte chunk of a (token, head) row, which stays a contiguous row of the
// token-major block.  The rest write V with the token index fastest: thread
// (head, chunk, token) loads the token's 16-byte chunk of head-dim elements
// and stores each element into its head-dim row of the head-dim-major block,
// so that, for consecutive slots, the lanes of a wave fill consecutive
// positions of the same row.
template <int EB>
__device__ __forceinline__ void write_kv_block(
    int block, const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slots, int64_t num_tokens, int64_t chunks, int k_blocks,
    int chunks_per_row, int H, int D, int bs, int64_t total_slots, uint8_t* __restrict__ k_cache,
    void* __restrict__ v_cache) {
  using E = typename Elt<EB == 4 ? DT_F32 : DT_F16>::store_t;
  constexpr int VEC = 16 / EB;
  const bool is_k = block < k_blocks;
  const int64_t gid = (int64_t)(is_k ? block : block - k_blocks) * 256 + threadIdx.x;
  if (gid >= chunks) return;
  if (is_k) {
    const int chunk = (int)(gid % chunks_per_row);
    const int64_t th = gid / chunks_per_row;
    const int h = (int)(th % H);
    const int64_t t = th / H;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= total_slots) return;
    const int64_t blk = slot / bs;
    const int off = (int)(slot - blk * bs);
    uint8_t* kdst = k_cache + (((blk * H + h) * bs + off) * (int64_t)D) * EB + (int64_t)chunk * 16;
    *reinterpret_cast<uint4*>(kdst) = k_new[gid];
    return;
  }
  const int64_t t = gid % num_tokens;
  const int64_t hc = gid / num_tokens;
  const int chunk = (int)(hc % chunks_per_row);
  const int h = (int)(hc / chunks_per_row);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= total_slots) return;
  const int64_t blk = slot / bs;
  const int off = (int)(slot - blk * bs);
  const uint4 vv = v_new[(t * H + h) * chunks_per_row + chunk];
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
  E* vdst = reinterpret_cast<E*>(v_cache) + ((blk * H + h) * (int64_t)D + (int64_t)chunk * VEC) * bs + off;
  if constexpr (EB == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vdst[(int64_t)e * bs] = w[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vdst[(int64_t)(2 * e) * bs] = (E)(w[e] & 0xffffu);
      vdst[(int64_t)(2 * e + 1) * bs] = (E)(w[e] >> 16);
    }
  }
}

// Write launch geometry: `blocks` workgroups of 256 threads for K, as many
// for V; 0 when there is nothing to write.
struct WriteGeom {
  int64_t chunks, blocks, total_slots;
  int cpr, eb;
};
inline WriteGeom write_geom(int num_tokens, const PoolArgs& p) {
  WriteGeom w;
  w.eb = p.dtype == DT_F32 ? 4 : 2;
  w.cpr = p.head_dim * w.eb / 16;
  w.chunks = (int64_t)num_tokens * p.num_kv_heads * w.cpr;
  w.blocks = (w.chunks + 255) / 256;
  w.total_slots = (int64_t)p.num_blocks * p.block_size;
  return w;
}

}  // namespace pa
