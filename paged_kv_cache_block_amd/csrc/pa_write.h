// The slot-mapping write of new K/V, as a per-workgroup device function:
// the write kernel runs it on every workgroup, and the combined plan + write
// launch on all but its first.
#pragma once

#include "pa_internal.h"

namespace pa {

// New tokens are taken in groups of kWriteGroup consecutive tokens (a block
// of slots, when a sequence's new tokens fill one), so that each workgroup
// writes one head's rows of consecutive slots: contiguous runs of the
// destination block rather than 256-byte pieces scattered over the pool.
constexpr int kWriteGroup = 32;

// Pins a loaded value ahead of the code that follows, so that the compiler
// does not sink its load past the slot test (one memory wait per thread, not
// two).
__device__ __forceinline__ void keep_loaded(uint4& x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}

// One launch, two kinds of workgroup, each with the thread order that makes
// its stores contiguous.  The first k_blocks workgroups copy K: thread
// (group, head, token, chunk), chunk fastest, moves one 16-byte chunk of a
// (token, head) row; a workgroup fills consecutive rows of one head's
// token-major block.  The rest write V: thread (group, head, chunk, token),
// token fastest, loads the token's 16-byte chunk of head-dim elements and
// stores each element into its row of the head-dim-major block, so the lanes
// of a wave fill consecutive positions of the same rows.  Index arithmetic is
// 32-bit (the launchers reject more than 2^31 - 1 thread slots);
// chunks_per_row and bs are powers of two, so only the division by the head
// count remains.
template <int EB>
__device__ __forceinline__ void write_kv_block(
    int block, const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slots, int64_t num_tokens, int64_t chunks, int k_blocks,
    int chunks_per_row, int H, int D, int bs, int64_t total_slots, uint8_t* __restrict__ k_cache,
    void* __restrict__ v_cache) {
  using E = typename Elt<EB == 4 ? DT_F32 : DT_F16>::store_t;
  constexpr int VEC = 16 / EB;
  constexpr int LG = 5;   // log2(kWriteGroup)
  static_assert(1 << LG == kWriteGroup, "write group");
  const bool is_k = block < k_blocks;
  const uint32_t gid = (uint32_t)(is_k ? block : block - k_blocks) * 256u + threadIdx.x;
  if (gid >= (uint64_t)chunks) return;
  const int lcpr = __builtin_ctz((unsigned)chunks_per_row);
  const int lbs = __builtin_ctz((unsigned)bs);
  uint32_t chunk, lt, rest;
  if (is_k) {
    chunk = gid & (uint32_t)(chunks_per_row - 1);
    lt = (gid >> lcpr) & (kWriteGroup - 1);
    rest = gid >> (lcpr + LG);
  } else {
    lt = gid & (kWriteGroup - 1);
    chunk = (gid >> LG) & (uint32_t)(chunks_per_row - 1);
    rest = gid >> (lcpr + LG);
  }
  const uint32_t tg = rest / (uint32_t)H;
  const uint32_t h = rest - tg * (uint32_t)H;
  const uint32_t t = tg * kWriteGroup + lt;
  if (t >= (uint64_t)num_tokens) return;
  const uint32_t src = (t * (uint32_t)H + h) * (uint32_t)chunks_per_row + chunk;
  uint4 x = is_k ? k_new[src] : v_new[src];
  const int64_t slot = slots[t];
  keep_loaded(x);
  if (slot < 0 || slot >= total_slots) return;
  const int64_t blk = slot >> lbs;
  const int off = (int)(slot & (bs - 1));
  if (is_k) {
    uint8_t* kdst = k_cache + (((blk * H + h) * bs + off) * (int64_t)D) * EB + (int64_t)chunk * 16;
    *reinterpret_cast<uint4*>(kdst) = x;
    return;
  }
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
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
// for V (thread slots for whole token groups; those past the last token
// idle); 0 when there is nothing to write.
struct WriteGeom {
  int64_t chunks, blocks, total_slots;
  int cpr, eb;
};
inline WriteGeom write_geom(int num_tokens, const PoolArgs& p) {
  WriteGeom w;
  w.eb = p.dtype == DT_F32 ? 4 : 2;
  w.cpr = p.head_dim * w.eb / 16;
  const int64_t groups = ((int64_t)num_tokens + kWriteGroup - 1) / kWriteGroup;
  w.chunks = groups * kWriteGroup * p.num_kv_heads * w.cpr;
  w.blocks = (w.chunks + 255) / 256;
  w.total_slots = (int64_t)p.num_blocks * p.block_size;
  return w;
}

}  // namespace pa
