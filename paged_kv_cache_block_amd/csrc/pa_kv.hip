// Bit-exact KV movers: the slot-mapping scatter and the batched block copy.
//
// vLLM-SOSP23 page (Kernel 层实现): the reshape and block write of new K/V is
// one fused kernel, and block copies for copy-on-write are batched into one
// launch.  Pensieve page (统一Prefill和Generation阶段的执行过程): new K/V
// go into their allocated slots before attention runs.
//
// K keeps the token-major row of the input, so a (token, head) row lands as
// D * elt contiguous bytes, moved in 16-byte chunks.  V is head-dim major
// inside a block, so a (token, head) row becomes D elements spaced block_size
// apart; the write kernel orders its V threads token-fastest so that the
// elements of consecutive slots are stored side by side.  Block copies move
// 16-byte chunks.

#include "pa_write.h"

namespace pa {
namespace {

template <int EB>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slots, int64_t num_tokens, int64_t chunks, int k_blocks,
    int chunks_per_row, int H, int D, int bs, int64_t total_slots, uint8_t* __restrict__ k_cache,
    void* __restrict__ v_cache) {
  write_kv_block<EB>((int)blockIdx.x, k_new, v_new, slots, num_tokens, chunks, k_blocks,
                     chunks_per_row, H, D, bs, total_slots, k_cache, v_cache);
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t chunks_per_block,
                                                          int num_blocks) {
  const int p = blockIdx.x;
  const int src = pairs[2 * p];
  const int dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t s0 = (int64_t)src * chunks_per_block;
  const int64_t d0 = (int64_t)dst * chunks_per_block;
  for (int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x; c < chunks_per_block;
       c += (int64_t)gridDim.y * 256) {
    const uint4 a = k_cache[s0 + c];
    const uint4 b = v_cache[s0 + c];
    k_cache[d0 + c] = a;
    v_cache[d0 + c] = b;
  }
}

// The copies of pa_copy_blocks on every layer's pools: grid.z is the layer,
// whose pool pointers travel in the kernel arguments.
__global__ __launch_bounds__(256) void copy_blocks_layers_kernel(LayerPools lp,
                                                                 const int32_t* __restrict__ pairs,
                                                                 int64_t chunks_per_block,
                                                                 int num_blocks) {
  uint4* k_cache = reinterpret_cast<uint4*>(lp.k[blockIdx.z]);
  uint4* v_cache = reinterpret_cast<uint4*>(lp.v[blockIdx.z]);
  const int p = blockIdx.x;
  const int src = pairs[2 * p];
  const int dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t s0 = (int64_t)src * chunks_per_block;
  const int64_t d0 = (int64_t)dst * chunks_per_block;
  for (int64_t c = (int64_t)blockIdx.y * 256 + threadIdx.x; c < chunks_per_block;
       c += (int64_t)gridDim.y * 256) {
    const uint4 a = k_cache[s0 + c];
    const uint4 b = v_cache[s0 + c];
    k_cache[d0 + c] = a;
    v_cache[d0 + c] = b;
  }
}

// Whole-block copies between two pools, one of them host memory mapped into
// the device's address space.  Each thread moves four 16-byte chunks of K and
// four of V, loads first, so that eight transfers over the host link are in
// flight per thread.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const uint4* __restrict__ src_k,
                                                          const uint4* __restrict__ src_v,
                                                          uint4* __restrict__ dst_k,
                                                          uint4* __restrict__ dst_v, SwapPairs pairs,
                                                          int64_t chunks_per_block) {
  const int i = blockIdx.x;
  const int64_t s0 = (int64_t)pairs.p[2 * i] * chunks_per_block;
  const int64_t d0 = (int64_t)pairs.p[2 * i + 1] * chunks_per_block;
  const int64_t c0 = (int64_t)blockIdx.y * 1024 + threadIdx.x;
  if (c0 + 768 < chunks_per_block) {
    uint4 k[4], v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      k[u] = src_k[s0 + c0 + 256 * u];
      v[u] = src_v[s0 + c0 + 256 * u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dst_k[d0 + c0 + 256 * u] = k[u];
      dst_v[d0 + c0 + 256 * u] = v[u];
    }
    return;
  }
  for (int64_t c = c0; c < chunks_per_block; c += 256) {   // a block's last partial slice
    dst_k[d0 + c] = src_k[s0 + c];
    dst_v[d0 + c] = src_v[s0 + c];
  }
}

}  // namespace

hipError_t launch_swap_kernel(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const PoolArgs& p, const SwapPairs& pairs, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int eb = p.dtype == DT_F32 ? 4 : 2;
  const int64_t cpb = (int64_t)p.num_kv_heads * p.block_size * p.head_dim * eb / 16;
  const dim3 grid(n, (unsigned)((cpb + 1023) / 1024));
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(256), 0, s, (const uint4*)src_k,
                     (const uint4*)src_v, (uint4*)dst_k, (uint4*)dst_v, pairs, cpb);
  return hipGetLastError();
}

hipError_t launch_copy_blocks_layers(const LayerPools& lp, int num_layers, const PoolArgs& p,
                                     const int32_t* pairs, int num_pairs, hipStream_t s) {
  if (num_pairs == 0 || num_layers == 0) return hipSuccess;
  const int eb = p.dtype == DT_F32 ? 4 : 2;
  const int64_t cpb = (int64_t)p.num_kv_heads * p.block_size * p.head_dim * eb / 16;
  int gy = (int)((cpb + 255) / 256);
  if (gy > 64) gy = 64;
  hipLaunchKernelGGL(copy_blocks_layers_kernel, dim3(num_pairs, gy, num_layers), dim3(256), 0, s,
                     lp, pairs, cpb, p.num_blocks);
  return hipGetLastError();
}

hipError_t launch_write_kv(const void* k_new, const void* v_new, const int64_t* slots,
                           int num_tokens, void* k_cache, void* v_cache, const PoolArgs& p,
                           hipStream_t s) {
  const WriteGeom wg = write_geom(num_tokens, p);
  const int eb = wg.eb, cpr = wg.cpr;
  const int64_t chunks = wg.chunks, blocks = wg.blocks, total_slots = wg.total_slots;
  if (chunks == 0) return hipSuccess;
  if (chunks > 0x7fffffff) return hipErrorInvalidValue;   // 32-bit index arithmetic
  const dim3 grid((unsigned)(2 * blocks));
  if (eb == 4)
    hipLaunchKernelGGL(write_kv_kernel<4>, grid, dim3(256), 0, s, (const uint4*)k_new,
                       (const uint4*)v_new, slots, (int64_t)num_tokens, chunks, (int)blocks, cpr,
                       p.num_kv_heads, p.head_dim, p.block_size, total_slots, (uint8_t*)k_cache, v_cache);
  else
    hipLaunchKernelGGL(write_kv_kernel<2>, grid, dim3(256), 0, s, (const uint4*)k_new,
                       (const uint4*)v_new, slots, (int64_t)num_tokens, chunks, (int)blocks, cpr,
                       p.num_kv_heads, p.head_dim, p.block_size, total_slots, (uint8_t*)k_cache, v_cache);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const PoolArgs& p,
                              const int32_t* pairs, int num_pairs, hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const int eb = p.dtype == DT_F32 ? 4 : 2;
  const int64_t cpb = (int64_t)p.num_kv_heads * p.block_size * p.head_dim * eb / 16;
  int gy = (int)((cpb + 255) / 256);
  if (gy > 64) gy = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, gy), dim3(256), 0, s,
                     (uint4*)k_cache, (uint4*)v_cache, pairs, cpb, p.num_blocks);
  return hipGetLastError();
}

}  // namespace pa
