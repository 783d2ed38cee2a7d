// Vector-ALU paged attention for single query rows, and the split combine.
//
// vLLM-SOSP23 page (核心方法, Kernel 层实现) and Pensieve page (多Token注意力
// 内核运算原理): a decode token's attention is two matrix-vector products
// over its paged context, read block by block through the block table.
// Pensieve page (LLM与注意力机制): softmax(Q K^T * scale) V.
//
// One wavefront owns one (row, KV head, key split) and up to 8 query heads of
// that KV head's group, so each K/V block is read once for all of them.
// Keys are processed 64 at a time:
//   QK:  D / VEC lanes share one key row (16-byte loads along head_dim) and
//        reduce their partial dot products across the lane group;
//   softmax: lane j owns key j of the chunk; running max and sum per head
//        (online softmax, base 2 with the scale pre-multiplied by log2 e);
//   PV:  V is head-dim major inside a block, so a lane loads a run of
//        consecutive keys of one head-dim row and weights them by the chunk's
//        probabilities read back from LDS.
// A row with several splits writes (max, sum, unnormalised accumulator) to
// the workspace; combine_kernel merges them:
//   m = max_k m_k,  l = sum_k l_k 2^(m_k - m),  o = sum_k 2^(m_k - m) acc_k / l.

#include "pa_internal.h"

namespace pa {
namespace {

template <int DT, int D, int BS, int GH>
__global__ __launch_bounds__(64) void row_attn_kernel(AttnArgs a, PoolArgs p, WorkspaceLayout lay,
                                                     int split_tokens) {
  constexpr int EB = Elt<DT>::bytes;
  constexpr int VEC = 16 / EB;            // elements per 16-byte K load
  constexpr int LPR = D / VEC;            // lanes per key row
  constexpr int TPL = 64 / LPR;           // keys per K load
  constexpr int NK = LPR;                 // K loads per 64-key chunk
  constexpr int VV = VEC < BS ? VEC : BS; // elements per V load
  constexpr int RPV = BS / VV;            // lanes spanning one V row of a block
  constexpr int NVB = D * BS / VV / 64;   // V loads per block per lane
  constexpr int BPC = 64 / BS;            // blocks per chunk
  static_assert(NVB >= 1 && 64 % BS == 0, "shape");

  __shared__ float sc[GH][64];
  __shared__ float pl[GH][64];

  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const PlanCounts* pc = reinterpret_cast<const PlanCounts*>(ws + lay.counts);
  const int item = blockIdx.x;
  if (item >= pc->rows) return;
  const RowItem it = reinterpret_cast<const RowItem*>(ws + lay.rows)[item];
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int Hq = a.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int head0 = g * G + blockIdx.z * GH;

  const int s = it.seq;
  const int q0 = a.qsl[s];
  const int n = a.qsl[s + 1] - q0;
  const int L = a.context_lens[s];
  const int row = q0 + it.i;
  const int limit = L - n + it.i;                 // last visible key
  const int t0 = it.split * split_tokens;
  const int t1 = min(limit + 1, t0 + split_tokens);
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const int nb_max = p.num_blocks - 1;
  const int tb_max = a.max_blocks - 1;
  if (row >= a.total_q) {          // device batch disagrees with the host mirrors
    mark_dropped(a.ws, lay);
    return;
  }

  // Query slice of this lane, pre-scaled.
  float qv[GH][VEC];
  const int d0 = (lane % LPR) * VEC;
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) +
                        (((int64_t)row * Hq + head0 + h) * D + d0) * EB;
    const uint4 raw = *reinterpret_cast<const uint4*>(qp);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    unpack<DT, 4>(w, qv[h]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[h][e] *= a.scale_log2;
  }

  float m[GH], lsum[GH], acc[GH][NVB];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < NVB; ++j) acc[h][j] = 0.f;
  }

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v_cache);

  for (int c0 = t0; c0 < t1; c0 += 64) {
    // ---- scores of 64 keys ----
#pragma unroll 4
    for (int ii = 0; ii < NK; ++ii) {
      const int key = c0 + ii * TPL + lane / LPR;
      const bool valid = key < t1;
      float kf[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) kf[e] = 0.f;
      if (valid) {
        const int blk = min((unsigned)bt[min(key / BS, tb_max)], (unsigned)nb_max);
        const uint8_t* kp = kbase + ((((int64_t)blk * Hkv + g) * BS + key % BS) * D + d0) * EB;
        const uint4 raw = *reinterpret_cast<const uint4*>(kp);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        unpack<DT, 4>(w, kf);
      }
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) dot = fmaf(qv[h][e], kf[e], dot);
        dot = group_sum<LPR>(dot);
        if (lane % LPR == 0) sc[h][ii * TPL + lane / LPR] = valid ? dot : -INFINITY;
      }
    }
    __syncthreads();
    // ---- online softmax: lane j owns key c0 + j ----
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const float sv = sc[h][lane];
      const float mn = fmaxf(m[h], wave_max(sv));    // finite: key c0 is valid
      const float al = fast_exp2(m[h] - mn);
      const float pv = fast_exp2(sv - mn);
      lsum[h] = lsum[h] * al + wave_sum(pv);
      m[h] = mn;
      pl[h][lane] = pv;
#pragma unroll
      for (int j = 0; j < NVB; ++j) acc[h][j] *= al;
    }
    __syncthreads();
    // ---- weighted values ----
#pragma unroll
    for (int b = 0; b < BPC; ++b) {
      const int tb = c0 + b * BS;
      if (tb >= t1) break;
      const int blk = min((unsigned)bt[min(tb / BS, tb_max)], (unsigned)nb_max);
      const uint8_t* vb = vbase + (((int64_t)blk * Hkv + g) * D) * BS * EB;
#pragma unroll
      for (int j = 0; j < NVB; ++j) {
        const int vi = j * 64 + lane;
        const int d = vi / RPV;
        const int toff = (vi % RPV) * VV;
        float vf[VV];
        if constexpr (VV * EB == 16) {
          const uint4 raw = *reinterpret_cast<const uint4*>(vb + ((int64_t)d * BS + toff) * EB);
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
          unpack<DT, 4>(w, vf);
        } else {
          const uint2 raw = *reinterpret_cast<const uint2*>(vb + ((int64_t)d * BS + toff) * EB);
          const uint32_t w[2] = {raw.x, raw.y};
          unpack<DT, 2>(w, vf);
        }
#pragma unroll
        for (int e = 0; e < VV; ++e)
          if (tb + toff + e >= t1) vf[e] = 0.f;       // unwritten slots may hold NaN
#pragma unroll
        for (int h = 0; h < GH; ++h) {
#pragma unroll
          for (int e = 0; e < VV; ++e) acc[h][j] = fmaf(pl[h][b * BS + toff + e], vf[e], acc[h][j]);
        }
      }
    }
    __syncthreads();
  }

  // Lanes that shared a head-dim row hold partial sums over different keys.
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int j = 0; j < NVB; ++j) acc[h][j] = group_sum<RPV>(acc[h][j]);
  if (lane % RPV != 0) return;

  if (it.pslot < 0) {
    using store_t = typename Elt<DT>::store_t;
    store_t* o = reinterpret_cast<store_t*>(a.out);
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const float inv = 1.f / lsum[h];
#pragma unroll
      for (int j = 0; j < NVB; ++j) {
        const int d = (j * 64 + lane) / RPV;
        const float v = acc[h][j] * inv;
        const int64_t at = ((int64_t)row * Hq + head0 + h) * D + d;
        if constexpr (DT == DT_F32) o[at] = __float_as_uint(v);
        else if constexpr (DT == DT_F16) o[at] = f32_to_f16_bits(v);
        else o[at] = f32_to_bf16_bits(v);
      }
    }
  } else {
    float* po = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + lay.part_o);
    float2* pm = reinterpret_cast<float2*>(const_cast<uint8_t*>(ws) + lay.part_ml);
    const int64_t slot = it.pslot + it.split;
    if (slot >= lay.cap_partials) {
      mark_dropped(a.ws, lay);
      return;
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
#pragma unroll
      for (int j = 0; j < NVB; ++j) {
        const int d = (j * 64 + lane) / RPV;
        po[(slot * Hq + head0 + h) * D + d] = acc[h][j];
      }
      if (lane == 0) pm[slot * Hq + head0 + h] = make_float2(m[h], lsum[h]);
    }
  }
}

// Merge the split states of one row: a thread owns four consecutive output
// elements of one head.  Split states are fetched eight at a time with
// independent loads and merged in one pass with a running max, so a row costs
// one memory latency per eight splits.
template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, WorkspaceLayout lay, int D) {
  constexpr int U = 8;
  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const PlanCounts* pc = reinterpret_cast<const PlanCounts*>(ws + lay.counts);
  if ((int)blockIdx.x >= pc->combs) return;
  const CombItem ci = reinterpret_cast<const CombItem*>(ws + lay.combs)[blockIdx.x];
  const int Hq = a.num_q_heads;
  const int q4 = D >> 2;                       // 4-element groups per head
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int h = e / q4;
  const int d = (e - h * q4) * 4;
  if (h >= Hq) return;
  if (ci.row >= a.total_q || ci.pslot < 0 || ci.pslot + ci.nsplit > lay.cap_partials) {
    mark_dropped(a.ws, lay);
    return;
  }
  const float4* po = reinterpret_cast<const float4*>(
      reinterpret_cast<const float*>(ws + lay.part_o) + (int64_t)ci.pslot * Hq * D + h * D + d);
  const float2* pm = reinterpret_cast<const float2*>(ws + lay.part_ml) + (int64_t)ci.pslot * Hq + h;
  const int64_t so = (int64_t)Hq * D / 4;      // stride between splits, in float4
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < ci.nsplit; k0 += U) {
    float2 ml[U];
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = k0 + u < ci.nsplit;
      ml[u] = in ? pm[(int64_t)(k0 + u) * Hq] : make_float2(-INFINITY, 0.f);
      o[u] = in ? po[(int64_t)(k0 + u) * so] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!(ml[u].y > 0.f)) continue;          // a split with no visible key
      const float mn = fmaxf(m, ml[u].x);
      const float sa = fast_exp2(m - mn);      // 0 while nothing is merged yet
      const float sb = fast_exp2(ml[u].x - mn);
      l = l * sa + ml[u].y * sb;
      acc.x = acc.x * sa + o[u].x * sb;
      acc.y = acc.y * sa + o[u].y * sb;
      acc.z = acc.z * sa + o[u].z * sb;
      acc.w = acc.w * sa + o[u].w * sb;
      m = mn;
    }
  }
  const float inv = 1.f / l;
  const int64_t at = ((int64_t)ci.row * Hq + h) * D + d;
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + at) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    uint2 w;
    w.x = pack2<DT>(acc.x * inv, acc.y * inv);
    w.y = pack2<DT>(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + at) = w;
  }
}

template <int DT, int D, int BS, int GH>
hipError_t launch_rows_t(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                         int num_items, int split_tokens, hipStream_t s) {
  const int G = a.num_q_heads / p.num_kv_heads;
  hipLaunchKernelGGL((row_attn_kernel<DT, D, BS, GH>), dim3(num_items, p.num_kv_heads, G / GH),
                     dim3(64), 0, s, a, p, lay, split_tokens);
  return hipGetLastError();
}

template <int DT, int D, int BS>
hipError_t launch_rows_g(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                         int num_items, int split_tokens, hipStream_t s) {
  switch (a.num_q_heads / p.num_kv_heads) {
    case 1: return launch_rows_t<DT, D, BS, 1>(a, p, lay, num_items, split_tokens, s);
    case 2: return launch_rows_t<DT, D, BS, 2>(a, p, lay, num_items, split_tokens, s);
    case 4: return launch_rows_t<DT, D, BS, 4>(a, p, lay, num_items, split_tokens, s);
    case 8:
    case 16: return launch_rows_t<DT, D, BS, 8>(a, p, lay, num_items, split_tokens, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, int D>
hipError_t launch_rows_bs(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                          int num_items, int split_tokens, hipStream_t s) {
  switch (p.block_size) {
    case 4: return launch_rows_g<DT, D, 4>(a, p, lay, num_items, split_tokens, s);
    case 8: return launch_rows_g<DT, D, 8>(a, p, lay, num_items, split_tokens, s);
    case 16: return launch_rows_g<DT, D, 16>(a, p, lay, num_items, split_tokens, s);
    case 32: return launch_rows_g<DT, D, 32>(a, p, lay, num_items, split_tokens, s);
    case 64: return launch_rows_g<DT, D, 64>(a, p, lay, num_items, split_tokens, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_rows_d(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                         int num_items, int split_tokens, hipStream_t s) {
  if (p.head_dim == 64) return launch_rows_bs<DT, 64>(a, p, lay, num_items, split_tokens, s);
  if (p.head_dim == 128) return launch_rows_bs<DT, 128>(a, p, lay, num_items, split_tokens, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_row_attention(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                                int num_items, int split_tokens, hipStream_t s) {
  if (num_items == 0) return hipSuccess;
  switch (p.dtype) {
    case DT_F32: return launch_rows_d<DT_F32>(a, p, lay, num_items, split_tokens, s);
    case DT_F16: return launch_rows_d<DT_F16>(a, p, lay, num_items, split_tokens, s);
    case DT_BF16: return launch_rows_d<DT_BF16>(a, p, lay, num_items, split_tokens, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                          int num_combs, hipStream_t s) {
  if (num_combs == 0) return hipSuccess;
  const dim3 grid(num_combs, (a.num_q_heads * p.head_dim / 4 + 255) / 256);
  switch (p.dtype) {
    case DT_F32: hipLaunchKernelGGL(combine_kernel<DT_F32>, grid, dim3(256), 0, s, a, lay, p.head_dim); break;
    case DT_F16: hipLaunchKernelGGL(combine_kernel<DT_F16>, grid, dim3(256), 0, s, a, lay, p.head_dim); break;
    case DT_BF16: hipLaunchKernelGGL(combine_kernel<DT_BF16>, grid, dim3(256), 0, s, a, lay, p.head_dim); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
