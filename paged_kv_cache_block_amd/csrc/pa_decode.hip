// MFMA decode attention (gfx950, fp16 / bf16): one query token per row.
//
// vLLM-SOSP23 page (核心方法, Kernel 层实现) and Pensieve page (多Token注意力
// 内核运算原理): a decode token's attention is two matrix-vector products over
// a paged context, read block by block through the block table.  Decode is
// bound by HBM (vLLM blog page, 挑战), so the design goal is that every byte of
// K and V is read once per KV head and that enough of them are in flight.
//
// One wavefront owns one (sequence, KV head, key split); wavefronts are
// numbered so that consecutive work items run on one XCD.  The up-to-16 query
// heads of the KV head's group form the columns of 16x16 MFMA tiles, so a K/V
// load serves all of them:
//   S^T[key][head]  = K[key][:] . Q[head][:]      v_mfma_f32_16x16x32_{f16,bf16}
//   online softmax per head (a head is one lane column of S^T)
//   O^T[d][head]   += V^T[d][key] . P^T[key][head]
// The V^T operand is read straight from HBM into registers: V is head-dim-
// major inside a block, so lane (row d, k-group c) loads the 8 consecutive
// keys 8c..8c+7 of head-dim row d.  K (token-major) is read as contiguous
// 1 KB pieces, each lane one 16-byte chunk, and reaches the operand layout
// (lane (row r, k-group c): 16 bytes of key row r) through LDS.
// The K rows are permuted so the four S^T values a lane gets from each of the
// two key tiles are exactly the 8 consecutive keys its P^T operand needs.
// Keys go 32 per step, double-buffered: the next step's K and V loads are in
// flight while the current step computes.  K rows are loaded as contiguous
// 1 KB pieces and pass through 8 KB of LDS per wave to reach the operand
// layout.

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLazyRescale = 8.f;  // log2 headroom before the running max moves

// Two floats to two packed 16-bit values, round to nearest even (hardware).
template <int DT>
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  if constexpr (DT == DT_F16) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <int DT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-byte load; NT streams past the caches (data read once).  A 32-key step
// reads only part of each V^T row of a block larger than 32 tokens, and the
// next step reads the rest, so those loads keep the caches.
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

template <int D>
struct Stage {
  u32x4 k[D / 16];      // the step's 32 K rows, as D/16 contiguous 1 KB pieces
  u32x4 v[D / 16];      // D/16 head-dim tiles, 8 keys each
};

// Position of 16-byte chunk j of key row r (0..31) in a wave's LDS copy of a
// step's K rows: rows of 2D bytes, chunks XOR-swizzled by row so that the
// operand reads (16 rows, one chunk) hit distinct banks.
template <int D>
__device__ __forceinline__ int kslot(int r, int j) {
  const int sw = D == 128 ? ((r & 3) | (((r >> 3) & 3) << 2)) : ((r & 3) | (((r >> 3) & 1) << 2));
  return r * (D / 8) + (j ^ sw);
}

template <int DT, int D, int BS, bool NT>
__global__ __launch_bounds__(64, 2) void decode_mfma_kernel(AttnArgs a, PoolArgs p,
                                                         WorkspaceLayout lay, int split_tokens) {
  constexpr int KS = D / 32;
  constexpr int NDT = D / 16;
  static_assert(BS == 16 || BS % 32 == 0, "a 32-key step spans two blocks of 16 or lies in one block");

  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const PlanCounts* pc = reinterpret_cast<const PlanCounts*>(ws + lay.counts);
  // Work items (row splits) in plan order, each over all KV heads, numbered
  // so that consecutive items -- the splits of one row, and rows of adjacent
  // sequences, which share prompt blocks when a block manager forks them --
  // run on one XCD.
  // With a.rows_dealt the plan lists items longest first and they are dealt
  // round-robin over the XCDs instead, whole items (all KV heads) at a time:
  // XCD x takes items x, x + 8, x + 16, ..., so each gets an even share of
  // the work (used when no block is read by two rows).
  const int Hkv = p.num_kv_heads;
  int item, g;
  if (a.rows_dealt) {
    const int pos = blockIdx.x >> 3;
    const int round = pos / Hkv;
    g = pos - round * Hkv;
    item = 8 * round + (blockIdx.x & 7);
  } else {
    const int logical = xcd_order(blockIdx.x, gridDim.x);
    item = logical / Hkv;
    g = logical - item * Hkv;
  }
  if (item >= pc->rows) return;
  const RowItem it = reinterpret_cast<const RowItem*>(ws + lay.rows)[item];

  const int lane = threadIdx.x;
  const int c16 = lane & 15;       // MFMA row of A / column of B and C
  const int grp = lane >> 4;       // k-group of A and B; row group of C
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  const int s = it.seq;
  const int q0 = a.qsl[s];
  const int n = a.qsl[s + 1] - q0;
  const int L = a.context_lens[s];
  const int row = q0 + it.i;
  if (row >= a.total_q) {
    mark_dropped(a.ws, lay);
    return;
  }
  const int t0 = it.split * split_tokens;
  const int t1 = min(L - n + it.i + 1, t0 + split_tokens);
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const unsigned nb_max = p.num_blocks - 1;
  const int tb_max = a.max_blocks - 1;
  const bool head_ok = c16 < G;
  const int head = g * G + (head_ok ? c16 : 0);

  // Q^T operand: column c16 is query head g*G + c16; k-group grp covers
  // head-dim elements 32ks + 8grp .. +8.
  u32x4 qreg[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)row * Hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = head_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * ks + 8 * grp)
                         : u32x4{0, 0, 0, 0};
  }

  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache);
  // Key offsets within a 32-key step: A row c16 of key tile u holds key
  // 8*(c16>>2) + 4u + (c16&3); lane group grp's V operand holds keys 8grp..8grp+7.
  const int krow0 = 8 * (c16 >> 2) + (c16 & 3);
  const int vkey = 8 * grp;
  // K is loaded as contiguous 1 KB pieces (piece i: keys KPI*i .. +KPI, lane
  // = 16-byte chunk; reads shaped so stream faster than 64-byte row pieces)
  // and rearranged into the MFMA operand layout through LDS.
  constexpr int CPRW = D / 8;          // 16-byte chunks per K row
  constexpr int KPI = 64 / CPRW;       // keys per 1 KB piece
  __shared__ __attribute__((aligned(16))) u32x4 kl[32 * CPRW];
  const int pkey = lane / CPRW, pchunk = lane % CPRW;

  // The split's block ids, one per lane, 64 blocks at a time (clamped to the
  // table row and the pool, so every load below stays inside them): a step
  // takes its ids with readlane, so its K/V loads wait on no table load.
  // The split starts on an even block (split_tokens is a multiple of 64), so
  // the two 16-token blocks of a step never straddle two windows.
  const int blk0 = t0 / BS;
  int win = -1;
  unsigned btlane = 0;
  auto block_id = [&](int b) -> unsigned {   // b: block of the sequence, wave-uniform
    const int w = (b - blk0) >> 6;
    if (w != win) {
      win = w;
      btlane = min((unsigned)bt[min(blk0 + 64 * w + lane, tb_max)], nb_max);
    }
    return (unsigned)__builtin_amdgcn_readlane((int)btlane, b - blk0 - 64 * w);
  };
  auto load = [&](int c0, Stage<D>& st) {
    const unsigned b0 = block_id(c0 / BS);
    unsigned b1 = b0;
    if constexpr (BS == 16) b1 = block_id(c0 / BS + 1);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int kk = KPI * i + pkey;                      // 0..31
      const unsigned blk = (BS == 16 && kk >= 16) ? b1 : b0;
      const int off = (c0 + kk) % BS;
      st.k[i] = ld16<NT>(kc + (((int64_t)blk * Hkv + g) * BS + off) * D + 8 * pchunk);
    }
    {
      const unsigned blk = (BS == 16 && vkey >= 16) ? b1 : b0;
      const int off = (c0 + vkey) % BS;
      const uint16_t* vp = vc + (((int64_t)blk * Hkv + g) * D + c16) * BS + off;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        st.v[dt] = ld16<NT && BS <= 32>(vp + (int64_t)16 * dt * BS);
    }
  };

  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](int c0, Stage<D>& st) {
    // K pieces to LDS, then the operands back in MFMA layout (one wave per
    // workgroup: the LDS ops of a wave complete in order, so no barrier).
#pragma unroll
    for (int i = 0; i < D / 16; ++i) kl[kslot<D>(KPI * i + pkey, pchunk)] = st.k[i];
    u32x4 kop[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kop[u][ks] = kl[kslot<D>(krow0 + 4 * u, 4 * ks + grp)];
    f32x4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[u] = mfma16<DT>(kop[u][ks], qreg[ks], sacc[u]);
    }
    // This lane holds head c16's scores for keys c0 + 8grp + (4u + i).
    const bool tail = c0 + 32 > t1;
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[u][i] * a.scale_log2;
        if (tail && c0 + vkey + 4 * u + i >= t1) x = -INFINITY;
        sv[4 * u + i] = x;
        mx = fmaxf(mx, x);
      }
    mx = xor_max<32>(xor_max<16>(mx));
    // The running max only moves when this step's max passes it by 2^8; the
    // weights stay below 2^8 and most steps skip rescaling O.
    if (mx > m_run + kLazyRescale) {               // per column (lane): may diverge
      const float alpha = fast_exp2(m_run - mx);   // 0 on the first step
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m_run = mx;
    }
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = fast_exp2(sv[e] - m_run);
      rs += sv[e];
    }
    rs = xor_sum<32>(xor_sum<16>(rs));
    l_run += rs;
    u32x4 pb;
#pragma unroll
    for (int w = 0; w < 4; ++w) pb[w] = cvt2<DT>(sv[2 * w], sv[2 * w + 1]);
    if (tail) {
      // Slots at or past t1 may be unwritten (NaN); zero them, never multiply.
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x = st.v[dt][w];
          if (c0 + vkey + 2 * w >= t1) x &= 0xffff0000u;
          if (c0 + vkey + 2 * w + 1 >= t1) x &= 0x0000ffffu;
          st.v[dt][w] = x;
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma16<DT>(st.v[dt], pb, o[dt]);
  };

  Stage<D> sa, sb;
  int c0 = t0;
  load(c0, sa);
  while (true) {
    if (c0 + 32 < t1) load(c0 + 32, sb);
    compute(c0, sa);
    c0 += 32;
    if (c0 >= t1) break;
    if (c0 + 32 < t1) load(c0 + 32, sa);
    compute(c0, sb);
    c0 += 32;
    if (c0 >= t1) break;
  }

  if (!head_ok) return;
  if (it.pslot < 0) {
    const float inv = 1.f / l_run;
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)row * Hq + head) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint2 w;
      w.x = pack2<DT>(o[dt][0] * inv, o[dt][1] * inv);
      w.y = pack2<DT>(o[dt][2] * inv, o[dt][3] * inv);
      *reinterpret_cast<uint2*>(op + 16 * dt) = w;
    }
  } else {
    const int64_t slot = it.pslot + it.split;
    if (slot >= lay.cap_partials) {
      mark_dropped(a.ws, lay);
      return;
    }
    float* po = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + lay.part_o) +
                (slot * Hq + head) * D + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (grp == 0) {
      float2* pm = reinterpret_cast<float2*>(const_cast<uint8_t*>(ws) + lay.part_ml);
      pm[slot * Hq + head] = make_float2(m_run, l_run);
    }
  }
}

template <int DT, int D, bool NT>
hipError_t launch_d(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay, int items,
                    int split, hipStream_t s) {
  const int64_t groups = decode_mfma_groups(items, p.num_kv_heads, a.rows_dealt != 0);
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups);
  if (p.block_size == 16)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 16, NT>), grid, dim3(64), 0, s, a, p, lay, split);
  else if (p.block_size == 32)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 32, NT>), grid, dim3(64), 0, s, a, p, lay, split);
  else if (p.block_size == 64)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 64, NT>), grid, dim3(64), 0, s, a, p, lay, split);
  else if (p.block_size == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<DT, D, 128, NT>), grid, dim3(64), 0, s, a, p, lay, split);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_nt(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay, int items,
                     int split, bool stream_kv, hipStream_t s) {
  return stream_kv ? launch_d<DT, D, true>(a, p, lay, items, split, s)
                   : launch_d<DT, D, false>(a, p, lay, items, split, s);
}

}  // namespace

int64_t decode_mfma_groups(int64_t num_items, int num_kv_heads, bool dealt) {
  return (dealt ? (num_items + 7) / 8 * 8 : num_items) * num_kv_heads;
}

bool decode_mfma_supported(const PoolArgs& p, int group) {
  return (p.dtype == DT_F16 || p.dtype == DT_BF16) && (p.block_size == 16 || p.block_size == 32 || p.block_size == 64 || p.block_size == 128) &&
         (p.head_dim == 64 || p.head_dim == 128) && group <= 16;
}

hipError_t launch_decode_mfma(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                              int num_items, int split_tokens, bool stream_kv, hipStream_t s) {
  if (num_items == 0) return hipSuccess;
  if (p.dtype == DT_F16) {
    if (p.head_dim == 64) return launch_nt<DT_F16, 64>(a, p, lay, num_items, split_tokens, stream_kv, s);
    if (p.head_dim == 128) return launch_nt<DT_F16, 128>(a, p, lay, num_items, split_tokens, stream_kv, s);
  } else if (p.dtype == DT_BF16) {
    if (p.head_dim == 64) return launch_nt<DT_BF16, 64>(a, p, lay, num_items, split_tokens, stream_kv, s);
    if (p.head_dim == 128) return launch_nt<DT_BF16, 128>(a, p, lay, num_items, split_tokens, stream_kv, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
