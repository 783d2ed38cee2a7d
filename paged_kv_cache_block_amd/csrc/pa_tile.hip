// MFMA multi-token paged attention (gfx950, fp16 / bf16).
//
// Pensieve page (多Token注意力内核运算原理, figure 9): with several new tokens
// per request the work is two matrix-matrix products over a context whose
// blocks sit at random physical places; Q is ragged across requests.
// (融合因果掩码与内核实现): the causal mask is applied inside the kernel and
// the score matrix is never materialised.
//
// Work item: one sequence, one KV head and a tile of 128 packed rows, where
// row r is (new token r / G, query head g*G + r % G); all G query heads of a
// KV head share each K/V tile.  Four wavefronts take 32 rows each.
//
// Per 32-key tile the workgroup stages K (token-major) and V (head-dim-major)
// in LDS, then every wavefront computes, with v_mfma_f32_32x32x16_{f16,bf16}:
//   S^T[key][row] = K[key][:] . Q[row][:]           (D/16 MFMAs)
//   online softmax per row (a row is one lane column of S^T, split over the
//   two lane halves), causal mask from absolute key positions
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]      (D/32 x 2 MFMAs)
// Working on the transposes keeps each row's statistics inside a lane pair
// and lets both operands of the second product be read as 16-byte runs.
// The K rows feeding S^T are permuted so that the eight keys a lane holds for
// each P^T operand are consecutive, which is what the V^T operand reads.

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Key (within a 32-key tile) held by accumulator element e of lane half hh.
__device__ __forceinline__ int acc_key(int e, int hh) { return 16 * (e >> 3) + 8 * hh + (e & 7); }

// Key whose K row is loaded as row r of the S^T product.  Row r of a 32x32
// accumulator lands in element 4*(r>>3) + (r&3) of lane half (r>>2)&1; this
// map sends it to acc_key of that element.
__device__ __forceinline__ int row_key(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void tile_attn_kernel(AttnArgs a, PoolArgs p,
                                                       WorkspaceLayout lay) {
  constexpr int KS = D / 16;        // k-steps of the QK product
  constexpr int NDT = D / 32;       // 32-row head-dim tiles of O^T
  constexpr int KROW = D + 8;       // LDS row stride of K (elements), padded
  constexpr int VROW = 32 + 8;      // LDS row stride of V^T (elements), padded
  constexpr int KCH = D / 64;       // 16-byte K chunks per thread per tile
  constexpr int VCH = D / 64;       // 16-byte V chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[D * VROW];

  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const PlanCounts* pc = reinterpret_cast<const PlanCounts*>(ws + lay.counts);
  if ((int)blockIdx.x >= pc->tiles) return;
  const TileItem ti = reinterpret_cast<const TileItem*>(ws + lay.tiles)[blockIdx.x];

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int g = blockIdx.y;
  const int Hq = a.num_q_heads;
  const int Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int s = ti.seq;
  const int q0 = a.qsl[s];
  const int n = a.qsl[s + 1] - q0;
  const int L = a.context_lens[s];
  const int R = n * G;
  const int r0 = ti.tile * kTileRows;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const int nb_max = p.num_blocks - 1;
  const int tb_max = a.max_blocks - 1;

  // This lane's row.
  const int r = r0 + 32 * wv + col;
  const bool row_ok = r < R && q0 + r / G < a.total_q;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int p_row = row_ok ? L - n + qi : -1;
  // Key ranges: the workgroup's and this wave's (rows ascend, so the last
  // row of a range has the largest causal limit).
  const int kend = L - n + (min(R, r0 + kTileRows) - 1) / G + 1;
  const bool wave_on = r0 + 32 * wv < R;
  const int wend = wave_on ? L - n + (min(R, r0 + 32 * wv + 32) - 1) / G + 1 : 0;

  // Q^T operand of the QK product: lane (col, hh) holds Q[row col][16ks+8hh .. +8].
  u32x4 qreg[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(q0 + qi) * Hq + hq) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0, 0, 0, 0};
  }

  f32x16 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache);
  u32x4 kbuf[KCH], vbuf[VCH];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + 256 * c;
      const int tok = idx / (D / 8);
      const int dc = idx % (D / 8);
      const int key = kt * 32 + tok;
      if (key < kend) {
        const int blk = min((unsigned)bt[min(key / BS, tb_max)], (unsigned)nb_max);
        kbuf[c] = *reinterpret_cast<const u32x4*>(
            kc + (((int64_t)blk * Hkv + g) * BS + key % BS) * D + dc * 8);
      } else {
        kbuf[c] = u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + 256 * c;
      const int d = idx >> 2;
      const int tc = idx & 3;
      const int key0 = kt * 32 + tc * 8;
      if (key0 < kend) {
        const int blk = min((unsigned)bt[min(key0 / BS, tb_max)], (unsigned)nb_max);
        u32x4 v = *reinterpret_cast<const u32x4*>(
            vc + (((int64_t)blk * Hkv + g) * D + d) * BS + key0 % BS);
        if (key0 + 8 > kend) {       // unwritten slots may hold NaN
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t x = v[w];
            if (key0 + 2 * w >= kend) x &= 0xffff0000u;
            if (key0 + 2 * w + 1 >= kend) x &= 0x0000ffffu;
            v[w] = x;
          }
        }
        vbuf[c] = v;
      } else {
        vbuf[c] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + 256 * c;
      *reinterpret_cast<u32x4*>(&Ks[(idx / (D / 8)) * KROW + (idx % (D / 8)) * 8]) = kbuf[c];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + 256 * c;
      *reinterpret_cast<u32x4*>(&Vs[(idx >> 2) * VROW + (idx & 3) * 8]) = vbuf[c];
    }
  };

  const int ntiles = (kend + 31) / 32;
  const int krow = row_key(col);
  load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kt + 1);
    const int kt0 = kt * 32;
    if (!wave_on || kt0 >= wend) continue;

    // S^T = K . Q^T
    f32x16 sacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(&Ks[krow * KROW + 16 * ks + 8 * hh]);
      sacc = mfma32<DT>(ka, qreg[ks], sacc);
    }

    // Online softmax for row `col` (this lane holds 16 of its 32 keys).
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kt0 + acc_key(e, hh);
      sv[e] = key <= p_row ? sacc[e] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sv[e] = fast_exp2(sv[e] - m_use);
      rs += sv[e];
    }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[t][e] *= alpha;

    // P^T operands: keys 8hh..8hh+7 and 16+8hh..16+8hh+7 of the tile.
    u32x4 pb[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int w = 0; w < 4; ++w) pb[st][w] = pack2<DT>(sv[8 * st + 2 * w], sv[8 * st + 2 * w + 1]);

    // O^T += V^T . P^T
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 va =
            *reinterpret_cast<const u32x4*>(&Vs[(32 * t + col) * VROW + 16 * st + 8 * hh]);
        o[t] = mfma32<DT>(va, pb[st], o[t]);
      }
    }
  }

  if (!row_ok) return;
  const float inv = 1.f / l_run;
  uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)(q0 + qi) * Hq + hq) * D;
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * t + 8 * a4 + 4 * hh;
      uint2 w;
      w.x = pack2<DT>(o[t][4 * a4] * inv, o[t][4 * a4 + 1] * inv);
      w.y = pack2<DT>(o[t][4 * a4 + 2] * inv, o[t][4 * a4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
  }
}

template <int DT, int D>
hipError_t launch_tile_d(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                         int num_tiles, hipStream_t s) {
  const dim3 grid(num_tiles, p.num_kv_heads);
  if (p.block_size == 16)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 16>), grid, dim3(256), 0, s, a, p, lay);
  else if (p.block_size == 32)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 32>), grid, dim3(256), 0, s, a, p, lay);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool tile_path_supported(const PoolArgs& p) {
  return (p.dtype == DT_F16 || p.dtype == DT_BF16) && (p.block_size == 16 || p.block_size == 32) &&
         (p.head_dim == 64 || p.head_dim == 128);
}

hipError_t launch_tile_attention(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                                 int num_tiles, hipStream_t s) {
  if (num_tiles == 0) return hipSuccess;
  if (p.dtype == DT_F16) {
    if (p.head_dim == 64) return launch_tile_d<DT_F16, 64>(a, p, lay, num_tiles, s);
    if (p.head_dim == 128) return launch_tile_d<DT_F16, 128>(a, p, lay, num_tiles, s);
  } else if (p.dtype == DT_BF16) {
    if (p.head_dim == 64) return launch_tile_d<DT_BF16, 64>(a, p, lay, num_tiles, s);
    if (p.head_dim == 128) return launch_tile_d<DT_BF16, 128>(a, p, lay, num_tiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
