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
// Keys go 64 per iteration through a two-stage LDS ring: while the waves
// compute on one stage, every thread holds the next tile's K/V chunks in
// registers and writes them to the other stage afterwards; one barrier per
// iteration.  Each wave computes, with v_mfma_f32_32x32x16_{f16,bf16}:
//   S^T[key][row] = K[key][:] . Q[row][:]           (2 x D/16 MFMAs)
//   online softmax per row (a row is one lane column of S^T, split over the
//   two lane halves), causal mask from absolute key positions
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]      (D/32 x 4 MFMAs)
// Working on the transposes keeps each row's statistics inside a lane pair
// and lets both operands of the second product be read as 16-byte runs.
// The K rows feeding S^T are permuted so that the eight keys a lane holds for
// each P^T operand are consecutive, which is what the V^T operand reads.
// The running max is only raised (and O rescaled) when a row's max grows by
// more than 2^8, so most iterations skip the rescale.
// Workgroups are numbered so that the tiles sharing one (sequence, KV head)
// run on one XCD and reuse its L2.

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKeys = 64;          // keys per iteration
constexpr int kTabWin = 256;       // block-table entries staged in LDS at a time
constexpr float kLazyRescale = 8.f;  // log2 headroom before the running max moves

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

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

// acc + the two packed 16-bit values of w (v_dot2 with a ones vector).
template <int DT>
__device__ __forceinline__ float dot2_ones(uint32_t w, float acc) {
  if constexpr (DT == DT_F16) {
    const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
  } else {
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
  }
}

// Key (within a 32-key half tile) held by accumulator element e of lane half hh.
__device__ __forceinline__ int acc_key(int e, int hh) { return 16 * (e >> 3) + 8 * hh + (e & 7); }

// Key whose K row is loaded as row r of the S^T product.  Row r of a 32x32
// accumulator lands in element 4*(r>>3) + (r&3) of lane half (r>>2)&1; this
// map sends it to acc_key of that element.
__device__ __forceinline__ int row_key(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

// The other lane half's copy of x (lanes l and l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// Logical work index of this workgroup: consecutive logical indices share
// K/V, and each XCD (workgroups dispatched round-robin over 8) gets one
// contiguous range of them.
__device__ __forceinline__ int xcd_order(int bid, int n) {
  const int xcd = bid & 7, pos = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + min(xcd, rem) + pos;
}

template <int DT, int D, int BS>
__global__ __launch_bounds__(256, 2) void tile_attn_kernel(AttnArgs a, PoolArgs p,
                                                          WorkspaceLayout lay, int num_tiles) {
  constexpr int KS = D / 16;        // k-steps of the QK product
  constexpr int NDT = D / 32;       // 32-row head-dim tiles of O^T
  constexpr int KROW = D + 8;       // LDS row stride of K (elements), padded
  constexpr int VROW = kKeys + 8;   // LDS row stride of V^T (elements), padded
  constexpr int KCH = kKeys * D / 8 / 256;   // 16-byte K chunks per thread per tile
  constexpr int VCH = D * kKeys / 8 / 256;   // 16-byte V chunks per thread per tile
  constexpr int KSTAGE = kKeys * KROW;
  constexpr int VSTAGE = D * VROW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * KSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * VSTAGE];
  __shared__ unsigned btab[kTabWin];

  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const PlanCounts* pc = reinterpret_cast<const PlanCounts*>(ws + lay.counts);
  const int Hkv = p.num_kv_heads;
  const int logical = xcd_order(blockIdx.x, gridDim.x);
  const int g = logical / num_tiles;
  const int item = logical - g * num_tiles;
  if (item >= pc->tiles) return;
  const TileItem ti = reinterpret_cast<const TileItem*>(ws + lay.tiles)[item];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int Hq = a.num_q_heads;
  const int G = Hq / Hkv;
  const int s = ti.seq;
  const int q0 = a.qsl[s];
  const int n = a.qsl[s + 1] - q0;
  const int L = a.context_lens[s];
  const int R = n * G;
  const int r0 = ti.tile * kTileRows;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const unsigned nb_max = p.num_blocks - 1;
  const int tb_max = a.max_blocks - 1;
  const float c = a.scale_log2;

  // This lane's row.
  const int r = r0 + 32 * wv + col;
  const bool row_ok = r < R && q0 + r / G < a.total_q;
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int p_row = row_ok ? L - n + qi : -1;
  // Key ranges: the workgroup's and this wave's (rows ascend, so the last
  // row of a range has the largest causal limit, the first the smallest).
  const int kend = L - n + (min(R, r0 + kTileRows) - 1) / G + 1;
  const bool wave_on = r0 + 32 * wv < R;
  const bool wave_full = r0 + 32 * wv + 32 <= R;
  const int wend = wave_on ? L - n + (min(R, r0 + 32 * wv + 32) - 1) / G + 1 : 0;
  const int wfirst = wave_on ? L - n + (r0 + 32 * wv) / G : 0;

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

  // Per-thread parts of the tile loads.  K chunk j is key kt0 + ktok + KRP*j,
  // head-dim chunk kdc; V chunk j is head-dim row vd + 32*j, keys
  // kt0 + vkey .. +8.  Offsets are within a block's (block, head) slice.
  constexpr int TPR = D / 8;            // 16-byte chunks per K row
  constexpr int KRP = 256 / TPR;        // K rows per pass of the workgroup
  const int ktok = tid / TPR;
  const int kdc = tid % TPR;
  const int vd = tid >> 3;
  const int vkey = 8 * (tid & 7);
  const uint64_t kstride = (uint64_t)Hkv * BS * D;     // elements per physical block
  int kofs[KCH];
#pragma unroll
  for (int j = 0; j < KCH; ++j) kofs[j] = ((g * BS + (ktok + KRP * j) % BS) * D) + kdc * 8;
  int vofs[VCH];
#pragma unroll
  for (int j = 0; j < VCH; ++j) vofs[j] = ((g * D + vd + 32 * j) * BS) + vkey % BS;

  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache);
  u32x4 kbuf[KCH], vbuf[VCH];

  // The sequence's block ids, kTabWin at a time, clamped to the pool (so
  // every load below stays inside it).  A 64-key tile never straddles two
  // windows (kTabWin is a multiple of 64/BS).
  int win = -1;
  auto ensure_window = [&](int kt) {
    const int w = (kt * kKeys / BS) / kTabWin;
    if (w == win) return;
    __syncthreads();
    for (int i = tid; i < kTabWin; i += 256)
      btab[i] = min((unsigned)bt[min(w * kTabWin + i, tb_max)], nb_max);
    __syncthreads();
    win = w;
  };
  auto load_tile = [&](int kt) {
    ensure_window(kt);
    const int kt0 = kt * kKeys;
    const int b0 = kt0 / BS - win * kTabWin;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const unsigned blk = btab[b0 + (ktok + KRP * j) / BS];
      kbuf[j] = *reinterpret_cast<const u32x4*>(kc + blk * kstride + kofs[j]);
    }
    const unsigned vblk = btab[b0 + vkey / BS];
#pragma unroll
    for (int j = 0; j < VCH; ++j)
      vbuf[j] = *reinterpret_cast<const u32x4*>(vc + vblk * kstride + vofs[j]);
    if (kt0 + kKeys > kend) {
      // Tail tile: slots at or past kend may be unwritten (NaN).  Zero the V
      // entries (a zero probability must not meet them); K rows there are
      // masked to -inf before the softmax.  The empty asm keeps this a real
      // branch instead of selects executed on every tile.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < VCH; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x = vbuf[j][w];
          if (kt0 + vkey + 2 * w >= kend) x &= 0xffff0000u;
          if (kt0 + vkey + 2 * w + 1 >= kend) x &= 0x0000ffffu;
          vbuf[j][w] = x;
        }
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* kd = Ks + stage * KSTAGE + ktok * KROW + kdc * 8;
    uint16_t* vd_ = Vs + stage * VSTAGE + vd * VROW + vkey;
#pragma unroll
    for (int j = 0; j < KCH; ++j) *reinterpret_cast<u32x4*>(kd + KRP * j * KROW) = kbuf[j];
#pragma unroll
    for (int j = 0; j < VCH; ++j) *reinterpret_cast<u32x4*>(vd_ + 32 * j * VROW) = vbuf[j];
  };

  const int ntiles = (kend + kKeys - 1) / kKeys;
  const int krow = row_key(col);
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < ntiles) load_tile(kt + 1);
    const int kt0 = kt * kKeys;
    if (wave_on && kt0 < wend) {
      const uint16_t* ks_ = Ks + stage * KSTAGE;
      const uint16_t* vs_ = Vs + stage * VSTAGE;
      // S^T = K . Q^T for keys kt0 + [0, 32) and kt0 + [32, 64).
      f32x16 sacc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[u][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(
              &ks_[(32 * u + krow) * KROW + 16 * ks + 8 * hh]);
          sacc[u] = mfma32<DT>(ka, qreg[ks], sacc[u]);
        }
      }
      // Causal mask (a select), only where some key passes some row's limit.
      if (!wave_full || kt0 + kKeys - 1 > wfirst) {
        const int lim = p_row - kt0 - 8 * hh;    // key kt0 + 32u + 16(e>>3) + 8hh + (e&7)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * u + 16 * (e >> 3) + (e & 7) > lim) sacc[u][e] = -INFINITY;
      }
      // Online softmax and P.V per 32-key half: while the VALU works on one
      // half, the MFMAs of the other half's products are in flight.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[u][e]);
        mx = fmaxf(mx, swap_halves(mx));
        const float m_cand = mx * c;
        const bool raise = m_cand > m_run + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float m_new = raise ? m_cand : m_run;
          const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;   // 0 on the first raise
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < NDT; ++t) o[t] *= alpha;
          m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        u32x4 pb[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[u][e] = fast_exp2(fmaf(sacc[u][e], c, -m_use));
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pb[v2][w] = cvt2<DT>(sacc[u][8 * v2 + 2 * w], sacc[u][8 * v2 + 2 * w + 1]);
        // Row sum of the rounded probabilities the MFMA consumes (packed dot
        // products with ones), so O is normalised by exactly its own weights.
        float rs = 0.f;
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w) rs = dot2_ones<DT>(pb[v2][w], rs);
        rs += swap_halves(rs);
        l_run += rs;
        // O^T += V^T . P^T over the half's 2 k-steps of 16 keys.
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
#pragma unroll
          for (int v2 = 0; v2 < 2; ++v2) {
            const u32x4 va = *reinterpret_cast<const u32x4*>(
                &vs_[(32 * t + col) * VROW + 32 * u + 16 * v2 + 8 * hh]);
            o[t] = mfma32<DT>(va, pb[v2], o[t]);
          }
        }
      }
    }
    if (kt + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
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
      w.x = cvt2<DT>(o[t][4 * a4] * inv, o[t][4 * a4 + 1] * inv);
      w.y = cvt2<DT>(o[t][4 * a4 + 2] * inv, o[t][4 * a4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
  }
}

template <int DT, int D>
hipError_t launch_tile_d(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                         int num_tiles, hipStream_t s) {
  const dim3 grid(num_tiles * p.num_kv_heads);
  if (p.block_size == 16)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 16>), grid, dim3(256), 0, s, a, p, lay, num_tiles);
  else if (p.block_size == 32)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 32>), grid, dim3(256), 0, s, a, p, lay, num_tiles);
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
  if ((int64_t)num_tiles * p.num_kv_heads > 0x7fffffff) return hipErrorInvalidValue;
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
