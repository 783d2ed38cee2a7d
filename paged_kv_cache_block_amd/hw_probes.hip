// Hardware ceilings the attention kernels are measured against (MI355X,
// gfx950).  A standalone program, built next to the library:
//
//   paged_kv_cache_block_amd/hw_probes read   HBM read rate: sequential and
//                                             random 4 KB chunks, and the two
//                                             load shapes the decode kernel
//                                             could use for its K operand
//   paged_kv_cache_block_amd/hw_probes lds    ds_read_b128 bytes per clock per CU
//   paged_kv_cache_block_amd/hw_probes ldsmap ds_read_b128 rate for the lane ->
//                                             address maps an MFMA operand read
//                                             from a padded or swizzled tile uses
//   paged_kv_cache_block_amd/hw_probes mfma   32x32x16 bf16 MFMA rate, and how
//                                             vector work overlaps it within one
//                                             wave and across two waves of a SIMD
//   paged_kv_cache_block_amd/hw_probes attnloop  an attention-shaped loop: per 32-key
//                                             half, 8 dependent MFMAs from LDS
//                                             operands, a softmax, 8 more MFMAs,
//                                             with parts switched off
//
// Every kernel writes one output element per thread into a buffer sized for
// its grid and reads only inside its own input buffer.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CK(x)                                                                         \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

namespace {

constexpr double kNominalHz = 2.4e9;   // clock the published peaks assume

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// ---- read ------------------------------------------------------------------
// Sequential: grid-stride over n 16-byte chunks, U loads in flight per thread.
template <int U, bool NT>
__global__ __launch_bounds__(256) void read_seq(const u32x4* __restrict__ p, size_t n, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * 256 * U;
  u32x4 acc = {0, 0, 0, 0};
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i + 256 * (U - 1) < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + 256 * u) : p[i + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Random 4 KB chunks (chunk-aligned, hashed from wave and iteration), 8 KB per
// iteration per wave (8 loads of 1 KB in flight).  SHAPE 0: each load reads
// 1 KB contiguously (lane = 16-byte chunk); SHAPE 1: each load reads 16 rows
// of 64 bytes, rows 256 bytes apart (lane (row r, group c) = 16 bytes at
// r * 256 + 64 * load + 16 * c), the shape of a 16x16x32 MFMA A operand over
// 256-byte key rows.
template <int SHAPE, bool NT>
__global__ __launch_bounds__(64) void read_chunks(const u32x4* __restrict__ p, uint32_t nchunks,
                                                  int iters, uint32_t* out) {
  const int lane = threadIdx.x;
  const int r = lane & 15, c = lane >> 4;
  u32x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t ch = mix32(blockIdx.x * 7919u + it * 104729u + k * 31u) % nchunks;
      const u32x4* base = p + (size_t)ch * 256;   // 4 KB = 256 chunks of 16 bytes
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const int idx = SHAPE == 0 ? l * 64 + lane : r * 16 + l * 4 + c;
        v[k * 4 + l] = NT ? __builtin_nontemporal_load(base + idx) : base[idx];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  out[blockIdx.x * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---- lds -------------------------------------------------------------------
// Each wave reads 1 KB per ds_read_b128 (lane l: 16 bytes at l * 16 + 1 KB * j,
// conflict free) from a 64 KB buffer.
template <int NT>
__global__ __launch_bounds__(NT) void lds_read(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];
  for (int i = threadIdx.x; i < 16384; i += NT) buf[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  u32x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int off = ((lane * 4) + 256 * ((j + wv * 3 + it) & 63)) & 16383;
      acc ^= *reinterpret_cast<const u32x4*>(&buf[off]);
    }
  }
  out[blockIdx.x * NT + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---- ldsmap ----------------------------------------------------------------
// Byte address read by lane `lane` for map M: a 64-lane ds_read_b128 of one
// 32x32x16 MFMA operand, lane (c = lane & 31, h = lane >> 5) taking 16 bytes
// of row r(c) at column chunk h of a tile with the given row pitch.
//   0: contiguous 1 KB (lane * 16)
//   1: r = c, pitch 272 B (128 16-bit values + 8 of padding)
//   2: r = a permutation of c (16 (c>>4) + 8 ((c>>2)&1) + 4 ((c>>3)&1) + (c&3)), pitch 272 B
//   3: r = c, pitch 256 B (no padding)
//   4: r = c, pitch 256 B, 16-byte chunk index XOR (r & 15)
//   5: r = c, pitch 264 B
//   6: r = c, pitch 288 B
//   7: permuted r as in 2, pitch 256 B, chunk XOR (r & 15)
//   8: r = c, pitch 256 B, chunk XOR ((r >> 1) & 15)
//   9: permuted r as in 2, pitch 288 B
__device__ __forceinline__ uint32_t lds_map(int m, int lane) {
  const int c = lane & 31, h = lane >> 5;
  const int rp = 16 * (c >> 4) + 8 * ((c >> 2) & 1) + 4 * ((c >> 3) & 1) + (c & 3);
  switch (m) {
    case 0: return lane * 16;
    case 1: return c * 272 + 16 * h;
    case 2: return rp * 272 + 16 * h;
    case 3: return c * 256 + 16 * h;
    case 4: return c * 256 + 16 * (h ^ (c & 15));
    case 5: return c * 264 + 16 * h;
    case 6: return c * 288 + 16 * h;
    case 7: return rp * 256 + 16 * (h ^ (rp & 15));
    case 8: return c * 256 + 16 * (h ^ ((c >> 1) & 15));
    default: return rp * 288 + 16 * h;
  }
}

// 8 waves, each issuing 16 reads per iteration at lds_map(M) plus a per-read
// offset that is a multiple of 4 KB (so the bank pattern is the map's).
template <int M>
__global__ __launch_bounds__(512) void lds_map_read(uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];   // 64 KB
  for (int i = threadIdx.x; i < 16384; i += 512) buf[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t a = lds_map(M, lane);   // < 32 * 288 = 9216
  u32x4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t off = (4096u * ((j + wv * 3 + it) % 13) + a) / 4;   // < 49152 + 9216 bytes
      acc ^= *reinterpret_cast<const u32x4*>(&buf[off]);
    }
  }
  out[blockIdx.x * 512 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---- mfma ------------------------------------------------------------------
__device__ __forceinline__ void mfma_operands(u32x4& a, u32x4& b) {
  const uint32_t lane = threadIdx.x & 63;
  a = u32x4{lane * 3u, lane * 5u, lane * 7u, lane * 11u} & 0x3f003f00u;   // small bf16 values
  b = u32x4{lane * 13u, lane * 17u, lane * 19u, lane * 23u} & 0x3f003f00u;
}
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One wave: a dependent MFMA chain, each MFMA followed by NV independent
// vector ops (fma, or exp2 when EXP), fenced so the order holds.
template <int NV, bool EXP>
__global__ __launch_bounds__(256) void mfma_then_valu(float* out, int iters) {
  u32x4 a, b;
  mfma_operands(a, b);
  f32x16 c0 = {};
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = 0.001f * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c0 = mfma(a, b, c0);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if constexpr (EXP) x[v & 15] = __builtin_amdgcn_exp2f(x[v & 15]);
        else x[v & 15] = fmaf(x[v & 15], 0.999f, 0.001f);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
  for (int e = 0; e < 16; ++e) s += c0[e] + x[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// 512-thread workgroups (two waves per SIMD; waves w and w + 4 share a SIMD):
// waves 0-3 run a dependent MFMA chain (it_mfma x 4 MFMAs), waves 4-7 run 16
// independent vector chains (it_valu x 16 ops; exp2 when EXP).
template <bool EXP>
__global__ __launch_bounds__(512) void mfma_and_valu_waves(float* out, int it_mfma, int it_valu) {
  float s = 0.f;
  if ((threadIdx.x >> 6) < 4) {
    u32x4 a, b;
    mfma_operands(a, b);
    f32x16 c0 = {};
    for (int it = 0; it < it_mfma; ++it) {
#pragma unroll
      for (int k = 0; k < 4; ++k) c0 = mfma(a, b, c0);
    }
    for (int e = 0; e < 16; ++e) s += c0[e];
  } else {
    float x[16];
    for (int i = 0; i < 16; ++i) x[i] = 0.001f * (threadIdx.x + i);
    for (int it = 0; it < it_valu; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (EXP) x[i] = __builtin_amdgcn_exp2f(x[i]);
        else x[i] = fmaf(x[i], 0.999f, 0.001f);
      }
    }
    for (int i = 0; i < 16; ++i) s += x[i];
  }
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

// ---- attnloop --------------------------------------------------------------
// 8 waves (two per SIMD), each repeating per 32-key half: 16 operand reads of
// 1 KB from LDS, S = 8 dependent 32x32x16 MFMAs, a softmax over S (max,
// exp2, bf16 packing, row sum) and 8 PV MFMAs into 4 accumulators: the
// multi-token kernel's operand bytes and MFMAs per half.  MODE bit 0: a
// barrier every 4 halves; bit 1: waves 4-7 start 8 MFMAs late; bit 2: no
// softmax (S packed as is); bit 3: no MFMAs (vector work only).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
template <int MODE>
__global__ __launch_bounds__(512) void attn_loop(float* out, int iters) {
  constexpr bool BAR = MODE & 1, OFF = MODE & 2, NOSM = MODE & 4, NOM = MODE & 8;
  __shared__ __attribute__((aligned(16))) u32x4 ops[2][16][64];   // two stages of 16 operands
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 2 * 16 * 64; i += 512) {
    const uint32_t x = i * 2654435761u;
    (&ops[0][0][0])[i] = u32x4{x, x * 3u, x * 5u, x * 7u} & 0x3c003c00u;   // small bf16 values
  }
  __syncthreads();
  u32x4 q[8];
  for (int k = 0; k < 8; ++k) q[k] = u32x4{lane * 3u + k, lane * 5u, lane * 7u, lane * 11u} & 0x3c003c00u;
  f32x16 o[4] = {};
  f32x16 dummy = {};
  float m = 0.f, l = 0.f;
  if (OFF && wv >= 4) {
#pragma unroll
    for (int k = 0; k < 8; ++k) dummy = mfma(q[k], q[7 - k], dummy);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it = 0; it < iters; ++it) {
    const int st = it & 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 kop[8], vop[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        kop[k] = ops[st][(k + u) & 15][lane];
        vop[k] = ops[st][(8 + k + u) & 15][lane ^ 32];
      }
      f32x16 s = {};
      if (!NOM) {
#pragma unroll
        for (int k = 0; k < 8; ++k) s = mfma(kop[k], q[k], s);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = __builtin_bit_cast(float, kop[e & 7][e >> 3]) * 1e-3f;
      }
      u32x4 pb[2];
      if (!NOSM) {
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mu = fmaxf(m, mx);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], 0.0883f, -mu));
        float rs = 0.f;
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pb[v2][w] = pack_bf16(s[8 * v2 + 2 * w], s[8 * v2 + 2 * w + 1]);
            rs += s[8 * v2 + 2 * w] + s[8 * v2 + 2 * w + 1];
          }
        l += rs;
        m = mu;
      } else {
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w) pb[v2][w] = __builtin_bit_cast(uint32_t, s[8 * v2 + 2 * w]) & 0x3c003c00u;
      }
      if (!NOM) {
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int t = 0; t < 4; ++t) o[t] = mfma(vop[4 * v2 + t], pb[v2], o[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t][0] += __builtin_bit_cast(float, pb[t & 1][t]);
      }
    }
    if (BAR) __syncthreads();
  }
  float r = m + l;
  for (int t = 0; t < 4; ++t)
    for (int e = 0; e < 16; ++e) r += o[t][e] + dummy[e];
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

// The same loop with the multi-token kernel's other parts switched on: 64 KB
// LDS stages (each half reads its own 16 operands), a barrier every 4 halves,
// and MODE bit 0: the kernel's softmax (a row max raised only past 2^8
// behind a wave-wide ballot and branch, cross-lane steps by permlane, row
// sums by v_dot2 over the packed probabilities unless bit 3 asks for fp32
// adds); bit 1: 8 16-byte global loads per thread per 4 halves from an
// L2-resident 2 MB buffer; bit 2: their stores into the other LDS stage.
template <int MODE>
__global__ __launch_bounds__(512) void attn_stage(const u32x4* __restrict__ src, float* out, int iters) {
  constexpr bool RS = MODE & 1, LD = MODE & 2, STO = MODE & 4, ADDS = MODE & 8;
  extern __shared__ __attribute__((aligned(16))) u32x4 ops[];   // 2 stages x 64 operands x 64 lanes
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  for (int i = tid; i < 2 * 64 * 64; i += 512) {
    const uint32_t x = i * 2654435761u;
    ops[i] = u32x4{x, x * 3u, x * 5u, x * 7u} & 0x3c003c00u;
  }
  __syncthreads();
  u32x4 q[8];
  for (int k = 0; k < 8; ++k) q[k] = u32x4{lane * 3u + k, lane * 5u, lane * 7u, lane * 11u} & 0x3c003c00u;
  f32x16 o[4] = {};
  float m_run = -INFINITY, l_run = 0.f;
  u32x4 buf[8];
  for (int j = 0; j < 8; ++j) buf[j] = u32x4{0, 0, 0, 0};
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  for (int it = 0; it < iters; ++it) {
    const int st = it & 1;
    const u32x4* stg = ops + st * 64 * 64;
    if (LD) {
#pragma unroll
      for (int j = 0; j < 8; ++j) buf[j] = src[((it & 31) * 8 + j) * 512 + tid] & 0x3c003c00u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x4 kop[8], vop[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        kop[k] = stg[(16 * u + k) * 64 + lane];
        vop[k] = stg[(16 * u + 8 + k) * 64 + lane];
      }
      f32x16 s = {};
#pragma unroll
      for (int k = 0; k < 8; ++k) s = mfma(kop[k], q[k], s);
      u32x4 pb[2];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      float rs = 0.f;
      if (RS) {
        const uint32_t mu = __float_as_uint(mx);
        const auto sw = __builtin_amdgcn_permlane32_swap(mu, mu, false, false);
        const float m_cand = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * 0.0883f;
        const bool raise = m_cand > m_run + 8.f;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float m_new = raise ? m_cand : m_run;
          const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < 4; ++t) o[t] *= alpha;
          m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], 0.0883f, -m_use));
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pb[v2][w] = pack_bf16(s[8 * v2 + 2 * w], s[8 * v2 + 2 * w + 1]);
            if (ADDS) rs += s[8 * v2 + 2 * w] + s[8 * v2 + 2 * w + 1];
            else rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb[v2][w]), one, rs, false);
          }
        const uint32_t ru = __float_as_uint(rs);
        const auto rw = __builtin_amdgcn_permlane32_swap(ru, ru, false, false);
        l_run += __uint_as_float(rw[0]) + __uint_as_float(rw[1]);
      } else {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mu = fmaxf(m_run, mx);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], 0.0883f, -mu));
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pb[v2][w] = pack_bf16(s[8 * v2 + 2 * w], s[8 * v2 + 2 * w + 1]);
            rs += s[8 * v2 + 2 * w] + s[8 * v2 + 2 * w + 1];
          }
        l_run += rs;
        m_run = mu;
      }
#pragma unroll
      for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = mfma(vop[4 * v2 + t], pb[v2], o[t]);
    }
    if (STO) {
      u32x4* dst = ops + (st ^ 1) * 64 * 64;
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j * 512 + tid] = buf[j];
    }
    __syncthreads();
  }
  float r = m_run + l_run;
  for (int t = 0; t < 4; ++t)
    for (int e = 0; e < 16; ++e) r += o[t][e];
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

struct Timer {
  hipEvent_t e0, e1;
  Timer() {
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
  }
  ~Timer() {
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  // Best of `reps` timed launches after one warm-up, in ms.
  template <typename F>
  float best(F launch, int reps = 5) {
    launch();
    (void)hipDeviceSynchronize();
    float b = 1e30f;
    for (int r = 0; r < reps; ++r) {
      (void)hipEventRecord(e0);
      launch();
      (void)hipEventRecord(e1);
      (void)hipEventSynchronize(e1);
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, e0, e1);
      if (ms < b) b = ms;
    }
    return b;
  }
};

int probe_read(int cus) {
  const size_t bytes = (size_t)4 << 30;
  u32x4* p;
  CK(hipMalloc(&p, bytes));
  CK(hipMemset(p, 1, bytes));
  const int max_grid = cus * 64;
  uint32_t* out;
  CK(hipMalloc(&out, sizeof(uint32_t) * 256 * (size_t)max_grid));
  Timer t;
  const size_t n = bytes / 16;
  auto seq = [&](const char* name, void (*k)(const u32x4*, size_t, uint32_t*), int grid) {
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, 0, p, n, out); });
    printf("read sequential %-28s grid %6d : %.3f ms  %.2f TB/s\n", name, grid, ms, bytes / (ms * 1e-3) / 1e12);
  };
  for (int g : {cus * 8, cus * 32}) {
    seq("16 B loads, 8 in flight", read_seq<8, false>, g);
    seq("16 B nt loads, 8 in flight", read_seq<8, true>, g);
  }
  const int grid = cus * 32, iters = 64;   // grid * iters * 8 KB = 4 GiB read
  const uint32_t nch = (uint32_t)(bytes / 4096);
  auto chunks = [&](const char* name, void (*k)(const u32x4*, uint32_t, int, uint32_t*)) {
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(grid), dim3(64), 0, 0, p, nch, iters, out); });
    const double rb = (double)grid * iters * 8192;
    printf("read random 4 KB chunks %-36s : %.3f ms  %.2f TB/s\n", name, ms, rb / (ms * 1e-3) / 1e12);
  };
  chunks("1 KB contiguous per load, nt", read_chunks<0, true>);
  chunks("16 rows x 64 B per load, nt", read_chunks<1, true>);
  chunks("1 KB contiguous per load", read_chunks<0, false>);
  chunks("16 rows x 64 B per load", read_chunks<1, false>);
  CK(hipFree(p));
  CK(hipFree(out));
  return 0;
}

int probe_lds(int cus) {
  uint32_t* out;
  CK(hipMalloc(&out, sizeof(uint32_t) * 1024 * (size_t)cus * 2));
  Timer t;
  const int iters = 4096;
  auto run = [&](void (*k)(uint32_t*, int), int waves, int wgs) {
    const int grid = cus * wgs;
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(grid), dim3(64 * waves), 0, 0, out, iters); });
    const double b = (double)grid * waves * iters * 16 * 1024;
    printf("lds ds_read_b128, %d workgroup(s) of %2d waves per CU (%2d waves/CU): %.3f ms, %.1f TB/s, "
           "%.1f B/clk/CU at 2.4 GHz\n", wgs, waves, waves * wgs, ms, b / (ms * 1e-3) / 1e12,
           b / (ms * 1e-3) / cus / kNominalHz);
  };
  run(lds_read<256>, 4, 1);
  run(lds_read<256>, 4, 2);
  run(lds_read<512>, 8, 1);
  run(lds_read<512>, 8, 2);
  run(lds_read<1024>, 16, 1);
  run(lds_read<1024>, 16, 2);
  CK(hipFree(out));
  return 0;
}

int probe_ldsmap(int cus) {
  uint32_t* out;
  CK(hipMalloc(&out, sizeof(uint32_t) * 512 * (size_t)cus * 2));
  Timer t;
  const int iters = 4096;
  const char* names[] = {"contiguous 1 KB", "rows, pitch 272 B", "permuted rows, pitch 272 B",
                         "rows, pitch 256 B", "rows, pitch 256 B, chunk ^ (r & 15)", "rows, pitch 264 B",
                         "rows, pitch 288 B", "permuted rows, pitch 256 B, chunk ^ (r & 15)",
                         "rows, pitch 256 B, chunk ^ ((r >> 1) & 15)", "permuted rows, pitch 288 B"};
  void (*kern[])(uint32_t*, int) = {lds_map_read<0>, lds_map_read<1>, lds_map_read<2>, lds_map_read<3>,
                                    lds_map_read<4>, lds_map_read<5>, lds_map_read<6>, lds_map_read<7>,
                                    lds_map_read<8>, lds_map_read<9>};
  for (int m = 0; m < 10; ++m) {
    for (int wgs : {1, 2}) {
      const int grid = cus * wgs;
      const float ms = t.best([&] { hipLaunchKernelGGL(kern[m], dim3(grid), dim3(512), 0, 0, out, iters); });
      const double b = (double)grid * 8 * iters * 16 * 1024;
      printf("ldsmap %-46s %2d waves/CU: %.1f B/clk/CU at 2.4 GHz\n", names[m], 8 * wgs,
             b / (ms * 1e-3) / cus / kNominalHz);
    }
  }
  CK(hipFree(out));
  return 0;
}

int probe_attnloop(int cus) {
  float* out;
  CK(hipMalloc(&out, sizeof(float) * 512 * (size_t)cus));
  Timer t;
  const int iters = 2000;
  auto run = [&](const char* name, void (*k)(float*, int)) {
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(cus), dim3(512), 0, 0, out, iters); });
    const double slots = 2.0 * iters * 4 * 16;   // MFMA slots per SIMD: 2 waves x halves x 16
    const double cyc = ms * 1e-3 * kNominalHz;
    printf("attnloop %-40s %.3f ms, %.1f nominal cycles per MFMA slot, %.2f of the 32-cycle MFMA rate\n", name, ms,
           cyc / slots, slots * 32 / cyc);
  };
  run("MFMAs + softmax", attn_loop<0>);
  run("MFMAs + softmax, barrier per 4 halves", attn_loop<1>);
  run("MFMAs + softmax, barrier, offset waves", attn_loop<3>);
  run("MFMAs + softmax, offset waves", attn_loop<2>);
  run("MFMAs only (operands from LDS)", attn_loop<4>);
  run("MFMAs only, barrier", attn_loop<5>);
  run("softmax only (operands from LDS)", attn_loop<8>);
  // The kernel's parts, with 64 KB stages and a barrier every 4 halves.
  u32x4* src;
  const size_t src_bytes = (size_t)32 * 8 * 512 * 16;   // 2 MB, stays in L2
  CK(hipMalloc(&src, src_bytes));
  CK(hipMemset(src, 0, src_bytes));
  const size_t lds = 2 * 64 * 64 * 16;
  auto run2 = [&](const char* name, void (*k)(const u32x4*, float*, int)) -> int {
    CK(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(cus), dim3(512), lds, 0, src, out, iters); });
    const double slots = 2.0 * iters * 4 * 16;
    const double cyc = ms * 1e-3 * kNominalHz;
    printf("attnloop %-40s %.3f ms, %.1f nominal cycles per MFMA slot, %.2f of the 32-cycle MFMA rate\n", name, ms,
           cyc / slots, slots * 32 / cyc);
    return 0;
  };
  if (run2("64 KB stages, simple softmax", attn_stage<0>)) return 1;
  if (run2("+ kernel softmax (dot2 row sums)", attn_stage<1>)) return 1;
  if (run2("+ kernel softmax (fp32 row sums)", attn_stage<1 | 8>)) return 1;
  if (run2("+ tile loads", attn_stage<2>)) return 1;
  if (run2("+ tile loads and LDS stores", attn_stage<2 | 4>)) return 1;
  if (run2("+ LDS stores only", attn_stage<4>)) return 1;
  if (run2("+ kernel softmax (fp32), loads, stores", attn_stage<1 | 2 | 4 | 8>)) return 1;
  CK(hipFree(src));
  CK(hipFree(out));
  return 0;
}

int probe_mfma(int cus) {
  float* out;
  CK(hipMalloc(&out, sizeof(float) * 512 * (size_t)cus));
  Timer t;
  const int iters = 20000;
  auto one_wave = [&](const char* name, void (*k)(float*, int)) {
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(cus), dim3(256), 0, 0, out, iters); });
    printf("one wave per SIMD, MFMA chain %-22s : %.1f cycles per MFMA at 2.4 GHz (%.0f TFLOP/s)\n", name,
           ms * 1e-3 * kNominalHz / (iters * 4.0), (double)cus * 4 * iters * 4 * 32768.0 / (ms * 1e-3) / 1e12);
  };
  one_wave("alone", mfma_then_valu<0, false>);
  one_wave("+ 4 fma per MFMA", mfma_then_valu<4, false>);
  one_wave("+ 8 fma per MFMA", mfma_then_valu<8, false>);
  one_wave("+ 16 fma per MFMA", mfma_then_valu<16, false>);
  one_wave("+ 2 exp2 per MFMA", mfma_then_valu<2, true>);
  one_wave("+ 8 exp2 per MFMA", mfma_then_valu<8, true>);
  auto two_waves = [&](const char* name, void (*k)(float*, int, int), int im, int iv) {
    const float ms = t.best([&] { hipLaunchKernelGGL(k, dim3(cus), dim3(512), 0, 0, out, im, iv); });
    printf("two waves per SIMD, %-44s : %.3f ms\n", name, ms);
  };
  two_waves("MFMA wave alone (40K MFMAs)", mfma_and_valu_waves<false>, 10000, 0);
  two_waves("fma wave alone (160K fma)", mfma_and_valu_waves<false>, 0, 10000);
  two_waves("exp2 wave alone (160K exp2)", mfma_and_valu_waves<true>, 0, 10000);
  two_waves("MFMA wave beside fma wave", mfma_and_valu_waves<false>, 10000, 10000);
  two_waves("MFMA wave beside exp2 wave", mfma_and_valu_waves<true>, 10000, 10000);
  CK(hipFree(out));
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "";
  hipDeviceProp_t prop;
  CK(hipGetDeviceProperties(&prop, 0));
  printf("device %s, %d CUs, clock %d kHz\n", prop.name, prop.multiProcessorCount, prop.clockRate);
  if (!strcmp(mode, "read")) return probe_read(prop.multiProcessorCount);
  if (!strcmp(mode, "lds")) return probe_lds(prop.multiProcessorCount);
  if (!strcmp(mode, "mfma")) return probe_mfma(prop.multiProcessorCount);
  if (!strcmp(mode, "ldsmap")) return probe_ldsmap(prop.multiProcessorCount);
  if (!strcmp(mode, "attnloop")) return probe_attnloop(prop.multiProcessorCount);
  fprintf(stderr, "usage: %s read|lds|ldsmap|mfma|attnloop\n", argv[0]);
  return 2;
}
