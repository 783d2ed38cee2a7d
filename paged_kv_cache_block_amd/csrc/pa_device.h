// Device helpers shared by the gfx950 kernels of libpagedattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct Elt;
template <> struct Elt<DT_F32> { static constexpr int bytes = 4; using store_t = uint32_t; };
template <> struct Elt<DT_F16> { static constexpr int bytes = 2; using store_t = uint16_t; };
template <> struct Elt<DT_BF16> { static constexpr int bytes = 2; using store_t = uint16_t; };

constexpr float kLog2e = 1.4426950408889634f;

// ---- element <-> float ----------------------------------------------------
template <int DT> __device__ __forceinline__ float lo_to_float(uint32_t w);
template <int DT> __device__ __forceinline__ float hi_to_float(uint32_t w);

template <> __device__ __forceinline__ float lo_to_float<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi_to_float<DT_F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <> __device__ __forceinline__ float lo_to_float<DT_BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <> __device__ __forceinline__ float hi_to_float<DT_BF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Unpack 4 bytes-per-word storage into floats: N words -> N (f32) or 2N values.
template <int DT, int NW>
__device__ __forceinline__ void unpack(const uint32_t (&w)[NW], float* out) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < NW; ++i) out[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      out[2 * i] = lo_to_float<DT>(w[i]);
      out[2 * i + 1] = hi_to_float<DT>(w[i]);
    }
  }
}

// float -> storage bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32: RNE
}
template <int DT> __device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == DT_F16)
    return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
  else
    return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// ---- wave reductions ------------------------------------------------------
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Logical work index of workgroup `bid` of an n-workgroup 1-D grid.  The
// dispatcher hands workgroups to the 8 XCDs round-robin; this numbering gives
// each XCD one contiguous range of logical indices, so work items that read
// the same K/V (consecutive logical indices) share that XCD's L2.
__device__ __forceinline__ int xcd_order(int bid, int n) {
  const int xcd = bid & 7, pos = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + min(xcd, rem) + pos;
}

// x and its copy in lane l ^ M (M = 16 or 32), by v_permlane16_swap /
// v_permlane32_swap: a VALU op, where a shuffle would be an LDS round trip.
// Each lane receives its own value in one result and its partner's in the
// other, so a symmetric combine of the two needs no select.
template <int M>
__device__ __forceinline__ void xor_pair(float x, float& p, float& q) {
  static_assert(M == 16 || M == 32, "lane distance");
  const uint32_t u = __float_as_uint(x);
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    p = __uint_as_float(r[0]);
    q = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    p = __uint_as_float(r[0]);
    q = __uint_as_float(r[1]);
  }
}
template <int M> __device__ __forceinline__ float xor_max(float x) {
  float p, q;
  xor_pair<M>(x, p, q);
  return fmaxf(p, q);
}
template <int M> __device__ __forceinline__ float xor_sum(float x) {
  float p, q;
  xor_pair<M>(x, p, q);
  return p + q;
}

// ---- workspace plan records ------------------------------------------------
// One vector-ALU work item: a query row (seq, i) and one split of its keys.
struct RowItem {
  int32_t seq;
  int32_t i;       // row index within the sequence's new tokens
  int32_t split;   // split index
  int32_t pslot;   // first partial slot of the row, or -1 if it has one split
};
// One MFMA work item: a tile of packed (token, head) rows of one sequence,
// and one split of its keys.
struct TileItem {
  int32_t seq;
  int32_t tile;
  int32_t split;   // key split index
  int32_t pslot;   // partial slot of the sequence's first token, or -1 (keys not split)
};
// One combine item: a row whose splits must be merged.
struct CombItem {
  int32_t row;     // global query row
  int32_t pslot;
  int32_t nsplit;
  int32_t seq;
};
// Written by the planner at the start of every attention call.  `mismatch`
// is nonzero when the work the device derives from context_lens /
// query_start_loc differs from what the host derived from their mirrors (the
// grids were sized from the latter); `dropped` is set by any kernel that had
// to skip work because an index left the batch or the workspace.
struct PlanCounts {
  int32_t rows, tiles, combs, partials;
  int32_t mismatch, dropped;
};

}  // namespace pa

namespace pa {

// Work a sequence contributes to the plan.  The host (for launch sizes) and
// the plan kernel (for the item lists) both call this, so they agree.
struct SeqWork {
  int32_t row_first;  // first row index that goes to the row kernel
  int32_t rows;       // rows that go to the row kernel
  int32_t tiles;      // MFMA tiles
};

__host__ __device__ inline SeqWork seq_work(int n, int vector_all, int group, int tile_rows) {
  SeqWork w{0, 0, 0};
  if (n <= 0) return w;
  if (vector_all || n == 1) {
    w.rows = n;
  } else {
    w.tiles = (n * group + tile_rows - 1) / tile_rows;
  }
  return w;
}

// Splits of a row whose causal limit admits `keys` keys.
__host__ __device__ inline int row_splits(int keys, int split_tokens) {
  if (keys <= split_tokens) return 1;
  return (keys + split_tokens - 1) / split_tokens;
}

// Key splits of the multi-token path: split k covers keys
// [k * split_tokens, (k + 1) * split_tokens); split_tokens = 0 means one.
__host__ __device__ inline int key_splits(int keys, int split_tokens) {
  if (split_tokens <= 0 || keys <= split_tokens) return 1;
  return (keys + split_tokens - 1) / split_tokens;
}

// Keys visible to tile t of a sequence with n new tokens and context L
// (exclusive end: one past the causal limit of the tile's last row).
__host__ __device__ inline int tile_key_end(int n, int L, int group, int tile_rows, int t) {
  const int R = n * group;
  const int last = (t + 1) * tile_rows < R ? (t + 1) * tile_rows : R;
  return L - n + (last - 1) / group + 1;
}

// Multi-token work of one sequence under a key split: tile items (one per
// tile and split that holds a key of the tile), tokens whose splits need a
// combine, and partial slots (n x splits of the whole context, token-major).
struct TileWork {
  int32_t items, combs, slots;
};
__host__ __device__ inline TileWork tile_work(int n, int L, int group, int tile_rows, int tiles,
                                              int split_tokens) {
  TileWork w{0, 0, 0};
  if (tiles == 0) return w;
  const int ns = key_splits(L, split_tokens);
  if (ns == 1) {
    w.items = tiles;
    return w;
  }
  for (int t = 0; t < tiles; ++t)
    w.items += key_splits(tile_key_end(n, L, group, tile_rows, t), split_tokens);
  // Token i sees L - n + i + 1 keys: more than one split from i0 on.
  const int i0 = split_tokens - (L - n) > 0 ? split_tokens - (L - n) : 0;
  w.combs = n > i0 ? n - i0 : 0;
  w.slots = n * ns;
  return w;
}

}  // namespace pa
