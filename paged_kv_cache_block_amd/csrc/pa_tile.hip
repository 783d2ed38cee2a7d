// MFMA multi-token paged attention (gfx950, fp16 / bf16).
//
// Pensieve page (多Token注意力内核运算原理, figure 9): with several new tokens
// per request the work is two matrix-matrix products over a context whose
// blocks sit at random physical places; Q is ragged across requests.
// (融合因果掩码与内核实现): the causal mask is applied inside the kernel and
// the score matrix is never materialised.
//
// Work item: one sequence, one KV head and a tile of 32 * NW packed rows
// (NW = 4 or 8 wavefronts of 32 rows), where row r is (new token r / G,
// query head g*G + r % G); all G query heads of a KV head share each K/V
// tile.
//
// Keys go 64 (4 waves) or 128 (8 waves) per iteration through a two-stage
// LDS ring fed from registers: while the waves compute on one stage, the
// next tile waits in registers for the other stage (with 64-key tiles the
// tile after it is in flight as well); one barrier per iteration.  Each wave
// computes, per 32-key half, with v_mfma_f32_32x32x16_{f16,bf16}:
//   S^T[key][row] = K[key][:] . Q[row][:]           (D/16 MFMAs)
//   online softmax per row (a row is one lane column of S^T, split over the
//   two lane halves), causal mask from absolute key positions
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]      (D/32 x 2 MFMAs)
// Working on the transposes keeps each row's statistics inside a lane pair
// and lets both operands of the second product be read as 16-byte runs.
// The K rows feeding S^T are permuted so that the eight keys a lane holds for
// each P^T operand are consecutive, which is what the V^T operand reads.
// The running max is only raised (and O rescaled) when a row's max grows by
// more than 2^8, so most iterations skip the rescale.  The LDS operands of a
// half are read before its softmax, so their latency hides behind it.
// Work items come longest first from the plan, and workgroups are numbered
// so that each XCD gets an even share of them (see the item mapping below).

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Key (within a 32-key half tile) held by accumulator element e of lane half hh.
constexpr __host__ __device__ int acc_key(int e, int hh) { return 16 * (e >> 3) + 8 * hh + (e & 7); }

// Key whose K row is loaded as row r of the S^T product.  Row r of a 32x32
// accumulator lands in element 4*(r>>3) + (r&3) of lane half (r>>2)&1; this
// map sends it to acc_key of that element.
constexpr __host__ __device__ int row_key(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}
constexpr bool row_key_matches_acc_key() {
  for (int r = 0; r < 32; ++r)
    if (row_key(r) != acc_key(4 * (r >> 3) + (r & 3), (r >> 2) & 1)) return false;
  return true;
}
static_assert(row_key_matches_acc_key(), "K row order must match the accumulator layout");

// NW = waves per workgroup (4 or 8), 32 rows each: the K/V tile staged in
// LDS serves 32 * NW rows, so larger workgroups issue fewer loads and LDS
// stores per MFMA.  Two waves per SIMD either way.
template <int DT, int D, int BS, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void tile_attn_kernel(AttnArgs a, PoolArgs p,
                                                                   WorkspaceLayout lay, int num_tiles) {
  constexpr int NT = 64 * NW;       // threads per workgroup
  constexpr int KS = D / 16;        // k-steps of the QK product
  constexpr int NDT = D / 32;       // 32-row head-dim tiles of O^T
  // Keys per iteration: 128 for 8 waves (one register set of loads in
  // flight), 64 for 4 waves (two sets).
  constexpr int kKeys = NW == 8 ? 128 : 64;
  constexpr int NH = kKeys / 32;    // 32-key halves per tile
  constexpr int KCH = kKeys * D / 8 / NT;    // 16-byte K chunks per thread per tile
  constexpr int VCH = D * kKeys / 8 / NT;    // 16-byte V chunks per thread per tile
  // LDS holds each tile in MFMA operand order: one 16-byte slot per lane, a
  // "run" of 32 slots per lane half, so that an operand read is two
  // contiguous 512-byte runs (one base address per lane plus an immediate).
  // Run r of K is (32-key half u, k-step ks, lane half hh) with
  // r = 2 (u KS + ks) + hh; run r of V^T is (u, head-dim tile t, k-step v2,
  // hh) with r = 4 (u NDT + t) + 2 v2 + hh.  The LDS takes a 16-byte store 8
  // lanes at a time into a 128-byte window of banks (the bank-conflict counter
  // shows it: pitches that spread 16 lanes over 256 bytes left the V stores
  // 2-way conflicted), so the run pitch carries p extra slots that send each
  // 8-lane group of a tile store to 8 distinct 16-byte bank groups: K lanes
  // hold 8 chunks of one key row (pitch = 16 bytes mod 128: p = 1), V lanes 4
  // key chunks x 2 head-dim rows (pitch = 32 bytes mod 128: p = 2).  Reads
  // are 16 consecutive slots per quarter wave, conflict-free with any pitch.
  constexpr int KRUN = 8 * (32 + 1);   // K run pitch (elements)
  constexpr int VRUN = 8 * (32 + 2);   // V^T run pitch (elements)
  constexpr int KSTAGE = 2 * NH * KS * KRUN;
  constexpr int VSTAGE = 4 * NH * NDT * VRUN;
  constexpr int TROWS = 32 * NW;    // rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * KSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * VSTAGE];
  __shared__ unsigned btab[kTabWin];

  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const PlanCounts* pc = reinterpret_cast<const PlanCounts*>(ws + lay.counts);
  const int Hkv = p.num_kv_heads;
  // The plan lists work items longest first.  With a multiple of 8 KV heads,
  // each XCD takes whole heads (their lists are alike, so the XCDs' shares
  // are too), so that the tiles sharing one (sequence, head) meet in its L2,
  // and runs them item-major over its heads: its workgroups start in list
  // order, longest first.  (The dispatcher hands workgroup b to XCD b % 8.)
  // Otherwise the list goes round-robin over the XCDs, item by item, so that
  // each gets long and short items.
  int g, item;
  if (Hkv % 8 == 0) {
    const int hpx = Hkv >> 3;                  // KV heads per XCD
    const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
    item = pos / hpx;
    g = xcd * hpx + (pos - item * hpx);
  } else {
    item = blockIdx.x / Hkv;
    g = blockIdx.x - item * Hkv;
  }
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
  const int r0 = ti.tile * TROWS;
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks;
  const unsigned nb_max = p.num_blocks - 1;
  const int tb_max = a.max_blocks - 1;
  const float c = a.scale_log2;

  // This lane's row.
  const int wr0 = r0 + 32 * wv;               // first row of the wave
  const int r = wr0 + col;
  const bool row_ok = r < R && q0 + r / G < a.total_q;
  if (r < R && !row_ok) mark_dropped(a.ws, lay);   // rows past total_q: the batch disagrees
  const int qi = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  const int p_row = row_ok ? L - n + qi : -1;
  // Key ranges: the workgroup's and this wave's (rows ascend, so the last
  // row of a range has the largest causal limit, the first the smallest).
  const int kend = L - n + (min(R, r0 + TROWS) - 1) / G + 1;
  // Keys of this item: the whole causal range, or one split of it.
  const int S = a.prefill_split;
  const int k0 = ti.pslot < 0 ? 0 : ti.split * S;
  const int k1 = ti.pslot < 0 ? kend : min(kend, k0 + S);
  const bool wave_on = wr0 < R;
  const bool wave_full = wr0 + 32 <= R;
  const int wfirst = wave_on ? L - n + wr0 / G : 0;

  // Q^T operands of the QK product: lane (col, hh) holds Q[row][16ks+8hh .. +8].
  u32x4 qreg[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)(q0 + qi) * Hq + hq) * D + 8 * hh;
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
  // head-dim chunk kdc.  V chunk j is head-dim row 4 (vdg + VDP j) + (tid>>2 & 3),
  // keys kt0 + vkey .. +8 with vkey = 32 (vgrp % NH) + 8 (tid & 3): four lanes
  // read 64 contiguous bytes of a row.  Offsets are within a block's
  // (block, head) slice.
  constexpr int TPR = D / 8;            // 16-byte chunks per K row
  constexpr int KRP = NT / TPR;         // K rows per pass of the workgroup
  constexpr int VDP = NT / 16 / NH;     // 4-row head-dim groups per pass
  const int ktok = tid / TPR;
  const int kdc = tid % TPR;
  const int vgrp = tid >> 4;
  const int vd = 4 * (vgrp / NH) + ((tid >> 2) & 3);
  const int vkey = 32 * (vgrp % NH) + 8 * (tid & 3);
  const uint64_t kstride = (uint64_t)Hkv * BS * D;     // elements per physical block
  int kofs[KCH];
#pragma unroll
  for (int j = 0; j < KCH; ++j) kofs[j] = ((g * BS + (ktok + KRP * j) % BS) * D) + kdc * 8;
  int vofs[VCH];
#pragma unroll
  for (int j = 0; j < VCH; ++j) vofs[j] = ((g * D + vd + 4 * VDP * j) * BS) + vkey % BS;

  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache);
  // One tile's K/V chunks of this thread, held in registers between the
  // global load and the LDS store.
  struct Buf {
    u32x4 k[KCH], v[VCH];
  };

  // The sequence's block ids, kTabWin at a time, clamped to the pool (so
  // every load below stays inside it).  A tile never straddles two windows
  // (kTabWin is a multiple of kKeys / BS).
  int win = -1;
  auto ensure_window = [&](int kt) {
    const int w = (kt * kKeys / BS) / kTabWin;
    if (w == win) return;
    __syncthreads();
    for (int i = tid; i < kTabWin; i += NT)
      btab[i] = min((unsigned)bt[min(w * kTabWin + i, tb_max)], nb_max);
    __syncthreads();
    win = w;
  };
  auto load_tile = [&](Buf& b, int kt) {
    ensure_window(kt);
    const int kt0 = kt * kKeys;
    const int b0 = kt0 / BS - win * kTabWin;
    const int kin = kt0 % BS;          // tile start inside its block (blocks larger than a tile)
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const unsigned blk = btab[b0 + (ktok + KRP * j) / BS];
      b.k[j] = *reinterpret_cast<const u32x4*>(kc + blk * kstride + kofs[j] + kin * D);
    }
    const unsigned vblk = btab[b0 + vkey / BS];
#pragma unroll
    for (int j = 0; j < VCH; ++j)
      b.v[j] = *reinterpret_cast<const u32x4*>(vc + vblk * kstride + vofs[j] + kin);
  };
  // Tail tile: slots at or past kend may be unwritten (NaN).  Zero the V
  // entries (a zero probability must not meet them); K rows there are masked
  // to -inf before the softmax.  Runs just before the tile is stored.
  auto zero_tail = [&](Buf& b, int kt) {
    const int kt0 = kt * kKeys;
    if (kt0 + kKeys > kend) {
      asm volatile("" ::: "memory");   // keep this a real branch, not selects
#pragma unroll
      for (int j = 0; j < VCH; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x = b.v[j][w];
          if (kt0 + vkey + 2 * w >= kend) x &= 0xffff0000u;
          if (kt0 + vkey + 2 * w + 1 >= kend) x &= 0x0000ffffu;
          b.v[j][w] = x;
        }
    }
  };
  // Operand-order slots of this thread's chunks (see KRUN / VRUN).  Key
  // ktok + KRP j sits at a fixed offset from key ktok's slot: KRP is 16
  // (then ktok < 16 and row_key adds 16 to it) or a multiple of 32; the
  // head-dim rows of V chunk j step by 4 VDP = 32.
  static_assert(KRP == 16 || KRP % 32 == 0, "K rows per pass");
  static_assert(4 * VDP == 32, "V^T rows per pass");
  const int kslot = (2 * KS * (ktok >> 5) + kdc) * KRUN + 8 * row_key(ktok & 31);
  const int vslot = (4 * NDT * (vkey >> 5) + ((vkey >> 3) & 3) + 4 * (vd >> 5)) * VRUN + 8 * (vd & 31);
  auto store_tile = [&](const Buf& b, int stage) {
    uint16_t* kd = Ks + stage * KSTAGE + kslot;
    uint16_t* vd_ = Vs + stage * VSTAGE + vslot;
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      *reinterpret_cast<u32x4*>(kd + 2 * KS * KRUN * ((KRP * j) >> 5) + 8 * ((KRP * j) & 31)) = b.k[j];
#pragma unroll
    for (int j = 0; j < VCH; ++j) *reinterpret_cast<u32x4*>(vd_ + 4 * VRUN * j) = b.v[j];
  };

  const int kt_first = k0 / kKeys;                 // splits are whole tiles
  const int kt_end = (k1 + kKeys - 1) / kKeys;
  const int wend = wave_on ? L - n + (min(R, wr0 + 32) - 1) / G + 1 : 0;
  // LDS operand reads of one 32-key half: K rows for S^T, V^T rows for O^T.
  // They are issued ahead of the MFMAs that consume them (the V^T of a half
  // and the K of the next half before the half's softmax), so their latency
  // hides behind that vector work.
  // Lane (col, hh) of a K operand holds key 32u + row_key(col): the store
  // put key 32u + k at slot row_key(k), and row_key is its own inverse.
  const int klane = hh * KRUN + 8 * col;
  const int vlane = hh * VRUN + 8 * col;
  auto read_k = [&](const uint16_t* ks_, int u, u32x4 (&kop)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kop[ks] = *reinterpret_cast<const u32x4*>(&ks_[klane + 2 * (u * KS + ks) * KRUN]);
  };
  auto read_v = [&](const uint16_t* vs_, int u, u32x4 (&vop)[NDT][2]) {
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int v2 = 0; v2 < 2; ++v2)
        vop[t][v2] = *reinterpret_cast<const u32x4*>(&vs_[vlane + (4 * (u * NDT + t) + 2 * v2) * VRUN]);
  };
  auto compute = [&](int kt, int stage) {
    const int kt0 = kt * kKeys;
    if (wave_on && kt0 < wend) {
      const uint16_t* ks_ = Ks + stage * KSTAGE;
      const uint16_t* vs_ = Vs + stage * VSTAGE;
      // One 32-key half at a time: S^T = K . Q^T, causal mask, online
      // softmax, O^T += V^T . P^T.
      const bool need_mask = !wave_full || kt0 + kKeys - 1 > wfirst;
      u32x4 kop[KS];
      read_k(ks_, 0, kop);
#pragma unroll
      for (int u = 0; u < NH; ++u) {
        if (u > 0 && NW != 8) read_k(ks_, u, kop);
        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32<DT>(kop[ks], qreg[ks], sacc);
        u32x4 vop[NDT][2];
        read_v(vs_, u, vop);
        // (With 4-wave workgroups the register sets of the tile loads leave
        // no room to hold the next half's K as well.)
        if (u + 1 < NH && NW == 8) read_k(ks_, u + 1, kop);
        // Causal mask (a select), only where some key passes some row's limit.
        if (need_mask) {
          const int lim = p_row - kt0 - 32 * u - 8 * hh;   // key kt0 + 32u + 16(e>>3) + 8hh + (e&7)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (16 * (e >> 3) + (e & 7) > lim) sacc[e] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
        const float m_cand = xor_max<32>(mx) * c;
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
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = fast_exp2(fmaf(sacc[e], c, -m_use));
        u32x4 pb[2];
        float rs = 0.f;
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            pb[v2][w] = cvt2<DT>(sacc[8 * v2 + 2 * w], sacc[8 * v2 + 2 * w + 1]);
            // Row sum of the fp32 probabilities (their rounding to the MFMA
            // operand type is unbiased; a v_dot2 sum of the rounded pairs
            // measured slower).
            rs += sacc[8 * v2 + 2 * w] + sacc[8 * v2 + 2 * w + 1];
          }
        l_run += xor_sum<32>(rs);
        // O^T += V^T . P^T over the half's 2 k-steps of 16 keys, the
        // independent accumulators back to back.
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2)
#pragma unroll
          for (int t = 0; t < NDT; ++t) o[t] = mfma32<DT>(vop[t][v2], pb[v2], o[t]);
      }
    }
  };

  // Two LDS stages: while tile kt is computed from one stage, tile kt+1
  // waits in registers for the other.  With 64-key tiles a second register
  // set keeps tile kt+2 in flight as well, so every load has two 64-key
  // iterations to arrive; a 128-key iteration is long enough on its own.
  // Past the last tile, loads and stores repeat the last tile into an idle
  // stage.
  const int last = kt_end - 1;
  if constexpr (NW == 8) {
    Buf ba;
    load_tile(ba, kt_first);
    zero_tail(ba, kt_first);
    store_tile(ba, 0);
    load_tile(ba, min(kt_first + 1, last));
    __syncthreads();
    for (int kt = kt_first; kt < kt_end; kt += 2) {
      compute(kt, 0);
      zero_tail(ba, min(kt + 1, last));
      store_tile(ba, 1);
      load_tile(ba, min(kt + 2, last));
      __syncthreads();
      if (kt + 1 >= kt_end) break;
      compute(kt + 1, 1);
      zero_tail(ba, min(kt + 2, last));
      store_tile(ba, 0);
      load_tile(ba, min(kt + 3, last));
      __syncthreads();
    }
  } else {
    Buf ba, bb;
    load_tile(ba, kt_first);
    zero_tail(ba, kt_first);
    store_tile(ba, 0);
    load_tile(ba, min(kt_first + 1, last));
    load_tile(bb, min(kt_first + 2, last));
    __syncthreads();
    for (int kt = kt_first; kt < kt_end; kt += 2) {
      compute(kt, 0);
      zero_tail(ba, min(kt + 1, last));
      store_tile(ba, 1);
      load_tile(ba, min(kt + 3, last));
      __syncthreads();
      if (kt + 1 >= kt_end) break;
      compute(kt + 1, 1);
      zero_tail(bb, min(kt + 2, last));
      store_tile(bb, 0);
      load_tile(bb, min(kt + 4, last));
      __syncthreads();
    }
  }

  if (!row_ok) return;
  const int ns_row = ti.pslot < 0 ? 1 : key_splits(p_row + 1, S);
  if (ns_row == 1) {
    // All of this row's keys are in split 0: normalise and store.
    if (ti.split != 0) return;
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
    return;
  }
  // The row's partial state over this split (none if no key of the row is
  // in it); the combine kernel merges the splits.
  if (p_row < k0) return;
  const int64_t slot = (int64_t)ti.pslot + (int64_t)qi * key_splits(L, S) + ti.split;
  if (slot >= lay.cap_partials) {
    mark_dropped(a.ws, lay);
    return;
  }
  float* po = reinterpret_cast<float*>(const_cast<uint8_t*>(ws) + lay.part_o) + (slot * Hq + hq) * D;
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
      *reinterpret_cast<float4*>(po + 32 * t + 8 * a4 + 4 * hh) =
          make_float4(o[t][4 * a4], o[t][4 * a4 + 1], o[t][4 * a4 + 2], o[t][4 * a4 + 3]);
  if (hh == 0) {
    float2* pm = reinterpret_cast<float2*>(const_cast<uint8_t*>(ws) + lay.part_ml);
    pm[slot * Hq + hq] = make_float2(m_run, l_run);
  }
}

template <int DT, int D, int NW>
hipError_t launch_tile_d(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                         int num_tiles, hipStream_t s) {
  const dim3 grid(num_tiles * p.num_kv_heads);
  if (p.block_size == 16)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 16, NW>), grid, dim3(64 * NW), 0, s, a, p, lay, num_tiles);
  else if (p.block_size == 32)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 32, NW>), grid, dim3(64 * NW), 0, s, a, p, lay, num_tiles);
  else if (p.block_size == 64)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 64, NW>), grid, dim3(64 * NW), 0, s, a, p, lay, num_tiles);
  else if (p.block_size == 128)
    hipLaunchKernelGGL((tile_attn_kernel<DT, D, 128, NW>), grid, dim3(64 * NW), 0, s, a, p, lay, num_tiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_tile_cb(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                          int num_tiles, int tile_rows, hipStream_t s) {
  if (tile_rows == 128) return launch_tile_d<DT, D, 4>(a, p, lay, num_tiles, s);
  if (tile_rows == 256) return launch_tile_d<DT, D, 8>(a, p, lay, num_tiles, s);
  return hipErrorInvalidValue;
}

}  // namespace

bool tile_path_supported(const PoolArgs& p) {
  return (p.dtype == DT_F16 || p.dtype == DT_BF16) && (p.block_size == 16 || p.block_size == 32 || p.block_size == 64 || p.block_size == 128) &&
         (p.head_dim == 64 || p.head_dim == 128);
}

hipError_t launch_tile_attention(const AttnArgs& a, const PoolArgs& p, const WorkspaceLayout& lay,
                                 int num_tiles, int tile_rows, hipStream_t s) {
  if (num_tiles == 0) return hipSuccess;
  if ((int64_t)num_tiles * p.num_kv_heads > 0x7fffffff) return hipErrorInvalidValue;
  if (p.dtype == DT_F16) {
    if (p.head_dim == 64) return launch_tile_cb<DT_F16, 64>(a, p, lay, num_tiles, tile_rows, s);
    if (p.head_dim == 128) return launch_tile_cb<DT_F16, 128>(a, p, lay, num_tiles, tile_rows, s);
  } else if (p.dtype == DT_BF16) {
    if (p.head_dim == 64) return launch_tile_cb<DT_BF16, 64>(a, p, lay, num_tiles, tile_rows, s);
    if (p.head_dim == 128) return launch_tile_cb<DT_BF16, 128>(a, p, lay, num_tiles, tile_rows, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
