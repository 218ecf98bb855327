// ufp4_quant.hip -- the fused RHT + 4-bit quantization kernels for gfx950.
//
// Two phases per call (the per-tensor scale makes every code depend on the
// absolute maximum of the whole transformed tensor):
//   phase A (ufp4_amax_kernel): load each tile, transform its row-wise and
//     column-wise blocks and write the tile's largest magnitudes to the
//     workspace (no atomics, no fences);
//   phase B (ufp4_quant_kernel): reduce the partials of its segment into the
//     per-tensor scales S_t = amax / (Qmax * 448), reload the tile, transform
//     again, compute the block scales, round and store packed codes and
//     scales for both layouts from the same registers
//     ([Z] "Key points": fused RHT+quantization, uniform E1M2 grid;
//     [A] "The UFP4 Recipe": E1M2 or INT4, SR only where requested; the
//     two-level NVFP4-style scale is named in [H] technical approach).
//
// Mapping.  A lane holds a 16-row x 8-column sub-tile (one 16-byte load per
// row).  Row-wise blocks (16 consecutive columns) span a lane pair: stages of
// half-width 1, 2, 4 run in-lane, the stage of half-width 8 pairs lanes l and
// l^1 through a DPP quad permutation.  Column-wise blocks (16 consecutive
// rows) are entirely in-lane.  No LDS transpose is needed: the same loaded
// registers feed both layouts.  Workgroups are remapped so that the ones
// dispatched to one XCD (round-robin over 8) walk down one column band, so
// the transposed outputs they write share L2 lines.
#include <hip/hip_ext.h>

#include "ufp4_internal.hpp"

namespace ufp4 {


struct TileInfo {
  bool active;
  bool bad;
  int32_t work;  // band * n_tiles + row tile: the tile's partial slot
  int32_t band;
  int32_t seg;
  int64_t m0;        // first local row of the tile inside its segment
  int64_t seg_row0;  // global first row of the segment
  int64_t M;         // rows of the segment
  int64_t P;         // rows rounded up to the block (column-wise length)
  int64_t coff;      // column-wise output offset of the segment
};

struct GroupLds {
  int64_t off[kMaxGroups + 1];
  int64_t ppre[kMaxGroups + 1];  // prefix of padded rows
  int32_t tpre[kMaxGroups + 1];  // prefix of row tiles
  int64_t runp[kThreads];        // scan of the threads' runs
  int32_t runt[kThreads];
  int32_t bad;
  int32_t seg;
};

__device__ __forceinline__ int32_t remap_xcd(int32_t b, int32_t nblocks) {
  // nblocks is a multiple of kNumXcd: workgroup b runs on XCD b % 8.
  const int32_t per = nblocks / kNumXcd;
  return (b % kNumXcd) * per + b / kNumXcd;
}

// Tile of work index w of a dense tensor.
__device__ __forceinline__ TileInfo dense_tile(const QuantParams& p, int32_t w) {
  TileInfo T;
  T.bad = false;
  T.work = w;
  T.active = w >= 0 && w < p.n_work;
  T.band = T.active ? w / p.n_tiles : 0;
  const int32_t t = T.active ? w % p.n_tiles : 0;
  T.seg = 0;
  T.seg_row0 = 0;
  T.M = p.rows;
  T.P = (p.rows + p.block - 1) / p.block * p.block;
  T.coff = 0;
  T.m0 = (int64_t)t * kTileRows;
  T.active = T.active && T.m0 < T.P;
  return T;
}

// Resolve the workgroup's tile.  For grouped calls every workgroup scans the
// offsets (at most kMaxGroups+1 values) into LDS and validates them.
__device__ __forceinline__ TileInfo tile_info(const QuantParams& p, GroupLds& g) {
  TileInfo T;
  T.bad = false;
  const int32_t w = remap_xcd((int32_t)blockIdx.x, (int32_t)gridDim.x);
  T.active = w < p.n_work;
  T.work = w;
  T.band = T.active ? w / p.n_tiles : 0;
  const int32_t t = T.active ? w % p.n_tiles : 0;
  if (p.offsets == nullptr) return dense_tile(p, w);
  const int E = p.num_groups;
  const int tid = threadIdx.x;
  if (tid == 0) g.bad = 0;
  for (int i = tid; i <= E; i += kThreads) g.off[i] = p.offsets[i];
  __syncthreads();
  // per-segment padded rows and tiles, then inclusive scans
  for (int i = tid; i < E; i += kThreads) {
    const int64_t m = g.off[i + 1] - g.off[i];
    if (m < 0) atomicOr(&g.bad, 1);
    const int64_t pm = m < 0 ? 0 : (m + p.block - 1) / p.block * p.block;
    g.ppre[i + 1] = pm;
    g.tpre[i + 1] = (int32_t)((pm + kTileRows - 1) / kTileRows);
  }
  if (tid == 0) {
    g.ppre[0] = 0;
    g.tpre[0] = 0;
    if (g.off[0] != 0 || g.off[E] != p.rows) g.bad = 1;
  }
  __syncthreads();
  // inclusive scans of entries 1..E: each thread scans a run of `per`
  // consecutive entries, the run totals are scanned across the threads
  // (Hillis-Steele), and each run then adds the total of the runs before it
  const int per = (E + kThreads - 1) / kThreads;
  const int nrun = (E + per - 1) / per;
  const int b0 = 1 + tid * per, b1 = min(E + 1, b0 + per);
  {
    int64_t sp = 0;
    int32_t sq = 0;
    for (int i = b0; i < b1; ++i) {
      sp += g.ppre[i];
      g.ppre[i] = sp;
      sq += g.tpre[i];
      g.tpre[i] = sq;
    }
    g.runp[tid] = sp;
    g.runt[tid] = sq;
  }
  __syncthreads();
  for (int s = 1; s < nrun; s <<= 1) {
    int64_t a = 0;
    int32_t b = 0;
    if (tid >= s) {
      a = g.runp[tid - s];
      b = g.runt[tid - s];
    }
    __syncthreads();
    if (tid >= s) {
      g.runp[tid] += a;
      g.runt[tid] += b;
    }
    __syncthreads();
  }
  if (tid > 0) {
    const int64_t a = g.runp[tid - 1];
    const int32_t b = g.runt[tid - 1];
    for (int i = b0; i < b1; ++i) {
      g.ppre[i] += a;
      g.tpre[i] += b;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (p.do_col && g.ppre[E] != p.padded_rows) g.bad = 1;
    if (g.tpre[E] > p.n_tiles) g.bad = 1;
    // segment holding tile t: largest e with tpre[e] <= t < tpre[e+1]
    int lo = 0, hi = E;  // invariant tpre[lo] <= t < tpre[hi] (if t < tpre[E])
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tpre[mid] <= t) lo = mid; else hi = mid;
    }
    g.seg = lo;
  }
  __syncthreads();
  T.bad = g.bad != 0;
  const int e = g.seg;
  T.seg = e;
  T.seg_row0 = g.off[e];
  T.M = g.off[e + 1] - g.off[e];
  T.P = g.ppre[e + 1] - g.ppre[e];
  T.coff = g.ppre[e];
  T.m0 = (int64_t)(t - g.tpre[e]) * kTileRows;
  T.active = T.active && !T.bad && t < g.tpre[E] && T.m0 < T.P;
  return T;
}

struct LaneGeom {
  int wave, lane, half, lc;
  int64_t m_h0;  // local row of this half's first row
  int64_t c0;    // first column of the lane
  bool lane_ok;
};

__device__ __forceinline__ LaneGeom lane_geom(const QuantParams& p, const TileInfo& T) {
  LaneGeom L;
  L.wave = threadIdx.x >> 6;
  L.lane = threadIdx.x & 63;
  L.half = L.lane >> 5;
  L.lc = L.lane & 31;
  L.m_h0 = T.m0 + 32 * L.wave + 16 * L.half;
  L.c0 = (int64_t)T.band * kBandCols + 8 * L.lc;
  L.lane_ok = L.c0 < p.cols;
  return L;
}

// Load rows [R0, R1) of the lane's 16 x 8 sub-tile (zeros outside the
// segment / tensor).  The loads are unconditional and in row order, so
// consumers that walk the rows in order start before the last row arrives;
// lanes or rows outside the data read an in-bounds address and are zeroed.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load; STREAM marks it non-temporal (last use of the data).
template <bool STREAM>
__device__ __forceinline__ uint4 load16(const uint16_t* a) {
  if (STREAM) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  return *reinterpret_cast<const uint4*>(a);
}

template <int R0, int R1, bool STREAM = false>
__device__ __forceinline__ void load_rows(const QuantParams& p, const TileInfo& T, const LaneGeom& L,
                                          uint32_t w[16][4]) {
  const int64_t rows_left = T.M - L.m_h0;
  const bool full = L.lane_ok && rows_left >= 16;
  if (__all(full)) {
    const uint16_t* ptr = p.x + (T.seg_row0 + L.m_h0) * p.ld + L.c0;
#pragma unroll
    for (int i = R0; i < R1; ++i) {
      const uint4 v = load16<STREAM>(ptr + (int64_t)i * p.ld);
      w[i][0] = v.x;
      w[i][1] = v.y;
      w[i][2] = v.z;
      w[i][3] = v.w;
    }
  } else {
    const int64_t c = L.lane_ok ? L.c0 : 0;
#pragma unroll
    for (int i = R0; i < R1; ++i) {
      const bool ok = L.lane_ok && i < rows_left;
      const int64_t m = ok ? L.m_h0 + i : 0;  // row 0 of an active segment exists
      const uint4 v = load16<STREAM>(p.x + (T.seg_row0 + m) * p.ld + c);
      w[i][0] = ok ? v.x : 0u;
      w[i][1] = ok ? v.y : 0u;
      w[i][2] = ok ? v.z : 0u;
      w[i][3] = ok ? v.w : 0u;
    }
  }
}

__device__ __forceinline__ void load_tile(const QuantParams& p, const TileInfo& T, const LaneGeom& L,
                                          uint32_t w[16][4]) {
  load_rows<0, 16>(p, T, L, w);
}

// Folded signs of the lane's half of a row-wise block (selected by lane
// parity once per kernel, so the butterflies read registers, not memory).
struct RowLaneSigns {
  HalfSigns h;
  float s4;   // multiplier of the partner value in the cross-lane stage
  float fin;  // output multiplier (0.25 d0, and -q4 on odd lanes)
};

__device__ __forceinline__ float lane_select(float even, float odd, float oddf) {
  // even + (odd - even) * oddf with oddf in {0, 1}: exact for the +-1 / +-0.25
  // values involved, and computed from uniform (scalar) operands, so no
  // per-lane address into the kernel arguments is ever formed
  return fmaf(odd - even, oddf, even);
}

template <bool RHT>
__device__ __forceinline__ RowLaneSigns row_lane_signs(const QuantParams& p, int parity) {
  RowLaneSigns r;
  const float oddf = (float)parity;
#pragma unroll
  for (int k = 0; k < 4; ++k) r.h.q1[k] = lane_select(p.hs[0].q1[k], p.hs[1].q1[k], oddf);
#pragma unroll
  for (int k = 0; k < 2; ++k) r.h.q2[k] = lane_select(p.hs[0].q2[k], p.hs[1].q2[k], oddf);
  r.h.q3 = lane_select(p.hs[0].q3, p.hs[1].q3, oddf);
  r.s4 = lane_select(p.s4[0], p.s4[1], oddf);
  r.fin = RHT ? lane_select(p.fin_lane[0], p.fin_lane[1], oddf) : 1.0f;
  return r;
}

// Last butterfly stage of a row-wise block across a lane pair, for the
// lane's 8 values: v += s4 * (the partner lane's v), one v_fmac_f32 with a DPP
// quad_perm [1,0,3,2] operand per value (the compiler does not fold a DPP
// move into a multiply-accumulate).  The leading s_nop provides the two wait
// states a DPP read needs after a VALU write of its source; inside the block
// each instruction reads a register no earlier instruction of the block
// wrote.  All lanes are active wherever this is used.
__device__ __forceinline__ void cross_stage8(float v[8], float s4) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
      : "v"(s4));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Max over the 16 outputs of a block from the values before its last
// butterfly stage: max(|a + q b|, |a - q b|) = fl(|a| + |b|) exactly, since
// one of the two is a sum of like-signed terms and rounding is monotone.
__device__ __forceinline__ float lastpair_max(float m, float a, float b) {
  return fmaxf(m, fabsf(a) + fabsf(b));
}

// Two's-complement nibbles -> sign-magnitude nibbles, eight at a time: for a
// negative nibble n (bit 3 set, |n| <= 7) the sign-magnitude code is
// (n ^ 7) + 1; nonnegative nibbles (and zero) are unchanged.
__device__ __forceinline__ uint32_t tc_to_signmag8(uint32_t P) {
  const uint32_t A = P & 0x88888888u;
  const uint32_t S = A >> 3;
  return (P ^ (A - S)) + S;
}

// Shift the low nibble of m in at the top of acc (acc >> 4 | m << 28).
__device__ __forceinline__ uint32_t push_nibble(uint32_t m, uint32_t acc) {
  return __builtin_amdgcn_alignbit(m, acc, 4u);
}

// Shift the magnitude index k (< 8) in at the top of acc as a sign-magnitude
// nibble with the sign of s: bit 31 of s is the new nibble's bit 3.
__device__ __forceinline__ uint32_t push_signmag(uint32_t k, float s, uint32_t acc) {
  // (a & ~m) | (b & m) with m the sign bit: one three-input op (table 0xD8)
  return (uint32_t)__builtin_amdgcn_bitop3_b32(__builtin_amdgcn_alignbit(k, acc, 4u), __float_as_uint(s),
                                               0x80000000u, 0xD8);
}

// Eight sign-magnitude nibbles: a zero magnitude loses its sign bit (bit 3
// of m + 7 is set iff the magnitude m <= 7 is nonzero; no carry leaves the
// nibble).
__device__ __forceinline__ uint32_t clear_neg_zero8(uint32_t P) {
  const uint32_t nz = (P & 0x77777777u) + 0x77777777u;
  return (uint32_t)__builtin_amdgcn_bitop3_b32(P, nz, 0x77777777u, 0xE0);  // P & (nz | 0x77777777)
}

// Stochastic rounding of eight values, given in grid steps for the uniform
// grids and as they are for E2M1, packed as eight nibbles (value j in nibble
// j): sign-magnitude codes, or two's-complement ones for INT4.
template <int GRID>
__device__ __forceinline__ uint32_t sr_pack8(const float* s, const uint32_t* rw) {
  uint32_t acc = 0u;
  if (GRID == kGridINT4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t k = sr_steps<GRID>(s[j], rw[j]);
      const uint32_t sg = (uint32_t)((int32_t)__float_as_uint(s[j]) >> 31);
      acc = push_nibble((k ^ sg) - sg, acc);
    }
    return acc;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t k = GRID == kGridE2M1 ? sr_e2m1_index(s[j], rw[j]) : sr_steps<GRID>(s[j], rw[j]);
    acc = push_signmag(k, s[j], acc);
  }
  return clear_neg_zero8(acc);
}

// The values of NB blocks in grid steps for stochastic rounding, in place:
// s = ((v fin) inv_b) kMul, where fin is the lane's multiplier (1/4 with the
// folded sign, or 1) and kMul = 1 / (grid step) (1 for E2M1, whose steps
// differ: its values stay as they are).  When M = fin inv_b kMul
// has |M| >= 2^-15 (or inv_b is 0) in every block of the wavefront, s is the
// one product v M, which gives the same index and sign: M is then exact;
// v fin is exact (a nonzero v is a multiple of 2^-133, a sum of bf16
// values); at normal magnitudes the power-of-two factors commute with
// rounding; and a product in the subnormal range, in either form, is a
// nonzero value below 2^-124 (|v fin inv_b| >= 2^-149), so index 0 with
// threshold 1.
template <int GRID, int NB, int N>
__device__ __forceinline__ void sr_steps_inplace(float (&v)[NB][N], const float inv[NB], float fin) {
  constexpr float kMul = GRID == kGridINT4 || GRID == kGridE2M1 ? 1.0f : 2.0f;
  bool fold = true;
#pragma unroll
  for (int b = 0; b < NB; ++b) fold &= (inv[b] == 0.0f) | (fabsf(fin * inv[b] * kMul) >= 0x1p-15f);
  if (__all(fold)) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float m = fin * inv[b] * kMul;
#pragma unroll
      for (int j = 0; j < N; ++j) v[b][j] *= m;
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < N; ++j) v[b][j] = ((v[b][j] * fin) * inv[b]) * kMul;
  }
}

// t clamped to [-top, top], NaN to a zero: the median of |t|, 0 and top (a
// NaN operand makes v_med3_f32 return the smallest of the three, 0 here; t
// is the result of arithmetic, so never a signaling NaN), with t's sign.
__device__ __forceinline__ float clamp_top(float t, float top) {
  return __builtin_copysignf(__builtin_amdgcn_fmed3f(fabsf(t), 0.0f, top), t);
}

// Eight values rounded to E2M1 (nearest, ties to even, saturating at +-6)
// by the hardware conversion, two per instruction into byte k of the word
// (value j in nibble j), as sign-magnitude codes; a zero result loses the
// sign the conversion keeps.  Each value is first clamped to [-6, 6] with
// NaN mapped to a zero (clamp_top), the code the oracle gives a NaN; the
// conversion saturates at +-6 itself, so the clamp changes nothing else.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* y) {
  uint32_t w = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = clamp_top(y[2 * k], 6.0f), b = clamp_top(y[2 * k + 1], 6.0f);
    // the byte select must be a constant: k is unrolled
    if (k == 0) w = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 0);
    if (k == 1) w = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 1);
    if (k == 2) w = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 2);
    if (k == 3) w = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, 3);
  }
  return clear_neg_zero8(w);
}

// fl(t + 1.5*2^23) has t rounded to the nearest integer (ties to even) in
// its low mantissa bits, as a two's-complement value, for |t| < 2^22.
constexpr float kMagic = 12582912.0f;

// ---------------------------------------------------------------- phase A
// Largest magnitudes of the tile's row-wise and column-wise transforms
// (before the final 1/4), reduced over the workgroup and returned to every
// thread.  Rows are consumed in load order, each as soon as it arrives: its
// row-wise half-blocks are transformed at once, and the column-wise
// butterflies advance one stage whenever the rows they pair are present, so
// the arithmetic overlaps the remaining loads.  mid() runs once, after the
// first eight rows (a place to issue loads whose results are needed only at
// the end); on_row(i) runs when row i is first used.
template <bool RHT, typename Mid, typename OnRow>
__device__ __forceinline__ float2 tile_amax(const QuantParams& p, const LaneGeom& L, const uint32_t (&w)[16][4],
                                            float (&red)[2][kThreads / 64], Mid&& mid, OnRow&& on_row) {
  float acc_r = 0.0f, acc_c = 0.0f;
  const bool do_row = p.do_row != 0, do_col = p.do_col != 0;
  const RowLaneSigns rs = row_lane_signs<RHT>(p, L.lc & 1);
  float cv[16][8];  // column-wise values of the lane's 8 columns, by row
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    on_row(i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cv[i][2 * k] = bf_lo(w[i][k]);
      cv[i][2 * k + 1] = bf_hi(w[i][k]);
    }
    if (do_row) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = cv[i][j];
      if (RHT) {
        fwht8_half(v, rs.h);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc_r = lastpair_max(acc_r, v[j], dpp_xor1(v[j]));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc_r = fmaxf(acc_r, fabsf(v[j]));
      }
    }
    if (i == 8) mid();
    if (RHT && do_col) {
      // column-wise stages of half-width 1, 2, 4 once their rows are here
      if (i % 2 == 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) bfly(cv[i - 1][c], cv[i][c], p.sg.q1[i / 2]);
      }
      if (i % 4 == 3) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          bfly(cv[i - 3][c], cv[i - 1][c], p.sg.q2[i / 4]);
          bfly(cv[i - 2][c], cv[i][c], p.sg.q2[i / 4]);
        }
      }
      if (i % 8 == 7) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int c = 0; c < 8; ++c) bfly(cv[i - 7 + j][c], cv[i - 3 + j][c], p.sg.q3[i / 8]);
        }
      }
    }
  }
  if (do_col) {
    // the last stage folds into the max
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc_c = RHT ? lastpair_max(acc_c, cv[j][c], cv[j + 8][c])
                    : fmaxf(acc_c, fmaxf(fabsf(cv[j][c]), fabsf(cv[j + 8][c])));
    }
  }
  acc_r = wave_max(acc_r);
  acc_c = wave_max(acc_c);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = acc_r;
    red[1][threadIdx.x >> 6] = acc_c;
  }
  __syncthreads();
  float r = red[0][0], c = red[1][0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) {
    r = fmaxf(r, red[0][i]);
    c = fmaxf(c, red[1][i]);
  }
  return make_float2(r, c);
}

template <bool RHT>
__global__ __launch_bounds__(kThreads) void ufp4_amax_kernel(QuantParams p) {
  __shared__ GroupLds g;
  __shared__ float red[2][kThreads / 64];
  const TileInfo T = tile_info(p, g);
  if (!T.active) return;  // uniform per workgroup; its partial slot is never read
  const LaneGeom L = lane_geom(p, T);
  uint32_t w[16][4];
  load_tile(p, T, L, w);
  const float2 m = tile_amax<RHT>(p, L, w, red, [] {}, [](int) {});
  if (threadIdx.x == 0) p.ws_part[T.work] = m;
}

// ---------------------------------------------------------------- phase B
// Per-tensor quantities of one layout of the workgroup's segment.
struct TensorScale {
  float S;     // S_t
  float D;     // fl(Qmax * S_t)
  float R4;    // fl(1 / D), times 1/4 under the transform (block maxima are
               // taken before the transform's final 1/4)
  bool fast;   // D normal and at most 2^120 (so R4 is exact), amax small
               // enough that 0.25 * inv_b is exact
};

// raw = max |transform before the 1/4| over the tensor (or max |x| without
// the transform).  S_t = amax / (Qmax * 448), 1 for an all-zero tensor.
template <bool RHT>
__device__ __forceinline__ TensorScale make_tensor_scale(float raw, float qmax) {
  TensorScale ts;
  const float a = RHT ? raw * 0.25f : raw;  // max of the scaled values (rounding is monotone)
  ts.S = (a > 0.0f) ? a / (qmax * 448.0f) : 1.0f;
  ts.D = qmax * ts.S;
  const float R = 1.0f / ts.D;
  ts.R4 = RHT ? R * 0.25f : R;
  ts.fast = ts.D >= 0x1p-126f && ts.D <= 0x1p+120f && a < 0x1p+119f;
  return ts;
}

// Block scales of NB blocks from their raw maxima (before the transform's
// final 1/4).  NV16: s_b = E4M3(fl(amax_b / D)), saturated.  When the
// per-tensor quantities allow it, fl(raw * R4) = fl(amax_b * fl(1/D)) lies
// within 3 ulp of amax_b / D, so if both ends of a +-2^-21 bracket around it
// encode to the same E4M3 code, that code is exact (E4M3 rounding is
// monotone).  Every block maximum is at most the tensor maximum, so the
// bracket stays below 448 (1 + 2^-20), inside the range where the hardware
// conversion rounds to nearest even and saturates to 448.  If any block of the
// wavefront is not decided that way (or its maximum is too small for the 1/4
// to be exact), the correctly rounded division decides for all of them.
// MX32: a power-of-two scale.  Returns true when every block of the
// wavefront allows the exact fast rounding (normal block scale, no tiny
// nonzero maximum); blocks outside the data hold zeros and always allow it.
// Under a provided (delayed) tensor maximum a block maximum may exceed it:
// DELAYED clamps the converter input at 448, where E4M3 saturates.
template <int GRID, bool MX, bool RHT, int NB, bool DELAYED = false>
__device__ __forceinline__ bool block_scales(const float raw[NB], const TensorScale& ts, bool fast_u,
                                             const float* lut_l, uint32_t sbyte[NB], float inv[NB]) {
  constexpr float kThr = RHT ? 0x1p-98f : 0x1p-100f;  // raw maxima whose 1/4 keeps codes exact
  bool bad = false;
  if (MX) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      mx_scale<GRID>(RHT ? raw[b] * 0.25f : raw[b], sbyte[b], inv[b]);
      bad |= (raw[b] != 0.0f) & !(raw[b] >= kThr);
    }
  } else {
    bool need_div = !fast_u;
    bool tiny[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) tiny[b] = (raw[b] != 0.0f) & (raw[b] < kThr);
    if (fast_u) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float q = DELAYED ? fminf(raw[b] * ts.R4, 448.0f) : raw[b] * ts.R4;
        const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q * 0x1.fffffp-1f,   // q (1 - 2^-21)
                                                                       q * 0x1.000004p+0f,  // q (1 + 2^-21)
                                                                       0, false);
        sbyte[b] = pk & 0xFFu;
        need_div |= (sbyte[b] != ((pk >> 8) & 0xFFu)) | tiny[b];
      }
    }
    if (__any(need_div)) {
#pragma unroll
      for (int b = 0; b < NB; ++b) sbyte[b] = e4m3_encode_sat((RHT ? raw[b] * 0.25f : raw[b]) / ts.D);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) inv[b] = lut_l[sbyte[b]];
    bad = !fast_u;
#pragma unroll
    for (int b = 0; b < NB; ++b) bad |= tiny[b] | ((raw[b] != 0.0f) & (sbyte[b] < 8u));
  }
  return !__any(bad);
}

// Staging of a tile's column-wise output for NK of each lane's 8 columns
// (32 NK of the band's 256): [chunk][staged column] with chunk = the 16-row
// block of one half-wavefront (8 per 128-row tile).  One padding entry per
// chunk row spreads the write-out reads over the LDS banks.
template <int NK>
struct ColStageT {
  uint2 codes[8][32 * NK + 1];
  uint8_t scales[8][32 * NK + 4];
};
using ColStage = ColStageT<8>;

// RTNE onto E1M2/INT4/E2M1C has an exact fast form; it needs no clamp when
// the block scale is a normal E4M3 value (then |y| <= 1.0625 Qmax) and the
// tensor maximum is the tensor's own (otherwise it clamps to +-Qmax).
template <int GRID, bool SR>
struct GridTraits {
  static constexpr bool kFast = !SR && GRID != kGridE2M1;      // uniform grids
  static constexpr float kMul = GRID == kGridINT4 ? 1.0f : 2.0f;  // grid step -> integer
  static constexpr float kTop = (float)grid_top<GRID>();          // clamp, in grid steps
};

// Row-wise pass over the lane's 16 rows, NR row blocks per step (4, or 2
// where registers are short): values, block scales, one wavefront vote,
// round, pack, store.  src(i, v)
// writes the lane's 8 transformed values of row i (before the transform's
// final 1/4; the row's own values without the transform) to v and returns
// the largest magnitude of the 16-element block (over the lane pair).  fin
// is the lane's output multiplier (the 1/4 and the folded sign).  Returns the
// largest block maximum seen (for DELAYED).
template <int GRID, bool SR, bool MX, bool RHT, bool DELAYED, int NR = 4, typename RowSrc>
__device__ __forceinline__ float row_pass(const QuantParams& p, const TileInfo& T, const LaneGeom& L,
                                          const TensorScale& tsr, const float* lut_l, float fin,
                                          RowSrc&& src) {
  using G = GridTraits<GRID, SR>;
  float tile_r = 0.0f;
  const bool fast_r = __builtin_amdgcn_readfirstlane((int)tsr.fast) != 0;
  const int parity = L.lc & 1;
  const int64_t C = p.cols;
  const int64_t tile_row0 = T.seg_row0 + T.m0;
  const uint32_t lrow = (uint32_t)(32 * L.wave + 16 * L.half);  // lane's first row in the tile
  const int B = MX ? 32 : 16;
  uint8_t* rc_base = p.row_codes + tile_row0 * (C / 2) + (int64_t)T.band * (kBandCols / 2);
  uint8_t* rsc_base = p.row_scales + tile_row0 * (C / B) + (int64_t)T.band * (kBandCols / B);
  const uint32_t rc_stride = (uint32_t)(C / 2), rsc_stride = (uint32_t)(C / B);
#pragma clang loop unroll(full)
  for (int g4 = 0; g4 < 16 / NR; ++g4) {
    float v[NR][8];
    float raw[NR], inv[NR];
    uint32_t sbyte[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      float m = src(NR * g4 + r, v[r]);
      if (MX) m = fmaxf(m, dpp_xor2(m));
      raw[r] = m;
    }
    const bool ok = block_scales<GRID, MX, RHT, NR, DELAYED>(raw, tsr, fast_r, lut_l, sbyte, inv);
    if (DELAYED) {
#pragma unroll
      for (int r = 0; r < NR; ++r) tile_r = fmaxf(tile_r, raw[r]);
    }
    uint32_t packed[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) packed[r] = 0u;
    if (G::kFast && ok) {
      // t = y / (grid step) as one product: an exact power-of-two rescaling
      // of fl(fl(v/4) * inv_b) for every element whose code can be nonzero
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float mult = inv[r] * (fin * G::kMul);
        uint32_t acc = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float t = v[r][j] * mult;
          if (MX || DELAYED) t = clamp_top(t, G::kTop);
          acc = push_nibble(__float_as_uint(t + kMagic), acc);
        }
        packed[r] = GRID == kGridINT4 ? acc : tc_to_signmag8(acc);
      }
    } else if (GRID == kGridE2M1 && !SR && ok) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = (v[r][j] * fin) * inv[r];
        packed[r] = e2m1_pack8(y);
      }
    } else {
      if (SR) sr_steps_inplace<GRID>(v, inv, fin);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int i = NR * g4 + r;
        if (SR) {
          const uint64_t base = (uint64_t)(T.seg_row0 + L.m_h0 + i) * (uint64_t)C + (uint64_t)L.c0;
          const Ctr4 r0 = sr_words4(base >> 2, 0u, p.sr_k0, p.sr_k1);
          const Ctr4 r1 = sr_words4((base >> 2) + 1, 0u, p.sr_k0, p.sr_k1);
          const uint32_t rw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
          packed[r] = sr_pack8<GRID>(v[r], rw);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            packed[r] |= quantize_code<GRID, false>((v[r][j] * fin) * inv[r], 0u) << (4 * j);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int i = NR * g4 + r;
      if (L.lane_ok && L.m_h0 + i < T.M) {
        const uint32_t li = lrow + (uint32_t)i;
        __builtin_nontemporal_store(packed[r], reinterpret_cast<uint32_t*>(rc_base + (li * rc_stride + 4u * (uint32_t)L.lc)));
        if (MX) {
          if ((L.lc & 3) == 0) rsc_base[li * rsc_stride + ((uint32_t)L.lc >> 2)] = (uint8_t)sbyte[r];
        } else if (parity == 0) {
          rsc_base[li * rsc_stride + ((uint32_t)L.lc >> 1)] = (uint8_t)sbyte[r];
        }
      }
    }
  }
  return tile_r;
}

// Column-wise pass over the lane's columns K0 .. K0+NK-1 (of its 8), two
// column blocks per step, then the write-out.  src(k, v) writes the lane's
// 16 transformed values of its column k (before the final 1/4) to v and
// returns their largest magnitude.  Codes and scales go to LDS first (chunk
// = one half-wavefront's 16 rows), then leave as contiguous 8-byte code runs
// and byte runs per output line, instead of one scattered store per lane and
// column.  The staging area is read by the write-out after a barrier; a
// caller that reuses it must synchronize first.  Returns the largest block
// maximum seen (for DELAYED).
template <int GRID, bool SR, bool MX, bool RHT, bool DELAYED, int K0 = 0, int NK = 8, typename ColSrc>
__device__ __forceinline__ float col_pass(const QuantParams& p, const TileInfo& T, const LaneGeom& L,
                                          const TensorScale& tsc, const float* lut_l, ColStageT<NK>& cst,
                                          ColSrc&& src) {
  static_assert(K0 % 2 == 0 && NK % 2 == 0 && K0 + NK <= 8, "whole column pairs of the lane");
  using G = GridTraits<GRID, SR>;
  float tile_c = 0.0f;
  const bool fast_c = __builtin_amdgcn_readfirstlane((int)tsc.fast) != 0;
  const float fin = RHT ? p.sg.fin : 1.0f;
  const int ch = 2 * L.wave + L.half;  // chunk of this half-wavefront
#pragma clang loop unroll(full)
  for (int g2 = K0 / 2; g2 < (K0 + NK) / 2; ++g2) {
    float v[2][16];
    float raw[2], inv[2];
    uint32_t sbyte[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float m = src(2 * g2 + r, v[r]);
      if (MX) m = fmaxf(m, __shfl_xor(m, 32));
      raw[r] = m;
    }
    const bool ok = block_scales<GRID, MX, RHT, 2, DELAYED>(raw, tsc, fast_c, lut_l, sbyte, inv);
    if (DELAYED) tile_c = fmaxf(tile_c, fmaxf(raw[0], raw[1]));
    uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
    if (G::kFast && ok) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float mult = inv[r] * (fin * G::kMul);
        uint32_t a0 = 0u, a1 = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float t0 = v[r][j] * mult, t1 = v[r][8 + j] * mult;
          if (MX || DELAYED) {
            t0 = clamp_top(t0, G::kTop);
            t1 = clamp_top(t1, G::kTop);
          }
          a0 = push_nibble(__float_as_uint(t0 + kMagic), a0);
          a1 = push_nibble(__float_as_uint(t1 + kMagic), a1);
        }
        lo[r] = GRID == kGridINT4 ? a0 : tc_to_signmag8(a0);
        hi[r] = GRID == kGridINT4 ? a1 : tc_to_signmag8(a1);
      }
    } else if (GRID == kGridE2M1 && !SR && ok) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = (v[r][j] * fin) * inv[r];
        lo[r] = e2m1_pack8(y);
        hi[r] = e2m1_pack8(y + 8);
      }
    } else {
      if (SR) sr_steps_inplace<GRID>(v, inv, fin);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (SR) {
          const int64_t cglob = L.c0 + 2 * g2 + r;
          const uint64_t base = (uint64_t)cglob * (uint64_t)p.padded_rows + (uint64_t)(T.coff + L.m_h0);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const Ctr4 r0 = sr_words4((base >> 2) + 2 * h, 1u, p.sr_k0, p.sr_k1);
            const Ctr4 r1 = sr_words4((base >> 2) + 2 * h + 1, 1u, p.sr_k0, p.sr_k1);
            const uint32_t rw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
            (h ? hi[r] : lo[r]) = sr_pack8<GRID>(&v[r][8 * h], rw);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            lo[r] |= quantize_code<GRID, false>((v[r][j] * fin) * inv[r], 0u) << (4 * j);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            hi[r] |= quantize_code<GRID, false>((v[r][8 + j] * fin) * inv[r], 0u) << (4 * j);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sc = NK * L.lc + 2 * g2 + r - K0;  // staged column
      cst.codes[ch][sc] = make_uint2(lo[r], hi[r]);
      cst.scales[ch][sc] = (uint8_t)sbyte[r];
    }
  }
  __syncthreads();
  // write-out: 8 threads per output line (column), one 8-byte code run each;
  // staged column sc is band column 8 (sc / NK) + K0 + sc % NK
  const int64_t Rp = p.padded_rows;
  const int B = MX ? 32 : 16;
  const int64_t band_c0 = (int64_t)T.band * kBandCols;
  const int64_t ncols = p.cols - band_c0 < kBandCols ? p.cols - band_c0 : kBandCols;
  const int64_t rows_here = T.P - T.m0;
  const int nch = rows_here >= kTileRows ? 8 : (int)(rows_here / 16);  // chunks that exist
  uint8_t* cc = p.col_codes + band_c0 * (Rp / 2) + (T.coff + T.m0) / 2;
  const bool run_aligned = ((T.coff + T.m0) & 127) == 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int q = threadIdx.x + j * kThreads;
    const int sc = q >> 3, chq = q & 7;
    const int col = 8 * (sc / NK) + K0 + sc % NK;
    if (col < ncols && chq < nch) {
      const uint2 cw = cst.codes[chq][sc];
      const u32x2 cv2 = {cw.x, cw.y};
      u32x2* dst = reinterpret_cast<u32x2*>(cc + (int64_t)col * (Rp / 2) + 8 * chq);
      // A tile's 64-byte run fills a line half when it starts on one (dense
      // tensors): written once, non-temporal.  Segment starts fall on any 16
      // rows, and then the run shares its lines with the neighbouring tiles'
      // runs: cached stores let the L2 merge them before they are written.
      if (run_aligned)
        __builtin_nontemporal_store(cv2, dst);
      else
        *dst = cv2;
    }
  }
  uint8_t* cs = p.col_scales + band_c0 * (Rp / B) + (T.coff + T.m0) / B;
  const int nsc = MX ? nch / 2 : nch;  // scale bytes per line in this tile
  constexpr int per = MX ? 4 : 8;
#pragma unroll
  for (int j = 0; j < NK * per / 8; ++j) {
    const int q = threadIdx.x + j * kThreads;
    const int sc = q / per, b = q % per;
    const int col = 8 * (sc / NK) + K0 + sc % NK;
    if (col < ncols && b < nsc) cs[(int64_t)col * (Rp / B) + b] = cst.scales[MX ? 2 * b : b][sc];
  }
  return tile_c;
}

// Quantize one tile whose rows are loaded (or in flight, in load order) in
// w, given the per-tensor scales of the two layouts and their inverse
// block-factor tables: row-wise codes and scales straight to memory,
// column-wise ones through the LDS staging area.  Both transforms are
// computed here.  KEEP: the rows are unpacked once and kept unpacked for the
// column-wise pass (fewer instructions); otherwise they are unpacked again
// there (fewer registers).
template <int GRID, bool SR, bool MX, bool RHT, bool KEEP = true, bool DELAYED = false>
__device__ __forceinline__ float2 quant_tile(const QuantParams& p, const TileInfo& T, const LaneGeom& L,
                                             const uint32_t (&w)[16][4], const TensorScale& tsr,
                                             const TensorScale& tsc, const float (&lut)[2][128], ColStage& cst) {
  // DELAYED: the tensor scales come from provided maxima, so a block may
  // exceed them; scales and codes saturate, and the lane's largest block
  // maxima (before the final 1/4) are returned for the next call.
  float tile_r = 0.0f, tile_c = 0.0f;
  // The sub-tile is unpacked once (row by row, in load order, inside the
  // row-wise pass) and kept for the column-wise pass.
  float xf[16][8];
  if (KEEP && !p.do_row) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xf[i][2 * k] = bf_lo(w[i][k]);
        xf[i][2 * k + 1] = bf_hi(w[i][k]);
      }
    }
  }
  const RowLaneSigns rs = row_lane_signs<RHT>(p, L.lc & 1);
  if (p.do_row) {
    tile_r = row_pass<GRID, SR, MX, RHT, DELAYED, SR ? 2 : 4>(
        p, T, L, tsr, lut[0], rs.fin, [&](int i, float(&v)[8]) __attribute__((always_inline)) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            xf[i][2 * k] = bf_lo(w[i][k]);
            xf[i][2 * k + 1] = bf_hi(w[i][k]);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = xf[i][j];  // (without KEEP, xf is dead beyond this row)
          if (RHT) {
            fwht8_half(v, rs.h);
            cross_stage8(v, rs.s4);
          }
          float m = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
          return fmaxf(m, dpp_xor1(m));
        });
  }
  if (p.do_col) {
    tile_c = col_pass<GRID, SR, MX, RHT, DELAYED>(
        p, T, L, tsc, lut[1], cst, [&](int k, float(&v)[16]) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[i] = KEEP ? xf[i][k] : ((k & 1) ? bf_hi(w[i][k >> 1]) : bf_lo(w[i][k >> 1]));
          if (RHT) fwht16_inlane(v, p.sg);
          float m = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(v[j]));
          return m;
        });
  }
  return make_float2(tile_r, tile_c);
}

template <int GRID, bool SR, bool MX, bool RHT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void ufp4_quant_kernel(QuantParams p) {
  __shared__ GroupLds g;
  __shared__ float lut[2][128];
  __shared__ float red[2][kThreads / 64];
  __shared__ ColStage cst;
  const TileInfo T = tile_info(p, g);
  if (blockIdx.x == 0) {
    // tensor scales nobody else writes: MX32 (always 1) and empty segments
    if (p.offsets && p.ws_status && threadIdx.x == 0) *p.ws_status = T.bad ? 6u : 0u;
    if (p.offsets == nullptr || !T.bad) {
      for (int e = threadIdx.x; e < p.num_groups; e += kThreads) {
        const bool empty = p.offsets != nullptr && g.off[e + 1] == g.off[e];
        if (MX || empty) {
          if (p.do_row && p.row_ts) p.row_ts[e] = 1.0f;
          if (p.do_col && p.col_ts) p.col_ts[e] = 1.0f;
        }
      }
    }
  }
  if (!T.active) return;  // uniform per workgroup
  const LaneGeom L = lane_geom(p, T);
  constexpr float qmax = grid_qmax<GRID>();
  TensorScale tsr{1.0f, qmax, 1.0f / qmax, false}, tsc = tsr;
  // Phase-A partials of the segment: the first 4 per thread are requested
  // before the tile, so their latency overlaps the tile loads.  The loads are
  // unconditional (clamped index, result selected afterwards), so they issue
  // back to back; a dense tensor's partials are contiguous.
  const uint32_t t0 = p.offsets ? (uint32_t)g.tpre[T.seg] : 0u;
  const uint32_t nt = p.offsets ? (uint32_t)(g.tpre[T.seg + 1] - g.tpre[T.seg]) : (uint32_t)p.n_tiles;
  const uint32_t cnt = MX ? 0u : nt * (uint32_t)p.n_band;
  auto part_index = [&](uint32_t j) -> uint32_t {
    return p.offsets ? (j / nt) * (uint32_t)p.n_tiles + t0 + j % nt : j;
  };
  float2 pre[4];
  if (!MX) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t i = threadIdx.x + q * kThreads;
      pre[q] = p.ws_part[part_index(i < cnt ? i : cnt - 1u)];
    }
  }
  // The first four rows are requested before the prologue and the rest after
  // it: with fewer requests ahead of them in the memory queues, the rows the
  // first group needs arrive sooner.
  uint32_t w[16][4];
  load_rows<0, 4, true>(p, T, L, w);
  if (!MX) {
    // per-tensor maximum of the segment from the phase-A partials
    float r = 0.0f, c = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool in = threadIdx.x + q * kThreads < cnt;
      r = fmaxf(r, in ? pre[q].x : 0.0f);
      c = fmaxf(c, in ? pre[q].y : 0.0f);
    }
    for (uint32_t i = threadIdx.x + 4 * kThreads; i < cnt; i += kThreads) {
      const float2 q = p.ws_part[part_index(i)];
      r = fmaxf(r, q.x);
      c = fmaxf(c, q.y);
    }
    r = wave_max(r);
    c = wave_max(c);
    if ((threadIdx.x & 63) == 0) {
      red[0][threadIdx.x >> 6] = r;
      red[1][threadIdx.x >> 6] = c;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
      r = fmaxf(r, red[0][i]);
      c = fmaxf(c, red[1][i]);
    }
    tsr = make_tensor_scale<RHT>(r, qmax);
    tsc = make_tensor_scale<RHT>(c, qmax);
    {
      const int t = threadIdx.x, l = t >> 7, cc = t & 127;
      const float S = l ? tsc.S : tsr.S;
      const float d = (cc == 127) ? 0.0f : e4m3_decode_pos((uint32_t)cc) * S;
      lut[l][cc] = (d == 0.0f) ? 0.0f : 1.0f / d;  // inverse dequantization factor per code
    }
    if (threadIdx.x == 0 && T.band == 0 && T.m0 == 0) {
      if (p.do_row && p.row_ts) p.row_ts[T.seg] = tsr.S;
      if (p.do_col && p.col_ts) p.col_ts[T.seg] = tsc.S;
    }
    __syncthreads();
  }
  load_rows<4, 16, true>(p, T, L, w);
  quant_tile<GRID, SR, MX, RHT, false>(p, T, L, w, tsr, tsc, lut, cst);
}

// ------------------------------------------------------------ delayed
// One kernel for a dense NV16 tensor whose per-tensor scales come from
// provided maxima (delayed scaling): the input is read once.  The provided
// maxima are p.amax_in[0 .. n_in), pairs (row-wise, column-wise) of maxima of
// the transformed values, reduced here (a value that is not a positive
// finite number counts as zero).  The kernel writes its own tile maxima, in
// the same units, to p.amax_out[T.work] for the next call.
__device__ __forceinline__ float given_max(float m) { return (m > 0.0f && m <= 3.4028235e38f) ? m : 0.0f; }

template <bool RHT>
__device__ __forceinline__ TensorScale given_tensor_scale(float a, float qmax) {
  TensorScale ts;
  ts.S = (a > 0.0f) ? a / (qmax * 448.0f) : 1.0f;
  ts.D = qmax * ts.S;
  const float R = 1.0f / ts.D;
  ts.R4 = RHT ? R * 0.25f : R;
  ts.fast = ts.D >= 0x1p-126f && ts.D <= 0x1p+120f && a < 0x1p+119f;
  return ts;
}

template <int GRID, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void ufp4_delayed_kernel(QuantParams p) {
  __shared__ float lut[2][128];
  __shared__ float red[2][kThreads / 64];
  __shared__ ColStage cst;
  const TileInfo T = dense_tile(p, remap_xcd((int32_t)blockIdx.x, (int32_t)gridDim.x));
  if (!T.active) return;  // uniform per workgroup
  const LaneGeom L = lane_geom(p, T);
  constexpr float qmax = grid_qmax<GRID>();
  const uint32_t cnt = (uint32_t)p.n_in;
  float2 pre = make_float2(0.0f, 0.0f);
  if (threadIdx.x < cnt) pre = p.amax_in[threadIdx.x];
  uint32_t w[16][4];
  load_rows<0, 4, true>(p, T, L, w);
  float r = given_max(pre.x), c = given_max(pre.y);
  for (uint32_t i = threadIdx.x + kThreads; i < cnt; i += kThreads) {
    const float2 q = p.amax_in[i];
    r = fmaxf(r, given_max(q.x));
    c = fmaxf(c, given_max(q.y));
  }
  r = wave_max(r);
  c = wave_max(c);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = r;
    red[1][threadIdx.x >> 6] = c;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    r = fmaxf(r, red[0][i]);
    c = fmaxf(c, red[1][i]);
  }
  const TensorScale tsr = given_tensor_scale<RHT>(r, qmax), tsc = given_tensor_scale<RHT>(c, qmax);
  {
    const int t = threadIdx.x, l = t >> 7, cc = t & 127;
    const float S = l ? tsc.S : tsr.S;
    const float d = (cc == 127) ? 0.0f : e4m3_decode_pos((uint32_t)cc) * S;
    lut[l][cc] = (d == 0.0f) ? 0.0f : 1.0f / d;  // inverse dequantization factor per code
  }
  if (threadIdx.x == 0 && T.band == 0 && T.m0 == 0) {
    if (p.do_row && p.row_ts) p.row_ts[0] = tsr.S;
    if (p.do_col && p.col_ts) p.col_ts[0] = tsc.S;
  }
  __syncthreads();  // also: every thread has read red
  load_rows<4, 16, true>(p, T, L, w);
  float2 m = quant_tile<GRID, SR, false, RHT, false, true>(p, T, L, w, tsr, tsc, lut, cst);
  m.x = wave_max(m.x);
  m.y = wave_max(m.y);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = m.x;
    red[1][threadIdx.x >> 6] = m.y;
  }
  __syncthreads();
  if (threadIdx.x == 0 && p.amax_out) {
    float a = red[0][0], b = red[1][0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) {
      a = fmaxf(a, red[0][i]);
      b = fmaxf(b, red[1][i]);
    }
    // maxima of the transformed values: the final 1/4 is exact
    p.amax_out[T.work] = RHT ? make_float2(a * 0.25f, b * 0.25f) : make_float2(a, b);
  }
}

// ------------------------------------------------- grouped delayed
// Delayed scaling for ragged expert segments (NV16): segment e's tensor
// scales come from the provided maxima p.amax_in[e] = (row-wise,
// column-wise) maxima of that segment's transformed values (the previous
// step's, for instance), so the input is read once by one kernel.  Each
// workgroup folds its tile maxima into p.amax_out[e] (when given; zeroed by
// the host beforehand) with an atomic max on the bit patterns, which order
// like the non-negative values; the updates are not waited for.
template <int GRID, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void ufp4_grouped_delayed_kernel(QuantParams p) {
  __shared__ GroupLds g;
  __shared__ float lut[2][128];
  __shared__ float red[2][kThreads / 64];
  __shared__ ColStage cst;
  const TileInfo T = tile_info(p, g);
  if (blockIdx.x == 0) {
    if (p.ws_status && threadIdx.x == 0) *p.ws_status = T.bad ? 6u : 0u;
    if (!T.bad) {
      for (int e = threadIdx.x; e < p.num_groups; e += kThreads) {
        if (g.off[e + 1] == g.off[e]) {  // empty segment: nothing to quantize, S_t = 1
          if (p.do_row && p.row_ts) p.row_ts[e] = 1.0f;
          if (p.do_col && p.col_ts) p.col_ts[e] = 1.0f;
        }
      }
    }
  }
  if (!T.active) return;  // uniform per workgroup
  const LaneGeom L = lane_geom(p, T);
  constexpr float qmax = grid_qmax<GRID>();
  const float2 given = p.amax_in[T.seg];
  uint32_t w[16][4];
  load_rows<0, 4, true>(p, T, L, w);
  const TensorScale tsr = given_tensor_scale<RHT>(given_max(given.x), qmax);
  const TensorScale tsc = given_tensor_scale<RHT>(given_max(given.y), qmax);
  {
    const int t = threadIdx.x, l = t >> 7, cc = t & 127;
    const float S = l ? tsc.S : tsr.S;
    const float d = (cc == 127) ? 0.0f : e4m3_decode_pos((uint32_t)cc) * S;
    lut[l][cc] = (d == 0.0f) ? 0.0f : 1.0f / d;  // inverse dequantization factor per code
  }
  if (threadIdx.x == 0 && T.band == 0 && T.m0 == 0) {
    if (p.do_row && p.row_ts) p.row_ts[T.seg] = tsr.S;
    if (p.do_col && p.col_ts) p.col_ts[T.seg] = tsc.S;
  }
  __syncthreads();
  load_rows<4, 16, true>(p, T, L, w);
  float2 m = quant_tile<GRID, SR, false, RHT, false, true>(p, T, L, w, tsr, tsc, lut, cst);
  m.x = wave_max(m.x);
  m.y = wave_max(m.y);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = m.x;
    red[1][threadIdx.x >> 6] = m.y;
  }
  __syncthreads();
  if (threadIdx.x == 0 && p.amax_out) {
    float a = red[0][0], b = red[1][0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) {
      a = fmaxf(a, red[0][i]);
      b = fmaxf(b, red[1][i]);
    }
    // maxima of the transformed values: the final 1/4 is exact
    if (RHT) {
      a *= 0.25f;
      b *= 0.25f;
    }
    uint32_t* out = reinterpret_cast<uint32_t*>(p.amax_out + T.seg);
    if (p.do_row) __hip_atomic_fetch_max(out, __float_as_uint(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.do_col) __hip_atomic_fetch_max(out + 1, __float_as_uint(b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------- bandwidth roof
// The memory traffic of a dense NV16 row+col call with no arithmetic: the
// same tile walk (XCD-aware order) and 16-byte non-temporal loads of the
// lane sub-tiles as the quantization kernels, and the call's output bytes
// (both layouts' codes and block scales) as coalesced stores (cached: the
// output's 8- to 128-byte pieces of lines are merged in the L2, which
// measured faster than non-temporal stores for this pattern).
// The stored value is the loaded words folded to one word and compared with
// a constant, so every load is live; it is zero unless a lane's 64 words
// xor to that constant.  Full tiles only (rows a multiple of 128, columns of
// 256; the host checks).
__global__ __launch_bounds__(kThreads) void ufp4_roof_kernel(QuantParams p) {
  const TileInfo T = dense_tile(p, remap_xcd((int32_t)blockIdx.x, (int32_t)gridDim.x));
  if (!T.active) return;
  const LaneGeom L = lane_geom(p, T);
  uint32_t w[16][4];
  load_rows<0, 16, true>(p, T, L, w);
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc ^= w[i][0] ^ w[i][1] ^ w[i][2] ^ w[i][3];
  const uint32_t z = (acc == 0x9E3779B9u) ? 1u : 0u;
  const u32x4 o = {z, z, z, z};
  const int t = threadIdx.x;
  const int64_t c0 = (int64_t)T.band * kBandCols;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // row-wise codes: 128 rows x 128 bytes
    const int i = t + kThreads * j, r = i >> 3, k = i & 7;
    *reinterpret_cast<u32x4*>(p.row_codes + (T.m0 + r) * (p.cols / 2) + c0 / 2 + 16 * k) = o;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // column-wise codes: 256 columns x 64 bytes
    const int i = t + kThreads * j, c = i >> 2, k = i & 3;
    *reinterpret_cast<u32x4*>(p.col_codes + (c0 + c) * (p.padded_rows / 2) + T.m0 / 2 + 16 * k) = o;
  }
  if (t < kTileRows)  // row-wise scales: 16 bytes per row
    *reinterpret_cast<u32x4*>(p.row_scales + (T.m0 + t) * (p.cols / 16) + c0 / 16) = o;
  const u32x2 o2 = {z, z};  // column-wise scales: 8 bytes per column
  *reinterpret_cast<u32x2*>(p.col_scales + (c0 + t) * (p.padded_rows / 16) + T.m0 / 16) = o2;
}

// ------------------------------------------------------- single pass
// One kernel for a dense NV16 tensor whose tiles the device can hold at
// once: each workgroup loads its tile, computes the tile maxima (phase A),
// keeps the tile in registers while the maxima of all tiles are exchanged
// through generation-tagged words in the workspace, then quantizes it
// (phase B) without reading it again.
//
// No workgroup waits for one that has not started: before publishing its
// maxima, a workgroup checks that every tile's start word carries this call's
// generation.  If some tile has not started within kGraceTicks, the device
// cannot hold all tiles at once (other work occupies it, or the grid is too
// large); the workgroup then publishes its maxima marked "left", and exits.
// Every started workgroup publishes without waiting, so every partial word
// is eventually written and the exchange completes.  The workgroups that stay
// see the same final words, so they agree on which tiles were left and share
// them out by rank, reloading each such tile.  The last workgroup to start
// always finds every tile started, so at least one stays.
constexpr uint64_t kGraceTicks = 10000;      // 100 us of the 100 MHz real-time counter
constexpr uint64_t kStuckTicks = 200000000;  // 2 s: only a device fault gets here
constexpr int kWatch = kMaxFusedTiles / kThreads;  // start words read per thread
constexpr int kAggregators = 8;             // workgroups that read every tile's maxima
constexpr int kResCopies = 64;              // copies of the aggregators' results line
static_assert(kResCopies <= kThreads && 2 * kAggregators * sizeof(uint64_t) == 128 &&
                  (size_t)kResCopies * 2 * kAggregators <= 64 * 16,
              "one results line per copy, written by one thread each, inside the workspace");
constexpr uint64_t kFallbackTicks = 3000;   // 30 us without an aggregator's answer
constexpr int kPollBase = 64;                         // the pollers: waves 1..3
constexpr int kPollers = kThreads - kPollBase;
constexpr int kPollWatch = (kMaxFusedTiles + kPollers - 1) / kPollers;  // tiles watched per poller
static_assert(kThreads == 256 && kMaxFusedTiles % 64 == 0, "left-mask words from the pollers' ballots");

__device__ __forceinline__ uint64_t ld_agent(uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* a, uint64_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The generation tag: the low half of a tagged word.
__device__ __forceinline__ uint32_t ld_tag(uint64_t* a) {
  return __hip_atomic_load(reinterpret_cast<uint32_t*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t rt_now() { return __builtin_amdgcn_s_memrealtime(); }

// Per-tensor scales of both layouts from the tensor maxima, the inverse
// block-factor tables built from them (ends with a workgroup barrier).
template <bool RHT>
__device__ __forceinline__ void tensor_setup(float r, float c, float qmax, TensorScale& tsr, TensorScale& tsc,
                                             float (&lut)[2][128]) {
  tsr = make_tensor_scale<RHT>(r, qmax);
  tsc = make_tensor_scale<RHT>(c, qmax);
  const int t = threadIdx.x, l = t >> 7, cc = t & 127;
  const float S = l ? tsc.S : tsr.S;
  const float d = (cc == 127) ? 0.0f : e4m3_decode_pos((uint32_t)cc) * S;
  lut[l][cc] = (d == 0.0f) ? 0.0f : 1.0f / d;  // inverse dequantization factor per code
  __syncthreads();
}

// State of one workgroup's part in a single-pass exchange.
//
// A call's words carry its generation tag (the workspace's generation word
// + 1), so words left by earlier calls are never taken for this call's.
// Each workgroup marks its start in its tile's start words (kFsReplicas
// copies: every workgroup reads all of them once, and a copy per group of
// readers keeps any one memory line from having all of them as readers),
// and after phase A publishes its tile maxima in its tile's pair of words.
// The last kAggregators tiles' workgroups ("aggregators") read every tile's
// pair and publish the tensor maxima in a result pair of their own, written
// into every one of kResCopies copies of the results line; every other
// workgroup reads only its own copy.  (Many workgroups reading the same
// memory lines while they are written delays every one of those accesses
// by microseconds.)  When some tile was left, or
// no aggregator has answered within kFallbackTicks (an aggregator left its
// tile), a workgroup reads every tile's pair itself.
struct Exchange {
  uint64_t t_begin;
  uint32_t tag;      // this call's generation (never 0)
  int32_t n;         // tiles of the call
  uint64_t* w_start; // [kFsReplicas][n] start words
  uint64_t* w_max;   // [n][2] the tile's row-wise maximum (bit 31 of the value: tile
                     // left) and column-wise maximum, side by side
  uint64_t* w_res;   // [kResCopies][kAggregators][2]: the aggregators' result pairs
                     // (row-wise maximum, bit 31: some tile left; column-wise), in
                     // kResCopies copies of one 128-byte line each
  int32_t rep;       // the copy of the start words this workgroup reads
  int32_t agg;       // this workgroup's aggregator index, or -1
  int32_t copy;      // the copy of the results line this workgroup reads
};

// Start of a single-pass call: the call's generation and the tile's start
// words.  The first tile also clears a failure status an earlier call left.
__device__ __forceinline__ Exchange exchange_begin(const QuantParams& p, const TileInfo& T) {
  Exchange X;
  X.t_begin = rt_now();
  X.n = p.n_work;
  X.w_start = p.fs_words;
  X.w_max = X.w_start + (size_t)kFsReplicas * kMaxFusedTiles;
  X.w_res = X.w_max + 2 * (size_t)kMaxFusedTiles;
  X.rep = T.work % kFsReplicas;
  X.agg = T.work >= X.n - kAggregators ? X.n - 1 - T.work : -1;
  X.copy = T.work % kResCopies;
  const uint32_t tag = __hip_atomic_load(p.fs_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  X.tag = tag ? tag : 1u;
  if (threadIdx.x < kFsReplicas) st_agent(&X.w_start[threadIdx.x * X.n + T.work], X.tag);
  if (threadIdx.x == 0 && T.work == 0 && p.ws_status)
    __hip_atomic_store(p.ws_status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return X;
}

// Every tile's start word, kWatch tiles per thread (read half-way through
// phase A, when every workgroup that can start has long since written its
// own).  The loads are unconditional (a clamped index, the result selected
// afterwards): a load under a branch would make the compiler wait there for
// every load in flight, the tile's rows included.
__device__ __forceinline__ void exchange_read_starts(const Exchange& X, uint32_t (&sw)[kWatch]) {
#pragma unroll
  for (int k = 0; k < kWatch; ++k) {
    const int32_t i = (int32_t)threadIdx.x + k * kThreads;
    const uint32_t t = ld_tag(&X.w_start[X.rep * X.n + (i < X.n ? i : 0)]);
    sw[k] = i < X.n ? t : X.tag;
  }
}

// The exchange did not complete within kStuckTicks (only a device fault
// gets here): report it and advance the generation, so that the next call
// on this workspace never takes this call's words for its own.
__device__ __forceinline__ void exchange_abort(const QuantParams& p, const Exchange& X) {
  if (threadIdx.x == 0) {
    if (p.ws_status) __hip_atomic_store(p.ws_status, 7u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.fs_gen, X.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Waves 1..3 read every tile's pair of words until each carries this call's
// generation (wave 0 published: its loads would wait for its stores to
// complete).  A round re-reads only the tiles not seen yet, all of its loads
// issued before any of their results is used (a load under a per-lane
// branch would be waited for on its own).  Each poller accumulates the
// maxima of its tiles and their left bits (lbits bit k: tile
// pt + k kPollers).  False if stuck (the caller exits).
__device__ __forceinline__ bool poll_all_tiles(const QuantParams& p, const Exchange& X, float& r, float& c,
                                               uint32_t& lbits) {
  const int32_t n = X.n;
  const int32_t pt = (int32_t)threadIdx.x - kPollBase;  // poller index (negative in wave 0)
  uint32_t need = 0u;
#pragma unroll
  for (int k = 0; k < kPollWatch; ++k)
    if (pt >= 0 && pt + k * kPollers < n) need |= 1u << k;
  constexpr int kBatch = 3;  // tiles whose words are in flight at once (registers are short)
  for (;;) {
#pragma unroll
    for (int k0 = 0; k0 < kPollWatch; k0 += kBatch) {
      uint64_t a[kBatch], b[kBatch];
#pragma unroll
      for (int k = k0; k < k0 + kBatch && k < kPollWatch; ++k) {
        a[k - k0] = 0u;
        b[k - k0] = 0u;
        if (need & (1u << k)) {
          const int32_t i = pt + k * kPollers;
          a[k - k0] = ld_agent(&X.w_max[2 * i]);
          b[k - k0] = ld_agent(&X.w_max[2 * i + 1]);
        }
      }
#pragma unroll
      for (int k = k0; k < k0 + kBatch && k < kPollWatch; ++k) {
        if ((need & (1u << k)) && (uint32_t)a[k - k0] == X.tag && (uint32_t)b[k - k0] == X.tag) {
          const uint32_t hi = (uint32_t)(a[k - k0] >> 32);
          need &= ~(1u << k);
          lbits |= (hi >> 31) << k;
          r = fmaxf(r, __uint_as_float(hi & 0x7FFFFFFFu));
          c = fmaxf(c, __uint_as_float((uint32_t)(b[k - k0] >> 32)));
        }
      }
    }
    if (__syncthreads_and(need == 0u)) return true;
    if (__syncthreads_or(rt_now() - X.t_begin > kStuckTicks)) {
      exchange_abort(p, X);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Publish the tile maxima m (row-wise, column-wise; before the final 1/4)
// and collect the tensor's.  Returns false when this workgroup leaves its
// tile (some tile had not started within the grace period, or the host
// forced it) or the exchange never completed (status 7); the workgroup then
// exits.  On true, r and c hold the tensor maxima (the same in every lane),
// any_left tells whether some tile was left and then left_mask marks them.
__device__ __forceinline__ bool exchange_maxima(const QuantParams& p, const TileInfo& T, const Exchange& X,
                                                const uint32_t (&sw)[kWatch], float2 m, float& r_out, float& c_out,
                                                bool& any_left, uint64_t* left_mask, float (&red)[2][kThreads / 64]) {
  __shared__ uint32_t found;
  const int32_t n = X.n;
  bool ok = true;
#pragma unroll
  for (int k = 0; k < kWatch; ++k) ok = ok && sw[k] == X.tag;
  bool all = __syncthreads_and(ok) != 0;
  bool left = p.fs_orphan_stride > 1 && T.work % p.fs_orphan_stride != 0;
  // (the start-word polls issue all of a thread's loads back to back:
  // clamped indexes, results selected afterwards)
  const int nk = (n + kThreads - 1) / kThreads;  // watched tiles per thread (uniform)
  while (!all && !left) {
    if (__syncthreads_or(rt_now() - X.t_begin > kGraceTicks)) {
      left = true;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    uint32_t t[kWatch];
#pragma unroll
    for (int k = 0; k < kWatch; ++k) {
      const int32_t i = (int32_t)threadIdx.x + k * kThreads;
      if (k < nk) t[k] = ld_tag(&X.w_start[X.rep * n + (i < n ? i : n - 1)]);
    }
    ok = true;
#pragma unroll
    for (int k = 0; k < kWatch; ++k)
      if (k < nk && (int32_t)threadIdx.x + k * kThreads < n && t[k] != X.tag) ok = false;
    all = __syncthreads_and(ok) != 0;
  }
  if (threadIdx.x == 0) {
    st_agent(&X.w_max[2 * T.work + 1], (uint64_t)X.tag | ((uint64_t)__float_as_uint(m.y) << 32));
    st_agent(&X.w_max[2 * T.work],
             (uint64_t)X.tag | ((uint64_t)(__float_as_uint(m.x) | (left ? 0x80000000u : 0u)) << 32));
  }
  if (left) return false;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float r = 0.0f, c = 0.0f;
  uint32_t lbits = 0u;
  bool flat = X.agg >= 0;  // aggregators read every tile's words
  if (!flat) {
    // wave 1 reads the aggregators' results (lane a: aggregator a) until one
    // carries this call's generation
    const int na = n < kAggregators ? n : kAggregators;
    const uint64_t t_wait = rt_now();
    if (threadIdx.x == 0) found = 0u;
    __syncthreads();
    for (;;) {
      if (wave == 1) {
        uint64_t a = 0u, b = 0u;
        if (lane < na) {
          a = ld_agent(&X.w_res[2 * (kAggregators * X.copy + lane)]);
          b = ld_agent(&X.w_res[2 * (kAggregators * X.copy + lane) + 1]);
        }
        const bool valid = lane < na && (uint32_t)a == X.tag && (uint32_t)b == X.tag;
        const uint64_t vm = __ballot(valid);
        if (vm) {
          const int src = __builtin_ctzll(vm);
          const uint32_t hi = (uint32_t)(__shfl(a, src) >> 32);
          r = __uint_as_float(hi & 0x7FFFFFFFu);
          c = __uint_as_float((uint32_t)(__shfl(b, src) >> 32));
          if (lane == 0) found = (hi >> 31) ? 2u : 1u;  // 2: some tile was left
        }
      }
      __syncthreads();
      if (found) break;
      if (__syncthreads_or(rt_now() - t_wait > kFallbackTicks)) break;  // (an aggregator left its tile)
      __builtin_amdgcn_s_sleep(1);
    }
    flat = found != 1u;  // no answer, or tiles were left: read every tile's words
    if (flat) {
      r = 0.0f;
      c = 0.0f;
    }
  }
  if (flat && !poll_all_tiles(p, X, r, c, lbits)) return false;
  r = wave_max(r);
  c = wave_max(c);
  any_left = flat && __syncthreads_or(lbits != 0u) != 0;
  if (any_left && wave > 0) {
    // poller p = 64 (wave - 1) + lane watches tiles p + 192 k: wave w's k-th
    // ballot covers tiles 64 (w - 1 + 3 k) .. +63
#pragma unroll
    for (int k = 0; k < kPollWatch; ++k) {
      const uint64_t bits = __ballot((lbits >> k) & 1u);
      if (lane == 0 && (wave - 1 + 3 * k) < kMaxFusedTiles / 64) left_mask[wave - 1 + 3 * k] = bits;
    }
  }
  if (lane == 0) {
    red[0][wave] = r;
    red[1][wave] = c;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    r = fmaxf(r, red[0][i]);
    c = fmaxf(c, red[1][i]);
  }
  if (X.agg >= 0 && threadIdx.x < kResCopies) {
    uint64_t* res = &X.w_res[2 * (kAggregators * threadIdx.x + X.agg)];
    st_agent(&res[1], (uint64_t)X.tag | ((uint64_t)__float_as_uint(c) << 32));
    st_agent(&res[0], (uint64_t)X.tag | ((uint64_t)(__float_as_uint(r) | (any_left ? 0x80000000u : 0u)) << 32));
  }
  // the same in every lane: keep the tensor quantities in scalar registers
  r_out = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r)));
  c_out = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c)));
  return true;
}

// The number of tiles that were left and this tile's rank among the ones
// that stay.  The staying tile of rank 0 (at least one tile always stays)
// advances the generation word: every workgroup has read it by now, so one
// writer suffices (stores from all workgroups to one word serialize at the
// memory and hold up each writer's following stores by microseconds).
__device__ __forceinline__ void exchange_ranks(const QuantParams& p, const TileInfo& T, const Exchange& X,
                                               bool any_left, const uint64_t* left_mask, int32_t& n_left,
                                               int32_t& q) {
  n_left = 0;
  int32_t below = 0;
  for (int j = 0; any_left && j < (X.n + 63) / 64; ++j) {
    const uint64_t mk = left_mask[j];
    n_left += __popcll(mk);
    if (64 * j + 63 < T.work) below += __popcll(mk);
    else if (64 * j < T.work) below += __popcll(mk & ((1ull << (T.work - 64 * j)) - 1ull));
  }
  q = T.work - below;
  if (threadIdx.x == 0 && q == 0) __hip_atomic_store(p.fs_gen, X.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Writes the per-tensor scales once per call (by the tile at the origin).
__device__ __forceinline__ void write_tensor_scales(const QuantParams& p, const TileInfo& T, const TensorScale& tsr,
                                                    const TensorScale& tsc) {
  if (threadIdx.x == 0 && T.band == 0 && T.m0 == 0) {
    if (p.do_row && p.row_ts) p.row_ts[0] = tsr.S;
    if (p.do_col && p.col_ts) p.col_ts[0] = tsc.S;
  }
}

// The tiles that were left: the q-th (by index) goes to the staying tile of
// rank q mod (number staying), which reloads and quantizes it.
template <int GRID, bool SR, bool RHT>
__device__ __forceinline__ void quantize_left_tiles(const QuantParams& p, const Exchange& X, const uint64_t* left_mask,
                                                    int32_t n_left, int32_t q, const TensorScale& tsr,
                                                    const TensorScale& tsc, const float (&lut)[2][128], ColStage& cst,
                                                    int32_t& pick) {
  const int32_t n = X.n, n_stay = n - n_left;
  for (; q < n_left; q += n_stay) {
    if (threadIdx.x == 0) {
      int32_t want = q, o = -1;
      for (int j = 0; j < (n + 63) / 64 && o < 0; ++j) {
        uint64_t mk = left_mask[j];
        const int cnt = __popcll(mk);
        if (want < cnt) {
          for (; want > 0; --want) mk &= mk - 1ull;
          o = 64 * j + (int)__builtin_ctzll(mk);
        } else {
          want -= cnt;
        }
      }
      pick = o;
    }
    __syncthreads();  // also: the previous tile's write-out has read the staging area
    const TileInfo U = dense_tile(p, pick);
    if (!U.active) break;  // (not reached: the q-th left tile exists for q < n_left)
    // Lane geometry re-derived through an opaque copy, so the compiler
    // recomputes the lane-dependent values inside this rarely used loop
    // instead of holding them in registers across the own tile's pass.
    LaneGeom LU = lane_geom(p, U);
    asm volatile("" : "+v"(LU.lc), "+v"(LU.lane), "+v"(LU.half), "+v"(LU.wave));
    LU.m_h0 = U.m0 + 32 * LU.wave + 16 * LU.half;
    LU.c0 = (int64_t)U.band * kBandCols + 8 * LU.lc;
    LU.lane_ok = LU.c0 < p.cols;
    uint32_t w[16][4];
    load_rows<0, 16, true>(p, U, LU, w);
    write_tensor_scales(p, U, tsr, tsc);
    quant_tile<GRID, SR, false, RHT, false>(p, U, LU, w, tsr, tsc, lut, cst);
  }
}

// LDS of the one-kernel variants: the tile's raw rows, kept from phase A to
// phase B, share their space with the column-wise staging area, which is
// used only after the rows have been read back.
constexpr size_t kFusedTileLds = 16 * kThreads * sizeof(uint4);
static_assert(sizeof(ColStage) <= kFusedTileLds, "staging area fits the tile buffer");

// The single pass for either layout alone: phase A's maxima, then both
// transforms computed again from the rows kept in LDS.
template <int GRID, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads, 2) void ufp4_fused_kernel(QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t big[kFusedTileLds];
  __shared__ float lut[2][128];
  __shared__ float red[2][kThreads / 64];
  __shared__ uint64_t left_mask[kMaxFusedTiles / 64];
  __shared__ int32_t pick;
  uint4 (&wl)[16][kThreads] = *reinterpret_cast<uint4 (*)[16][kThreads]>(big);
  ColStage& cst = *reinterpret_cast<ColStage*>(big);
  const TileInfo T = dense_tile(p, remap_xcd((int32_t)blockIdx.x, (int32_t)gridDim.x));
  if (!T.active) return;  // uniform per workgroup; owns no tile
  const Exchange X = exchange_begin(p, T);
  const LaneGeom L = lane_geom(p, T);
  uint32_t w[16][4];
  load_rows<0, 16, true>(p, T, L, w);
  uint32_t sw[kWatch];
  const float2 m = tile_amax<RHT>(p, L, w, red, [&] { exchange_read_starts(X, sw); },
                                  [&](int i) { wl[i][threadIdx.x] = make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]); });
  float r, c;
  bool any_left;
  if (!exchange_maxima(p, T, X, sw, m, r, c, any_left, left_mask, red)) return;
  constexpr float qmax = grid_qmax<GRID>();
  TensorScale tsr, tsc;
  tensor_setup<RHT>(r, c, qmax, tsr, tsc, lut);
  int32_t n_left, q;
  exchange_ranks(p, T, X, any_left, left_mask, n_left, q);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 u = wl[i][threadIdx.x];
    w[i][0] = u.x;
    w[i][1] = u.y;
    w[i][2] = u.z;
    w[i][3] = u.w;
  }
  __syncthreads();  // the staging area reuses the rows' space
  write_tensor_scales(p, T, tsr, tsc);
  quant_tile<GRID, SR, false, RHT>(p, T, L, w, tsr, tsc, lut, cst);
  quantize_left_tiles<GRID, SR, RHT>(p, X, left_mask, n_left, q, tsr, tsc, lut, cst, pick);
}

// Phase A of the row+column single pass.  As each row of the lane's 16 x 8
// sub-tile arrives it is stored raw to LDS (wl, for phase B's row-wise
// pass), its row-wise half blocks are transformed for their maxima only
// (the last butterfly stage folds into the maximum, as in tile_amax), and
// the column-wise butterflies advance one stage whenever the rows they pair
// are present.  After the last row the column-wise blocks are completed and
// KEPT: cv holds the lane's 8 transformed columns (before the final 1/4;
// the raw columns without the transform), cmax their block maxima, rmax the
// 16 row-wise block maxima (over the lane pair).  Returns the workgroup's
// tile maxima (row-wise, column-wise) in every thread.
template <bool RHT, typename Mid>
__device__ __forceinline__ float2 tile_amax_keep(const QuantParams& p, const LaneGeom& L, const uint32_t (&w)[16][4],
                                                 uint4 (&wl)[16][kThreads], float (&cv)[16][8], float (&rmax)[16],
                                                 float (&cmax)[8], float (&red)[2][kThreads / 64], Mid&& mid) {
  float acc_r = 0.0f, acc_c = 0.0f;
  const RowLaneSigns rs = row_lane_signs<RHT>(p, L.lc & 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    wl[i][threadIdx.x] = make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cv[i][2 * k] = bf_lo(w[i][k]);
      cv[i][2 * k + 1] = bf_hi(w[i][k]);
    }
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = cv[i][j];
    float mr = 0.0f;
    if (RHT) {
      fwht8_half(v, rs.h);
#pragma unroll
      for (int j = 0; j < 8; ++j) mr = lastpair_max(mr, v[j], dpp_xor1(v[j]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) mr = fmaxf(mr, fabsf(v[j]));
      mr = fmaxf(mr, dpp_xor1(mr));
    }
    rmax[i] = mr;
    acc_r = fmaxf(acc_r, mr);
    if (i == 8) mid();
    if (RHT) {
      if (i % 2 == 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) bfly(cv[i - 1][c], cv[i][c], p.sg.q1[i / 2]);
      }
      if (i % 4 == 3) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          bfly(cv[i - 3][c], cv[i - 1][c], p.sg.q2[i / 4]);
          bfly(cv[i - 2][c], cv[i][c], p.sg.q2[i / 4]);
        }
      }
      if (i % 8 == 7) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int c = 0; c < 8; ++c) bfly(cv[i - 7 + j][c], cv[i - 3 + j][c], p.sg.q3[i / 8]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (RHT) {
#pragma unroll
      for (int j = 0; j < 8; ++j) bfly(cv[j][c], cv[j + 8][c], p.sg.q4);
    }
    float mc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) mc = fmaxf(mc, fabsf(cv[i][c]));
    cmax[c] = mc;
    acc_c = fmaxf(acc_c, mc);
  }
  acc_r = wave_max(acc_r);
  acc_c = wave_max(acc_c);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = acc_r;
    red[1][threadIdx.x >> 6] = acc_c;
  }
  __syncthreads();
  float r = red[0][0], c = red[1][0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) {
    r = fmaxf(r, red[0][i]);
    c = fmaxf(c, red[1][i]);
  }
  return make_float2(r, c);
}

// The single pass for the row+column call (dense NV16).  Phase A transforms
// each column-wise block once and keeps the result in registers across the
// exchange, so phase B rounds the column-wise layout without recomputing it
// and recomputes only the row-wise transform, from the raw rows kept in LDS.
// Every block maximum is kept from phase A as well.
template <int GRID, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads, 2) void ufp4_single_kernel(QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t big[kFusedTileLds];
  __shared__ ColStageT<4> cst;  // the own tile's column-wise staging, half the columns at a time
  __shared__ float lut[2][128];
  __shared__ float red[2][kThreads / 64];
  __shared__ uint64_t left_mask[kMaxFusedTiles / 64];
  __shared__ int32_t pick;
  uint4 (&wl)[16][kThreads] = *reinterpret_cast<uint4 (*)[16][kThreads]>(big);
  ColStage& full = *reinterpret_cast<ColStage*>(big);  // reloaded tiles' staging, once the rows are read
  const TileInfo T = dense_tile(p, remap_xcd((int32_t)blockIdx.x, (int32_t)gridDim.x));
  if (!T.active) return;  // uniform per workgroup; owns no tile
  const Exchange X = exchange_begin(p, T);
  const LaneGeom L = lane_geom(p, T);
  float cv[16][8], rmax[16], cmax[8];
  uint32_t sw[kWatch];
  {
    uint32_t w[16][4];
    load_rows<0, 16, true>(p, T, L, w);
    const float2 m = tile_amax_keep<RHT>(p, L, w, wl, cv, rmax, cmax, red, [&] { exchange_read_starts(X, sw); });
    float r, c;
    bool any_left;
    if (!exchange_maxima(p, T, X, sw, m, r, c, any_left, left_mask, red)) return;
    constexpr float qmax = grid_qmax<GRID>();
    TensorScale tsr, tsc;
    tensor_setup<RHT>(r, c, qmax, tsr, tsc, lut);
    int32_t n_left, q;
    exchange_ranks(p, T, X, any_left, left_mask, n_left, q);
    write_tensor_scales(p, T, tsr, tsc);
    // column-wise first: it consumes the kept values, which frees their
    // registers for the row-wise pass; half the columns at a time, so the
    // staging area fits beside the raw rows
    auto col_src = [&](int k, float(&v)[16]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = cv[i][k];
      return cmax[k];
    };
    col_pass<GRID, SR, false, RHT, false, 0, 4>(p, T, L, tsc, lut[1], cst, col_src);
    __syncthreads();  // the first half's write-out has read the staging area
    col_pass<GRID, SR, false, RHT, false, 4, 4>(p, T, L, tsc, lut[1], cst, col_src);
    // the lane's row-wise signs, derived again through an opaque copy of
    // its parity rather than held in registers since phase A
    int parity = L.lc & 1;
    asm volatile("" : "+v"(parity));
    const RowLaneSigns rs = row_lane_signs<RHT>(p, parity);
    row_pass<GRID, SR, false, RHT, false, SR ? 2 : 4>(
        p, T, L, tsr, lut[0], rs.fin, [&](int i, float(&v)[8]) __attribute__((always_inline)) {
          const uint4 u = wl[i][threadIdx.x];
          v[0] = bf_lo(u.x);
          v[1] = bf_hi(u.x);
          v[2] = bf_lo(u.y);
          v[3] = bf_hi(u.y);
          v[4] = bf_lo(u.z);
          v[5] = bf_hi(u.z);
          v[6] = bf_lo(u.w);
          v[7] = bf_hi(u.w);
          if (RHT) {
            fwht8_half(v, rs.h);
            cross_stage8(v, rs.s4);
          }
          return rmax[i];
        });
    if (n_left > 0) {
      __syncthreads();  // every row has been read back: the tile area is free for reloaded tiles' staging
      quantize_left_tiles<GRID, SR, RHT>(p, X, left_mask, n_left, q, tsr, tsc, lut, full, pick);
    }
  }
}

__global__ void ufp4_fill_kernel(uint32_t* p, int64_t n, uint32_t value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// ---------------------------------------------------------------- host side
// A kernel launch; with timing events, through hipExtLaunchKernelGGL, which
// stamps the two events with the kernel's own start and end.
template <typename K>
static void launch(K kernel, const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (t0 || t1)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, t0, t1, 0u, p);
  else
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
}

hipError_t launch_amax(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (p.rht)
    launch(ufp4_amax_kernel<true>, p, grid, s, t0, t1);
  else
    launch(ufp4_amax_kernel<false>, p, grid, s, t0, t1);
  return hipGetLastError();
}

template <int GRID, bool SR, bool MX>
static void launch_quant_rht(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (p.rht)
    launch(ufp4_quant_kernel<GRID, SR, MX, true>, p, grid, s, t0, t1);
  else
    launch(ufp4_quant_kernel<GRID, SR, MX, false>, p, grid, s, t0, t1);
}

template <int GRID, bool MX>
static hipError_t launch_quant_grid(const QuantParams& p, int64_t grid, bool sr, hipStream_t s, hipEvent_t t0,
                                    hipEvent_t t1) {
  if (sr)
    launch_quant_rht<GRID, true, MX>(p, grid, s, t0, t1);
  else
    launch_quant_rht<GRID, false, MX>(p, grid, s, t0, t1);
  return hipGetLastError();
}

template <int GRID>
static hipError_t launch_quant_mx(const QuantParams& p, int64_t grid, bool sr, hipStream_t s, hipEvent_t t0,
                                  hipEvent_t t1) {
  return p.mx ? launch_quant_grid<GRID, true>(p, grid, sr, s, t0, t1)
              : launch_quant_grid<GRID, false>(p, grid, sr, s, t0, t1);
}

hipError_t launch_quant(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const bool sr = p.sr != 0;
  switch (p.grid) {
    case kGridE1M2: return launch_quant_mx<kGridE1M2>(p, grid, sr, s, t0, t1);
    case kGridINT4: return launch_quant_mx<kGridINT4>(p, grid, sr, s, t0, t1);
    case kGridE2M1: return launch_quant_mx<kGridE2M1>(p, grid, sr, s, t0, t1);
    case kGridE2M1C: return launch_quant_mx<kGridE2M1C>(p, grid, sr, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

template <int GRID, bool SR>
static void launch_fused_rht(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  // both layouts: the variant that keeps the column-wise transform
  if (p.do_row && p.do_col) {
    if (p.rht)
      launch(ufp4_single_kernel<GRID, SR, true>, p, grid, s, t0, t1);
    else
      launch(ufp4_single_kernel<GRID, SR, false>, p, grid, s, t0, t1);
  } else if (p.rht) {
    launch(ufp4_fused_kernel<GRID, SR, true>, p, grid, s, t0, t1);
  } else {
    launch(ufp4_fused_kernel<GRID, SR, false>, p, grid, s, t0, t1);
  }
}

template <int GRID>
static hipError_t launch_fused_grid(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (p.sr)
    launch_fused_rht<GRID, true>(p, grid, s, t0, t1);
  else
    launch_fused_rht<GRID, false>(p, grid, s, t0, t1);
  return hipGetLastError();
}

template <int GRID, bool SR>
static void launch_delayed_rht(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (p.rht)
    launch(ufp4_delayed_kernel<GRID, SR, true>, p, grid, s, t0, t1);
  else
    launch(ufp4_delayed_kernel<GRID, SR, false>, p, grid, s, t0, t1);
}

template <int GRID>
static hipError_t launch_delayed_grid(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0,
                                      hipEvent_t t1) {
  if (p.sr)
    launch_delayed_rht<GRID, true>(p, grid, s, t0, t1);
  else
    launch_delayed_rht<GRID, false>(p, grid, s, t0, t1);
  return hipGetLastError();
}

hipError_t launch_delayed(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  switch (p.grid) {
    case kGridE1M2: return launch_delayed_grid<kGridE1M2>(p, grid, s, t0, t1);
    case kGridINT4: return launch_delayed_grid<kGridINT4>(p, grid, s, t0, t1);
    case kGridE2M1: return launch_delayed_grid<kGridE2M1>(p, grid, s, t0, t1);
    case kGridE2M1C: return launch_delayed_grid<kGridE2M1C>(p, grid, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

template <int GRID>
static hipError_t launch_grouped_delayed_grid(const QuantParams& p, int64_t grid, hipStream_t s) {
  if (p.sr) {
    if (p.rht) launch(ufp4_grouped_delayed_kernel<GRID, true, true>, p, grid, s, nullptr, nullptr);
    else launch(ufp4_grouped_delayed_kernel<GRID, true, false>, p, grid, s, nullptr, nullptr);
  } else {
    if (p.rht) launch(ufp4_grouped_delayed_kernel<GRID, false, true>, p, grid, s, nullptr, nullptr);
    else launch(ufp4_grouped_delayed_kernel<GRID, false, false>, p, grid, s, nullptr, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_delayed(const QuantParams& p, int64_t grid, hipStream_t s) {
  switch (p.grid) {
    case kGridE1M2: return launch_grouped_delayed_grid<kGridE1M2>(p, grid, s);
    case kGridINT4: return launch_grouped_delayed_grid<kGridINT4>(p, grid, s);
    case kGridE2M1: return launch_grouped_delayed_grid<kGridE2M1>(p, grid, s);
    case kGridE2M1C: return launch_grouped_delayed_grid<kGridE2M1C>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fused(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  switch (p.grid) {
    case kGridE1M2: return launch_fused_grid<kGridE1M2>(p, grid, s, t0, t1);
    case kGridINT4: return launch_fused_grid<kGridINT4>(p, grid, s, t0, t1);
    case kGridE2M1: return launch_fused_grid<kGridE2M1>(p, grid, s, t0, t1);
    case kGridE2M1C: return launch_fused_grid<kGridE2M1C>(p, grid, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_roof(const QuantParams& p, int64_t grid, hipStream_t s) {
  launch(ufp4_roof_kernel, p, grid, s, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_fill(uint32_t* ptr, int64_t n, uint32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(ufp4_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ptr, n, value);
  return hipGetLastError();
}

}  // namespace ufp4
