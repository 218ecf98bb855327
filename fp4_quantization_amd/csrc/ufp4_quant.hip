// ufp4_quant.hip -- the fused RHT + 4-bit quantization kernels for gfx950.
//
// Two phases per call (the per-tensor scale makes every code depend on the
// absolute maximum of the whole transformed tensor):
//   phase A (ufp4_amax_kernel): load tiles, transform row-wise and
//     column-wise blocks, keep the largest magnitude; every workgroup writes
//     a partial, and the last workgroup to finish reduces them per segment
//     into the per-tensor scales S_t = amax / (Qmax * 448)
//     ([Z] "Key points": fused RHT+quantization; the two-level NVFP4-style
//     scale is named there and in [H] technical approach);
//   phase B (ufp4_quant_kernel): reload the tile, transform again, compute
//     the block scales, round ([Z] fix / [A] "The UFP4 Recipe": E1M2 or INT4,
//     SR only where requested) and store packed codes and scales for both
//     layouts from the same registers.
//
// Mapping.  A lane holds a 16-row x 8-column sub-tile (one 16-byte load per
// row).  Row-wise blocks (16 consecutive columns) span a lane pair: stages of
// half-width 1, 2, 4 run in-lane, the stage of half-width 8 pairs lanes l and
// l^1 through a DPP quad permutation.  Column-wise blocks (16 consecutive
// rows) are entirely in-lane.  No LDS transpose is needed: the same loaded
// registers feed both layouts.  Workgroups are remapped so that the ones
// dispatched to one XCD (round-robin over 8) walk down one column band, so
// the transposed outputs they write share L2 lines.
#include "ufp4_internal.hpp"

namespace ufp4 {

struct TileInfo {
  bool active;
  bool bad;
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
  int32_t bad;
  int32_t seg;
};

__device__ __forceinline__ int32_t remap_xcd(int32_t b, int32_t nblocks) {
  // nblocks is a multiple of kNumXcd: workgroup b runs on XCD b % 8.
  const int32_t per = nblocks / kNumXcd;
  return (b % kNumXcd) * per + b / kNumXcd;
}

// Resolve the workgroup's tile.  For grouped calls every workgroup scans the
// offsets (at most kMaxGroups+1 values) into LDS and validates them.
__device__ TileInfo tile_info(const QuantParams& p, GroupLds& g) {
  TileInfo T;
  T.bad = false;
  const int32_t w = remap_xcd((int32_t)blockIdx.x, (int32_t)gridDim.x);
  T.active = w < p.n_work;
  T.band = T.active ? w / p.n_tiles : 0;
  const int32_t t = T.active ? w % p.n_tiles : 0;
  if (p.offsets == nullptr) {
    T.seg = 0;
    T.seg_row0 = 0;
    T.M = p.rows;
    T.P = (p.rows + p.block - 1) / p.block * p.block;
    T.coff = 0;
    T.m0 = (int64_t)t * kTileRows;
    T.active = T.active && T.m0 < T.P;
    return T;
  }
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
  for (int s = 1; s < E; s <<= 1) {
    int64_t a = 0;
    int32_t b = 0;
    const int i = tid + 1;
    if (tid < E && tid >= s) {
      a = g.ppre[i - s];
      b = g.tpre[i - s];
    }
    __syncthreads();
    if (tid < E && tid >= s) {
      g.ppre[i] += a;
      g.tpre[i] += b;
    }
    __syncthreads();
  }
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

// Load the lane's 16 x 8 sub-tile (zeros outside the segment / tensor).
__device__ __forceinline__ void load_tile(const QuantParams& p, const TileInfo& T, const LaneGeom& L,
                                          uint32_t w[16][4]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t m = L.m_h0 + i;
    if (L.lane_ok && m < T.M) {
      const uint4 v = *reinterpret_cast<const uint4*>(p.x + (T.seg_row0 + m) * p.ld + L.c0);
      w[i][0] = v.x;
      w[i][1] = v.y;
      w[i][2] = v.z;
      w[i][3] = v.w;
    } else {
      w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0u;
    }
  }
}

// Folded signs of the lane's half of a row-wise block (selected by lane
// parity once per kernel, so the butterflies read registers, not memory).
struct RowLaneSigns {
  HalfSigns h;
  float s4;   // multiplier of the partner value in the cross-lane stage
  float fin;  // output multiplier (0.25 d0, and -q4 on odd lanes)
};

__device__ __forceinline__ RowLaneSigns row_lane_signs(const QuantParams& p, int parity) {
  RowLaneSigns r;
  const bool odd = parity != 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) r.h.q1[k] = odd ? p.hs[1].q1[k] : p.hs[0].q1[k];
#pragma unroll
  for (int k = 0; k < 2; ++k) r.h.q2[k] = odd ? p.hs[1].q2[k] : p.hs[0].q2[k];
  r.h.q3 = odd ? p.hs[1].q3 : p.hs[0].q3;
  r.s4 = odd ? p.s4[1] : p.s4[0];
  r.fin = p.rht ? (odd ? p.fin_lane[1] : p.fin_lane[0]) : 1.0f;
  return r;
}

// Row-wise transform of one row of the sub-tile: the lane's 8 values of the
// block's transform, before the lane's output multiplier.
__device__ __forceinline__ void row_transform(const QuantParams& p, const uint32_t wi[4],
                                              const RowLaneSigns& rs, float v[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf_lo(wi[k]);
    v[2 * k + 1] = bf_hi(wi[k]);
  }
  if (p.rht) {
    fwht8_half(v, rs.h);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(dpp_xor1(v[j]), rs.s4, v[j]);
  }
}

__device__ __forceinline__ void col_transform(const QuantParams& p, const uint32_t w[16][4], int k,
                                              float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (k & 1) ? bf_hi(w[i][k >> 1]) : bf_lo(w[i][k >> 1]);
  if (p.rht) fwht16_inlane(v, p.sg);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------- phase A
__global__ __launch_bounds__(kThreads) void ufp4_amax_kernel(QuantParams p) {
  __shared__ GroupLds g;
  __shared__ float red[2][kThreads / 64];
  __shared__ uint32_t seg_max[2][kMaxGroups];
  __shared__ int32_t is_last;
  const TileInfo T = tile_info(p, g);
  float acc_r = 0.0f, acc_c = 0.0f;
  if (T.active) {
    const LaneGeom L = lane_geom(p, T);
    uint32_t w[16][4];
    load_tile(p, T, L, w);
    if (p.do_row) {
      const RowLaneSigns rs = row_lane_signs(p, L.lc & 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v[8];
        row_transform(p, w[i], rs, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc_r = fmaxf(acc_r, fabsf(v[j]));
      }
    }
    if (p.do_col) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float v[16];
        col_transform(p, w, k, v);
#pragma unroll
        for (int j = 0; j < 16; ++j) acc_c = fmaxf(acc_c, fabsf(v[j]));
      }
    }
  }
  acc_r = wave_max(acc_r);
  acc_c = wave_max(acc_c);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = acc_r;
    red[1][wave] = acc_c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0][0], c = red[1][0];
    for (int i = 1; i < kThreads / 64; ++i) {
      r = fmaxf(r, red[0][i]);
      c = fmaxf(c, red[1][i]);
    }
    p.ws_part[blockIdx.x] = make_float4(T.active ? (float)T.seg : -1.0f, r, c, 0.0f);
    const uint32_t prev =
        __hip_atomic_fetch_add(p.ws_counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!is_last) return;
  // Last workgroup: reduce the partials per segment and publish the scales.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int E = p.num_groups;
  for (int i = threadIdx.x; i < E; i += kThreads) {
    seg_max[0][i] = 0u;
    seg_max[1][i] = 0u;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (int)gridDim.x; i += kThreads) {
    const float4 q = p.ws_part[i];
    const int e = (int)q.x;
    if (e >= 0 && e < E) {
      atomicMax(&seg_max[0][e], __float_as_uint(q.y));  // non-negative: bit order = value order
      atomicMax(&seg_max[1][e], __float_as_uint(q.z));
    }
  }
  __syncthreads();
  const float qmax448 = qmax_of(p.grid) * 448.0f;
  for (int e = threadIdx.x; e < E; e += kThreads) {
#pragma unroll
    for (int l = 0; l < 2; ++l) {
      float a = __uint_as_float(seg_max[l][e]);
      if (p.rht) a = a * 0.25f;  // max of the scaled values (monotone rounding)
      const float S = (a > 0.0f) ? a / qmax448 : 1.0f;
      p.ws_scale[2 * e + l] = S;
      if (l == 0 && p.do_row && p.row_ts && !T.bad) p.row_ts[e] = S;
      if (l == 1 && p.do_col && p.col_ts && !T.bad) p.col_ts[e] = S;
    }
  }
  if (threadIdx.x == 0) {
    *p.ws_status = T.bad ? 6u : 0u;
    __hip_atomic_store(p.ws_counter, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- phase B
template <int GRID, bool SR>
__global__ __launch_bounds__(kThreads) void ufp4_quant_kernel(QuantParams p) {
  __shared__ GroupLds g;
  __shared__ float lut[2][128];
  const TileInfo T = tile_info(p, g);
  if (p.mx && blockIdx.x == 0 && (p.offsets == nullptr || !T.bad)) {
    for (int e = threadIdx.x; e < p.num_groups; e += kThreads) {
      if (p.do_row && p.row_ts) p.row_ts[e] = 1.0f;
      if (p.do_col && p.col_ts) p.col_ts[e] = 1.0f;
    }
  }
  if (!T.active) return;  // uniform per workgroup
  const float qmax = grid_qmax<GRID>();
  float D[2] = {0.0f, 0.0f};
  if (!p.mx) {
    const float S0 = p.ws_scale[2 * T.seg + 0], S1 = p.ws_scale[2 * T.seg + 1];
    D[0] = qmax * S0;
    D[1] = qmax * S1;
    const int t = threadIdx.x;
    const int l = t >> 7, c = t & 127;
    const float S = l ? S1 : S0;
    // inverse dequantization factor of every E4M3 block-scale code
    const float d = (c == 127) ? 0.0f : e4m3_decode_pos((uint32_t)c) * S;
    lut[l][c] = (d == 0.0f) ? 0.0f : 1.0f / d;
    __syncthreads();
  }
  const LaneGeom L = lane_geom(p, T);
  uint32_t w[16][4];
  load_tile(p, T, L, w);
  const int parity = L.lc & 1;
  const RowLaneSigns rs = row_lane_signs(p, parity);
  const float fin_r = rs.fin;
  const float fin_c = p.rht ? p.sg.fin : 1.0f;
  const int64_t C = p.cols;

  if (p.do_row) {
#pragma clang loop unroll(full)
    for (int i = 0; i < 16; ++i) {
      float v[8];
      row_transform(p, w[i], rs, v);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = v[j] * fin_r;
        m = fmaxf(m, fabsf(v[j]));
      }
      m = fmaxf(m, dpp_xor1(m));
      if (p.mx) m = fmaxf(m, dpp_xor2(m));
      uint32_t sbyte;
      float inv;
      if (p.mx) {
        mx_scale<GRID>(m, sbyte, inv);
      } else {
        sbyte = e4m3_encode_sat(m / D[0]);
        inv = lut[0][sbyte];
      }
      const int64_t grow = T.seg_row0 + L.m_h0 + i;
      uint32_t packed = 0u;
      if (SR) {
        const uint64_t base = (uint64_t)grow * (uint64_t)C + (uint64_t)L.c0;
        const Ctr4 r0 = sr_words4(base >> 2, 0u, p.sr_k0, p.sr_k1);
        const Ctr4 r1 = sr_words4((base >> 2) + 1, 0u, p.sr_k0, p.sr_k1);
        packed = quantize_code<GRID, true>(v[0] * inv, r0.x) | (quantize_code<GRID, true>(v[1] * inv, r0.y) << 4) |
                 (quantize_code<GRID, true>(v[2] * inv, r0.z) << 8) | (quantize_code<GRID, true>(v[3] * inv, r0.w) << 12) |
                 (quantize_code<GRID, true>(v[4] * inv, r1.x) << 16) | (quantize_code<GRID, true>(v[5] * inv, r1.y) << 20) |
                 (quantize_code<GRID, true>(v[6] * inv, r1.z) << 24) | (quantize_code<GRID, true>(v[7] * inv, r1.w) << 28);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) packed |= quantize_code<GRID, false>(v[j] * inv, 0u) << (4 * j);
      }
      if (L.lane_ok && L.m_h0 + i < T.M) {
        *reinterpret_cast<uint32_t*>(p.row_codes + grow * (C / 2) + L.c0 / 2) = packed;
        if (p.mx) {
          if ((L.lc & 3) == 0) p.row_scales[grow * (C / 32) + L.c0 / 32] = (uint8_t)sbyte;
        } else if (parity == 0) {
          p.row_scales[grow * (C / 16) + L.c0 / 16] = (uint8_t)sbyte;
        }
      }
    }
  }

  if (p.do_col) {
    const bool blk_ok = L.m_h0 < T.P;  // this half's 16-row block exists
    const int64_t Rp = p.padded_rows;
    const int64_t pos0 = T.coff + L.m_h0;  // column-wise position of the block start
#pragma clang loop unroll(full)
    for (int k = 0; k < 8; ++k) {
      float v[16];
      col_transform(p, w, k, v);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[j] = v[j] * fin_c;
        m = fmaxf(m, fabsf(v[j]));
      }
      if (p.mx) m = fmaxf(m, __shfl_xor(m, 32));
      uint32_t sbyte;
      float inv;
      if (p.mx) {
        mx_scale<GRID>(m, sbyte, inv);
      } else {
        sbyte = e4m3_encode_sat(m / D[1]);
        inv = lut[1][sbyte];
      }
      const int64_t c = L.c0 + k;
      uint32_t lo = 0u, hi = 0u;
      if (SR) {
        const uint64_t base = (uint64_t)c * (uint64_t)Rp + (uint64_t)pos0;
        uint32_t word[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const Ctr4 r = sr_words4((base >> 2) + q, 1u, p.sr_k0, p.sr_k1);
          word[q] = quantize_code<GRID, true>(v[4 * q + 0] * inv, r.x) |
                    (quantize_code<GRID, true>(v[4 * q + 1] * inv, r.y) << 4) |
                    (quantize_code<GRID, true>(v[4 * q + 2] * inv, r.z) << 8) |
                    (quantize_code<GRID, true>(v[4 * q + 3] * inv, r.w) << 12);
        }
        lo = word[0] | (word[1] << 16);
        hi = word[2] | (word[3] << 16);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) lo |= quantize_code<GRID, false>(v[j] * inv, 0u) << (4 * j);
#pragma unroll
        for (int j = 0; j < 8; ++j) hi |= quantize_code<GRID, false>(v[8 + j] * inv, 0u) << (4 * j);
      }
      if (L.lane_ok && blk_ok) {
        *reinterpret_cast<uint2*>(p.col_codes + c * (Rp / 2) + pos0 / 2) = make_uint2(lo, hi);
        if (p.mx) {
          if (L.half == 0) p.col_scales[c * (Rp / 32) + pos0 / 32] = (uint8_t)sbyte;
        } else {
          p.col_scales[c * (Rp / 16) + pos0 / 16] = (uint8_t)sbyte;
        }
      }
    }
  }
}

__global__ void ufp4_fill_kernel(uint32_t* p, int64_t n, uint32_t value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// ---------------------------------------------------------------- host side
uint32_t rht_sign_mask(uint64_t seed) {
  // word 0 of Philox4x32-10(key = seed, counter = (0, 0, 2, 0))
  uint32_t c0 = 0, c1 = 0, c2 = 2, c3 = 0;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = (uint64_t)0xD2511F53u * c0, b = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(b >> 32) ^ c1 ^ k0, n1 = (uint32_t)b;
    const uint32_t n2 = (uint32_t)(a >> 32) ^ c3 ^ k1, n3 = (uint32_t)a;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0 & 0xFFFFu;
}

void fill_rht_signs(uint64_t seed, QuantParams& p) {
  const uint32_t mask = rht_sign_mask(seed);
  float d[16];
  for (int j = 0; j < 16; ++j) d[j] = ((mask >> j) & 1u) ? -1.0f : 1.0f;
  RhtSigns& S = p.sg;
  for (int q = 0; q < 8; ++q) S.q1[q] = d[2 * q] * d[2 * q + 1];
  for (int g = 0; g < 4; ++g) S.q2[g] = d[4 * g] * d[4 * g + 2];
  for (int g = 0; g < 2; ++g) S.q3[g] = d[8 * g] * d[8 * g + 4];
  S.q4 = d[0] * d[8];
  S.fin = 0.25f * d[0];
  for (int h = 0; h < 2; ++h) {
    for (int q = 0; q < 4; ++q) p.hs[h].q1[q] = S.q1[4 * h + q];
    for (int g = 0; g < 2; ++g) p.hs[h].q2[g] = S.q2[2 * h + g];
    p.hs[h].q3 = S.q3[h];
  }
  // stage 4 across a lane pair: the even lane (positions 0..7) computes
  // a + q4 b; the odd lane computes b - q4 a = -q4 (a - q4 b).
  p.s4[0] = S.q4;
  p.s4[1] = -S.q4;
  p.fin_lane[0] = S.fin;
  p.fin_lane[1] = S.fin * -S.q4;
}

int64_t grid_size_quant(int64_t rows, int64_t cols, int32_t groups, int32_t block, int32_t* n_band,
                        int32_t* n_tiles) {
  const int64_t nb = (cols + kBandCols - 1) / kBandCols;
  int64_t nt;
  if (groups <= 1) {
    const int64_t P = (rows + block - 1) / block * block;
    nt = (P + kTileRows - 1) / kTileRows;
  } else {
    // sum over segments of ceil(roundup(M_e, B) / 128) <= ceil((rows + B*E)/128) + E
    nt = (rows + (int64_t)block * groups + kTileRows - 1) / kTileRows + groups;
  }
  if (nt < 1) nt = 1;
  *n_band = (int32_t)nb;
  *n_tiles = (int32_t)nt;
  const int64_t work = nb * nt;
  return (work + kNumXcd - 1) / kNumXcd * kNumXcd;
}

hipError_t launch_amax(const QuantParams& p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL(ufp4_amax_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int GRID>
static hipError_t launch_quant_grid(const QuantParams& p, int64_t grid, bool sr, hipStream_t s) {
  if (sr)
    hipLaunchKernelGGL((ufp4_quant_kernel<GRID, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((ufp4_quant_kernel<GRID, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_quant(const QuantParams& p, int64_t grid, hipStream_t s) {
  const bool sr = p.sr != 0;
  switch (p.grid) {
    case kGridE1M2: return launch_quant_grid<kGridE1M2>(p, grid, sr, s);
    case kGridINT4: return launch_quant_grid<kGridINT4>(p, grid, sr, s);
    case kGridE2M1: return launch_quant_grid<kGridE2M1>(p, grid, sr, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill(uint32_t* ptr, int64_t n, uint32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(ufp4_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ptr, n, value);
  return hipGetLastError();
}

}  // namespace ufp4
