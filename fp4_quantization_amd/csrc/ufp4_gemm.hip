// ufp4_gemm.hip -- the consumer GEMM of two NV16-quantized operands on gfx950.
//
// C[m][n] = sum_k xa[m][k] * xb[n][k], where xa and xb are the dequantized
// row-wise layouts of an M x K and an N x K matrix (blocks of 16 along K,
// the GEMM reduction dimension, as the quantizer lays them out for the
// fwd_y, bwd_dx and bwd_dw products; [Z] "Key points": the fix quantizes
// the operands of all three training GEMMs).  Operands quantized with the
// same RHT signs multiply to the product of the untransformed matrices, the
// transform being orthonormal.
//
// Dequantization is exact in fp16: a grid value (at most 3 significant
// bits: k/2, k or an E2M1 value) times an E4M3 block scale (4 significant
// bits) needs at most 7 bits and lies in [2^-10, 2688], inside fp16's normal
// range.  So each workgroup expands its operand tiles to fp16 in LDS,
// multiplies them on the fp16 MFMA with fp32 accumulation (the products are
// exact), and applies the two tensor scales in the epilogue.  Results differ
// from an exact sum only by the fp32 accumulation order.
//
// Tiles are 256 x 256 per workgroup of 8 waves, K steps of 64, with two LDS
// buffers: each step first expands the next step's codes into the other
// buffer, then multiplies from its own, and ends in one barrier.
//
// The expansion is byte arithmetic: every grid value's fp16 encoding has a
// zero low byte, so one byte permute looks the high bytes of four codes up in
// an 8-entry table, a three-input bitwise op adds their signs, a second
// permute interleaves the zero low bytes, and a packed fp16 multiply applies
// the block scale.
#include <hip/hip_runtime.h>

#include "ufp4_internal.hpp"

namespace ufp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t g32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t g32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmM = 256, kGemmN = 256, kGemmK = 64;
constexpr int kGemmLd = kGemmK + 8;  // fp16 per LDS row: 144 bytes, 16-byte aligned rows

// High bytes of the fp16 encodings of the grid magnitudes by magnitude
// index (low word: indices 0..3, high word: 4..7).
template <int GRID>
__device__ __forceinline__ uint32_t f16_hi_lo() {
  return GRID == kGridINT4 ? 0x42403C00u : 0x3E3C3800u;  // {0, 1, 2, 3} / {0, .5, 1, 1.5}
}
template <int GRID>
__device__ __forceinline__ uint32_t f16_hi_hi() {
  return GRID == kGridE1M2 ? 0x43424140u    // 2, 2.5, 3, 3.5
         : GRID == kGridINT4 ? 0x47464544u  // 4, 5, 6, 7
                             : 0x46444240u; // 2, 3, 4, 6 (E2M1; the clamped grid uses 0..4)
}

// Two's-complement nibbles -> sign-magnitude nibbles, eight at a time (for
// a negative nibble n, |n| = (n ^ 7) + 1 with the sign bit kept).
__device__ __forceinline__ uint32_t signmag8(uint32_t P) {
  const uint32_t A = P & 0x88888888u, S = A >> 3;
  return (P ^ (A - S)) + S;
}

// Eight codes (element 2i in the low nibble of byte i) to four fp16 pairs
// times the block scale d2 = (d, d).
template <int GRID>
__device__ __forceinline__ void expand8(uint32_t word, f16x2 d2, uint32_t out[4]) {
  if (GRID == kGridINT4) word = signmag8(word);
  const uint32_t lo = f16_hi_lo<GRID>(), hi = f16_hi_hi<GRID>();
  // high bytes of the even (low-nibble) and odd (high-nibble) elements; the
  // sign bits are merged by one three-input bitwise op, a | (b & c)
  // (truth table 0xF8)
  const uint32_t he = (uint32_t)__builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(hi, lo, word & 0x07070707u),
                                                             word << 4, 0x80808080u, 0xF8);
  const uint32_t ho = (uint32_t)__builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(hi, lo, (word >> 4) & 0x07070707u),
                                                             word, 0x80808080u, 0xF8);
  // (element 2i, element 2i+1) = (0x00, he.byte i, 0x00, ho.byte i); selector
  // 0x0C gives a zero byte, 0..3 the bytes of he, 4..7 those of ho
  out[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x040C000Cu)) * d2);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x050C010Cu)) * d2);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x060C020Cu)) * d2);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x070C030Cu)) * d2);
}

// One 16-element block: 8 code bytes and its E4M3 scale byte, to 16 fp16
// values (eight words, element 2i in the low half of word i).
template <int GRID>
__device__ __forceinline__ void expand16(g32x2 codes, uint32_t sbyte, uint32_t o[8]) {
  // the hardware OCP E4M3 decode of the (non-negative) scale byte; exact,
  // and every E4M3 value is an fp16 value
  const _Float16 d = (_Float16)__builtin_amdgcn_cvt_pk_f32_fp8((int)(sbyte & 0x7Fu), false)[0];
  const f16x2 d2 = {d, d};
  expand8<GRID>(codes.x, d2, o);
  expand8<GRID>(codes.y, d2, o + 4);
}

// The 16 fp16 values of a block to dst (16-byte aligned).
__device__ __forceinline__ void store16(const uint32_t o[8], _Float16* dst) {
  g32x4* p = reinterpret_cast<g32x4*>(dst);
  p[0] = g32x4{o[0], o[1], o[2], o[3]};
  p[1] = g32x4{o[4], o[5], o[6], o[7]};
}

// Grid: (ceil(N/256), ceil(M/256)); 512 threads (8 waves).  Wave w computes
// the 64 x 128 sub-tile at rows 64 (w / 2), columns 128 (w % 2), as 2 x 4
// MFMA tiles of 32 x 32.  Per K step of 64 each thread stages two adjacent
// blocks of A (row t / 2, blocks 2 (t % 2) and 2 (t % 2) + 1 of the step: 16
// code bytes, one load) and two of B.  At the 144-byte row pitch both the
// fragment reads (consecutive rows) and these stores (two threads per row)
// fall on distinct LDS banks.  The expanded tiles are double-buffered: at
// the start of a step the next step's codes (requested one step earlier)
// are expanded and stored into the other buffer, the step after that is
// requested, then this step multiplies, and the step ends in one barrier.
constexpr int kGemmThreads = 512;

template <int GRID>
__global__ __launch_bounds__(kGemmThreads) void ufp4_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kGemmM][kGemmLd];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][kGemmN][kGemmLd];
  const int64_t m0 = (int64_t)blockIdx.y * kGemmM, n0 = (int64_t)blockIdx.x * kGemmN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 128;
  const int lr = t >> 1, lb = 2 * (t & 1);
  const int64_t am = m0 + lr, bn = n0 + lr;
  const bool a_ok = am < p.M, b_ok = bn < p.N;
  const int64_t kc = p.K / 2, ks = p.K / 16;
  const uint8_t* ac = p.a_codes + (a_ok ? am : 0) * kc + 8 * lb;
  const uint8_t* as = p.a_scales + (a_ok ? am : 0) * ks + lb;
  const uint8_t* bc = p.b_codes + (b_ok ? bn : 0) * kc + 8 * lb;
  const uint8_t* bs = p.b_scales + (b_ok ? bn : 0) * ks + lb;
  const int64_t nsteps = (p.K + kGemmK - 1) / kGemmK;
  struct Stage {
    g32x4 a, b;
    uint32_t sa, sb;
  };
  auto fetch = [&](int64_t st) {
    Stage f;
    const bool in = st * kGemmK + 16 * lb + 32 <= p.K;
    const int64_t off = in ? st * (kGemmK / 2) : 0, so = in ? st * (kGemmK / 16) : 0;
    f.a = (in && a_ok) ? *reinterpret_cast<const g32x4*>(ac + off) : g32x4{0u, 0u, 0u, 0u};
    f.b = (in && b_ok) ? *reinterpret_cast<const g32x4*>(bc + off) : g32x4{0u, 0u, 0u, 0u};
    f.sa = (in && a_ok) ? ((uint32_t)as[so] | ((uint32_t)as[so + 1] << 8)) : 0u;
    f.sb = (in && b_ok) ? ((uint32_t)bs[so] | ((uint32_t)bs[so + 1] << 8)) : 0u;
    return f;
  };
  auto put = [&](const Stage& f, int buf) {
    uint32_t e[8];
    expand16<GRID>(g32x2{f.a.x, f.a.y}, f.sa & 0xFFu, e);
    store16(e, &As[buf][lr][16 * lb]);
    expand16<GRID>(g32x2{f.a.z, f.a.w}, f.sa >> 8, e);
    store16(e, &As[buf][lr][16 * lb + 16]);
    expand16<GRID>(g32x2{f.b.x, f.b.y}, f.sb & 0xFFu, e);
    store16(e, &Bs[buf][lr][16 * lb]);
    expand16<GRID>(g32x2{f.b.z, f.b.w}, f.sb >> 8, e);
    store16(e, &Bs[buf][lr][16 * lb + 16]);
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  if (nsteps > 0) put(fetch(0), 0);
  Stage nxt = fetch(nsteps > 1 ? 1 : 0);
  __syncthreads();
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = (int)(st & 1);
    if (st + 1 < nsteps) {
      put(nxt, cur ^ 1);
      if (st + 2 < nsteps) nxt = fetch(st + 2);
    }
#pragma unroll
    for (int kk = 0; kk < kGemmK / 16; ++kk) {
      f16x8 fa[2], fb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const f16x8*>(&As[cur][wm + 32 * i + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const f16x8*>(&Bs[cur][wn + 32 * j + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  const float s = p.a_ts[0] * p.b_ts[0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn + 32 * j + (lane & 31);
        if (row < p.M && col < p.N) __builtin_nontemporal_store(acc[i][j][r] * s, &p.c[row * p.ldc + col]);
      }
}

// ------------------------------------------------------------------ MX32
// MX32 operands multiply on the scaled f8f6f4 MFMA (32 x 32 x 64, fp32
// accumulation), which takes one E8M0 scale per 32 elements along K per
// operand row: exactly the MX32 block scale, so no dequantization happens
// outside the matrix core.  Operand formats: E2M1 codes (and E2M1C codes,
// whose magnitudes 0..2 are E2M1 values with the same encodings) are OCP
// FP4 values as stored; E1M2 (k/2) and INT4 (k) values are exact in OCP FP8
// E4M3 and are expanded to it byte by byte.  The products of the scaled
// values are exact (a few significant bits times powers of two inside fp32's
// range), so c differs from the exact sum only by the accumulation order.
//
// Lane layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured on gfx950 with
// an in-bounds probe against a host model): lane l holds row (column of B)
// l % 32 and 32 values of the 64-element K slice; FP4: K positions
// 32 (l / 32) .. +31 in nibble order; FP8: 16 (l / 32) .. +15 in bytes 0..15
// and 32 + 16 (l / 32) .. +15 in bytes 16..31; its scale register holds the
// E8M0 byte of block l / 32 of the slice for that row.  The 32 x 32 result
// is laid out as for the other 32 x 32 MFMAs.
//
// Tiles are 256 x 256 per workgroup of 16 waves (each 64 x 64 as 2 x 2 MFMA
// tiles: 64 accumulator registers, so four waves fit per SIMD), K steps of
// 256 (FP4) or 128 (FP8) values, double-buffered in LDS: each thread stages
// one half of one A row (threads 0..511) or one B row (512..1023) per step,
// requested one step ahead.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kMxThreads = 1024;  // 16 waves: 4 x 4 wave tiles of 64 x 64

template <int GRID>
struct MxFmt {
  static constexpr bool kFp4 = GRID == kGridE2M1 || GRID == kGridE2M1C;
  static constexpr int kFmt = kFp4 ? 4 : 0;      // cbsz / blgp: FP4 E2M1 or FP8 E4M3
  static constexpr int kK = kFp4 ? 256 : 128;    // K values per step (per barrier)
  static constexpr int kSlices = kK / 64;        // MFMA K slices per step
  static constexpr int kBlocks = kK / 64;        // MX blocks each thread stages per operand row half
  static constexpr int kRowBytes = kFp4 ? kK / 2 : kK;  // one step of one row in LDS
  static constexpr int kPitch = kRowBytes + 16;  // LDS row pitch (spreads fragment reads over banks)
};

// Eight codes (element 2i in the low nibble of byte i) to eight E4M3 bytes
// (element e in byte e of out[e / 4]) for E1M2 (k/2) or INT4 (k); the sign
// bit of a code becomes the E4M3 sign (a negative zero stays zero).
template <int GRID>
__device__ __forceinline__ void expand8_e4m3(uint32_t word, uint32_t out[2]) {
  if (GRID == kGridINT4) word = signmag8(word);
  // E4M3 encodings of the magnitudes 0..7 (low word 0..3, high word 4..7)
  const uint32_t lo = GRID == kGridINT4 ? 0x44403800u : 0x3C383000u;  // {0,1,2,3} / {0,.5,1,1.5}
  const uint32_t hi = GRID == kGridINT4 ? 0x4E4C4A48u : 0x46444240u;  // {4..7} / {2,2.5,3,3.5}
  const uint32_t he = (uint32_t)__builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(hi, lo, word & 0x07070707u),
                                                             word << 4, 0x80808080u, 0xF8);
  const uint32_t ho = (uint32_t)__builtin_amdgcn_bitop3_b32(__builtin_amdgcn_perm(hi, lo, (word >> 4) & 0x07070707u),
                                                             word, 0x80808080u, 0xF8);
  out[0] = __builtin_amdgcn_perm(ho, he, 0x05010400u);  // elements 0..3
  out[1] = __builtin_amdgcn_perm(ho, he, 0x07030602u);  // elements 4..7
}

template <int GRID>
__global__ __launch_bounds__(kMxThreads) void ufp4_gemm_mx_kernel(GemmParams p) {
  using Fm = MxFmt<GRID>;
  __shared__ __attribute__((aligned(16))) uint8_t As[2][kGemmM][Fm::kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kGemmN][Fm::kPitch];
  // [buffer][operand][row][block of the step], read back one row at a time
  __shared__ __attribute__((aligned(8))) uint8_t Ss[2][2][kGemmM][Fm::kK / 32];
  constexpr int SW = Fm::kK / 128;  // 32-bit words of scale bytes per row and step
  constexpr int NB = Fm::kBlocks;   // MX blocks per thread and operand per step
  const int64_t m0 = (int64_t)blockIdx.y * kGemmM, n0 = (int64_t)blockIdx.x * kGemmN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wm = (wave >> 2) * 64, wn = (wave & 3) * 64;
  const int op = t >> 9;                   // operand this thread stages: 0 A, 1 B
  const int lr = (t & 511) >> 1, h = t & 1;  // staged row, half of the K step
  const int64_t am = m0 + lr, bn = n0 + lr;
  const bool a_ok = am < p.M && op == 0, b_ok = bn < p.N && op == 1;
  const int64_t kc = p.K / 2, ks = p.K / 32;
  const uint8_t* ac = p.a_codes + (a_ok ? am : 0) * kc + 16 * NB * h;
  const uint8_t* as = p.a_scales + (a_ok ? am : 0) * ks + NB * h;
  const uint8_t* bc = p.b_codes + (b_ok ? bn : 0) * kc + 16 * NB * h;
  const uint8_t* bs = p.b_scales + (b_ok ? bn : 0) * ks + NB * h;
  const int64_t nsteps = (p.K + Fm::kK - 1) / Fm::kK;
  // codes of the thread's NB blocks (16 bytes each) of its operand row and
  // their scale bytes; a block past K (or a row past M / N) is zero with
  // scale 2^0
  struct Stage {
    g32x4 c[NB];
    uint8_t sc[NB];
  };
  const uint8_t* src = op == 0 ? ac : bc;
  const uint8_t* ss = op == 0 ? as : bs;
  const bool ok = op == 0 ? a_ok : b_ok;
  auto fetch = [&](int64_t st) {
    Stage f;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      // addresses stay inside the operands whether or not the load is used
      const bool in = st * Fm::kK + 32 * NB * h + 32 * q + 32 <= p.K;
      const int64_t off = in ? st * (Fm::kK / 2) + 16 * q : 0;
      const int64_t so = in ? st * (Fm::kK / 32) + q : 0;
      f.c[q] = (in && ok) ? *reinterpret_cast<const g32x4*>(src + off) : g32x4{0u, 0u, 0u, 0u};
      f.sc[q] = (in && ok) ? ss[so] : (uint8_t)127;
    }
    return f;
  };
  auto put_row = [&](const g32x4 (&c)[NB], uint8_t* dst) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      if (Fm::kFp4) {
        reinterpret_cast<g32x4*>(dst)[q] = c[q];
      } else {
        uint32_t e[8];
        expand8_e4m3<GRID>(c[q].x, e);
        expand8_e4m3<GRID>(c[q].y, e + 2);
        expand8_e4m3<GRID>(c[q].z, e + 4);
        expand8_e4m3<GRID>(c[q].w, e + 6);
        reinterpret_cast<g32x4*>(dst)[2 * q] = g32x4{e[0], e[1], e[2], e[3]};
        reinterpret_cast<g32x4*>(dst)[2 * q + 1] = g32x4{e[4], e[5], e[6], e[7]};
      }
    }
  };
  auto put = [&](const Stage& f, int buf) {
    constexpr int half_bytes = Fm::kRowBytes / 2;
    put_row(f.c, op == 0 ? &As[buf][lr][half_bytes * h] : &Bs[buf][lr][half_bytes * h]);
#pragma unroll
    for (int q = 0; q < NB; ++q) Ss[buf][op][lr][NB * h + q] = f.sc[q];
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  if (nsteps > 0) put(fetch(0), 0);
  Stage nxt = fetch(nsteps > 1 ? 1 : 0);
  __syncthreads();
  const int g = lane >> 5, r32 = lane & 31;
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = (int)(st & 1);
    // stage the next step into the other buffer (last read before the
    // previous barrier) and request the one after; the staging registers
    // are free again before the fragments of this step are read
    if (st + 1 < nsteps) {
      put(nxt, cur ^ 1);
      if (st + 2 < nsteps) nxt = fetch(st + 2);
    }
    // the step's scale bytes of the lane's rows, shifted so that the byte of
    // slice kk's block for this lane's half (block 2 kk + g) sits at byte
    // 2 (kk % 2) of word kk / 2, which the MFMA's scale byte select takes
    uint32_t swa[2][SW], swb[2][SW];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < SW; ++q)
        swa[i][q] = reinterpret_cast<const uint32_t*>(&Ss[cur][0][wm + 32 * i + r32][0])[q] >> (8 * g);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < SW; ++q)
        swb[j][q] = reinterpret_cast<const uint32_t*>(&Ss[cur][1][wn + 32 * j + r32][0])[q] >> (8 * g);
#pragma unroll
    for (int kk = 0; kk < Fm::kSlices; ++kk) {
      i32x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm + 32 * i + r32;
        if (Fm::kFp4) {
          const g32x4 v = *reinterpret_cast<const g32x4*>(&As[cur][row][32 * kk + 16 * g]);
          fa[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        } else {
          const g32x4 v0 = *reinterpret_cast<const g32x4*>(&As[cur][row][64 * kk + 16 * g]);
          const g32x4 v1 = *reinterpret_cast<const g32x4*>(&As[cur][row][64 * kk + 32 + 16 * g]);
          fa[i] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn + 32 * j + r32;
        if (Fm::kFp4) {
          const g32x4 v = *reinterpret_cast<const g32x4*>(&Bs[cur][row][32 * kk + 16 * g]);
          fb[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        } else {
          const g32x4 v0 = *reinterpret_cast<const g32x4*>(&Bs[cur][row][64 * kk + 16 * g]);
          const g32x4 v1 = *reinterpret_cast<const g32x4*>(&Bs[cur][row][64 * kk + 32 + 16 * g]);
          fb[j] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (kk & 1)  // (the byte select must be a constant: kk is unrolled)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], Fm::kFmt, Fm::kFmt,
                                                                        2, (int)swa[i][kk >> 1], 2, (int)swb[j][kk >> 1]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], Fm::kFmt, Fm::kFmt,
                                                                        0, (int)swa[i][kk >> 1], 0, (int)swb[j][kk >> 1]);
    }
    __syncthreads();
  }
  const float s = p.a_ts[0] * p.b_ts[0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn + 32 * j + (lane & 31);
        if (row < p.M && col < p.N) __builtin_nontemporal_store(acc[i][j][r] * s, &p.c[row * p.ldc + col]);
      }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.N + kGemmN - 1) / kGemmN), (unsigned)((p.M + kGemmM - 1) / kGemmM));
  if (p.mx) {
    switch (p.grid) {
      case kGridE1M2: hipLaunchKernelGGL(ufp4_gemm_mx_kernel<kGridE1M2>, grid, dim3(kMxThreads), 0, s, p); break;
      case kGridINT4: hipLaunchKernelGGL(ufp4_gemm_mx_kernel<kGridINT4>, grid, dim3(kMxThreads), 0, s, p); break;
      case kGridE2M1: hipLaunchKernelGGL(ufp4_gemm_mx_kernel<kGridE2M1>, grid, dim3(kMxThreads), 0, s, p); break;
      case kGridE2M1C: hipLaunchKernelGGL(ufp4_gemm_mx_kernel<kGridE2M1C>, grid, dim3(kMxThreads), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (p.grid) {
    case kGridE1M2: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridE1M2>, grid, dim3(kGemmThreads), 0, s, p); break;
    case kGridINT4: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridINT4>, grid, dim3(kGemmThreads), 0, s, p); break;
    case kGridE2M1: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridE2M1>, grid, dim3(kGemmThreads), 0, s, p); break;
    case kGridE2M1C: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridE2M1C>, grid, dim3(kGemmThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ufp4
