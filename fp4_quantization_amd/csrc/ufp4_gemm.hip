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
// The expansion is byte arithmetic: every grid value's fp16 encoding has a
// zero low byte, so one byte permute looks the high bytes of four codes up in
// an 8-entry table, an OR adds their signs, a second permute interleaves the
// zero low bytes, and a packed fp16 multiply applies the block scale.
#include <hip/hip_runtime.h>

#include "ufp4_internal.hpp"

namespace ufp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t g32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t g32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmM = 128, kGemmN = 128, kGemmK = 32;
constexpr int kGemmLd = kGemmK + 8;  // fp16 per LDS row: 80 bytes, 16-byte aligned rows

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
  // high bytes of the even (low-nibble) and odd (high-nibble) elements
  const uint32_t he = __builtin_amdgcn_perm(hi, lo, word & 0x07070707u) | ((word << 4) & 0x80808080u);
  const uint32_t ho = __builtin_amdgcn_perm(hi, lo, (word >> 4) & 0x07070707u) | (word & 0x80808080u);
  // (element 2i, element 2i+1) = (0x00, he.byte i, 0x00, ho.byte i); selector
  // 0x0C gives a zero byte, 0..3 the bytes of he, 4..7 those of ho
  out[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x040C000Cu)) * d2);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x050C010Cu)) * d2);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x060C020Cu)) * d2);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(ho, he, 0x070C030Cu)) * d2);
}

// One 16-element block: 8 code bytes and its E4M3 scale byte, to 16 fp16
// values at dst (16-byte aligned).
template <int GRID>
__device__ __forceinline__ void dequant16(g32x2 codes, uint32_t sbyte, _Float16* dst) {
  const _Float16 d = (_Float16)e4m3_decode_pos(sbyte & 0x7Fu);  // exact: E4M3 values are fp16 values
  const f16x2 d2 = {d, d};
  uint32_t o[8];
  expand8<GRID>(codes.x, d2, o);
  expand8<GRID>(codes.y, d2, o + 4);
  g32x4* p = reinterpret_cast<g32x4*>(dst);
  p[0] = g32x4{o[0], o[1], o[2], o[3]};
  p[1] = g32x4{o[4], o[5], o[6], o[7]};
}

// Grid: (ceil(N/128), ceil(M/128)); 256 threads.  Wave w computes the 64 x 64
// sub-tile at rows 64 (w / 2), columns 64 (w % 2), as 2 x 2 MFMA tiles of
// 32 x 32.  Per K step of 32 each thread expands one block of A (row t / 2,
// block t % 2 of the step) and one of B; the next step's codes are loaded
// while the current step multiplies.
template <int GRID>
__global__ __launch_bounds__(kThreads) void ufp4_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 As[kGemmM][kGemmLd];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[kGemmN][kGemmLd];
  const int64_t m0 = (int64_t)blockIdx.y * kGemmM, n0 = (int64_t)blockIdx.x * kGemmN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int lr = t >> 1, lb = t & 1;
  const int64_t am = m0 + lr, bn = n0 + lr;
  const bool a_ok = am < p.M, b_ok = bn < p.N;
  const int64_t kc = p.K / 2, ks = p.K / 16;
  // rows outside the matrices read row 0 and are zeroed below
  const uint8_t* ac = p.a_codes + (a_ok ? am : 0) * kc + 8 * lb;
  const uint8_t* as = p.a_scales + (a_ok ? am : 0) * ks + lb;
  const uint8_t* bc = p.b_codes + (b_ok ? bn : 0) * kc + 8 * lb;
  const uint8_t* bs = p.b_scales + (b_ok ? bn : 0) * ks + lb;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  g32x2 na = {0u, 0u}, nb = {0u, 0u};
  uint32_t nsa = 0u, nsb = 0u;
  if (p.K > 0) {
    na = *reinterpret_cast<const g32x2*>(ac);
    nb = *reinterpret_cast<const g32x2*>(bc);
    nsa = as[0];
    nsb = bs[0];
  }
  for (int64_t k0 = 0; k0 < p.K; k0 += kGemmK) {
    const g32x2 ca = a_ok ? na : g32x2{0u, 0u}, cb = b_ok ? nb : g32x2{0u, 0u};
    const uint32_t sa = nsa, sb = nsb;
    if (k0 + kGemmK < p.K) {
      const int64_t k1 = k0 + kGemmK;
      na = *reinterpret_cast<const g32x2*>(ac + k1 / 2);
      nb = *reinterpret_cast<const g32x2*>(bc + k1 / 2);
      nsa = as[k1 / 16];
      nsb = bs[k1 / 16];
    }
    __syncthreads();  // the previous step's fragments have been read
    dequant16<GRID>(ca, sa, &As[lr][16 * lb]);
    dequant16<GRID>(cb, sb, &Bs[lr][16 * lb]);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *reinterpret_cast<const f16x8*>(&As[wm + 32 * i + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
        fb[i] = *reinterpret_cast<const f16x8*>(&Bs[wn + 32 * i + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
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
        if (row < p.M && col < p.N) p.c[row * p.ldc + col] = acc[i][j][r] * s;
      }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.N + kGemmN - 1) / kGemmN), (unsigned)((p.M + kGemmM - 1) / kGemmM));
  switch (p.grid) {
    case kGridE1M2: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridE1M2>, grid, dim3(kThreads), 0, s, p); break;
    case kGridINT4: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridINT4>, grid, dim3(kThreads), 0, s, p); break;
    case kGridE2M1: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridE2M1>, grid, dim3(kThreads), 0, s, p); break;
    case kGridE2M1C: hipLaunchKernelGGL(ufp4_gemm_kernel<kGridE2M1C>, grid, dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ufp4
