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
// Dequantization is exact in bf16: a grid value (at most 3 significant
// bits: k/2, k or an E2M1 value) times an E4M3 block scale (4 significant
// bits) needs at most 7 bits, within bf16's 8.  So each workgroup expands its
// operand tiles to bf16 in LDS, multiplies them on the bf16 MFMA with fp32
// accumulation, and applies the two tensor scales in the epilogue.  Results
// differ from an exact sum only by the fp32 accumulation order.
#include <hip/hip_runtime.h>

#include "ufp4_internal.hpp"

namespace ufp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t g32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t g32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmM = 128, kGemmN = 128, kGemmK = 32;
constexpr int kGemmLd = kGemmK + 8;  // bf16 per LDS row: 80 bytes, 16-byte aligned rows

// Two dequantized values as one bf16 pair (exact: at most 7 significant bits).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One 16-element block: 8 code bytes (element 2i in the low nibble of byte
// i) and its E4M3 scale byte, to 16 bf16 values at dst (16-byte aligned).
template <int GRID>
__device__ __forceinline__ void dequant16(g32x2 codes, uint32_t sbyte, __bf16* dst) {
  const float d = e4m3_decode_pos(sbyte & 0x7Fu);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t word = i < 4 ? codes.x : codes.y;
    const uint32_t c0 = (word >> (8 * (i & 3))) & 15u, c1 = (word >> (8 * (i & 3) + 4)) & 15u;
    o[i] = pack_bf16(code_value<GRID>(c0) * d, code_value<GRID>(c1) * d);
  }
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
  __shared__ __attribute__((aligned(16))) __bf16 As[kGemmM][kGemmLd];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[kGemmN][kGemmLd];
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
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *reinterpret_cast<const bf16x8*>(&As[wm + 32 * i + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
        fb[i] = *reinterpret_cast<const bf16x8*>(&Bs[wn + 32 * i + (lane & 31)][16 * kk + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
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
