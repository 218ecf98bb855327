// ufp4_misc.hip -- dequantization, statistics, the unit-scale rounding hook
// and the fp32 -> bf16 conversion between the layers of a quantized chain
// (gfx950).  None of these is on the quantization hot path.
#include "ufp4_internal.hpp"

namespace ufp4 {

__device__ __forceinline__ float e4m3_decode_full(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15u && m == 7u) return __builtin_nanf("");
  const float v = e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
  return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------- dequantize
// xhat = value(code) * d_b; with the inverse transform: the butterfly on xhat,
// then 1/4, then the signs (the transform is its own inverse up to D).
template <int GRID>
__global__ __launch_bounds__(256) void ufp4_dequant_kernel(DequantParams p) {
  const int64_t per_line = p.cols / 16;
  const int64_t nb = p.rows * per_line;
  const int B = p.mx ? 32 : 16;
  const float S = p.mx ? 1.0f : p.ts[0];
  RhtSigns plain;
#pragma unroll
  for (int k = 0; k < 8; ++k) plain.q1[k] = 1.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) plain.q2[k] = 1.0f;
  plain.q3[0] = plain.q3[1] = 1.0f;
  plain.q4 = 1.0f;
  plain.fin = 0.25f;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t l = b / per_line, j0 = (b % per_line) * 16;
    const int64_t o0 = l * p.cols + j0;
    const uint2 cw = *reinterpret_cast<const uint2*>(p.codes + o0 / 2);
    const uint32_t s = p.scales[o0 / B];
    const float d = p.mx ? ldexpf(1.0f, (int)s - 127) : e4m3_decode_full(s) * S;
    float v[16];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = code_value<GRID>(cw.x >> (4 * t)) * d;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[8 + t] = code_value<GRID>(cw.y >> (4 * t)) * d;
    if (p.inverse) {
      fwht16_inlane(v, plain);
#pragma unroll
      for (int t = 0; t < 16; ++t) v[t] = v[t] * (0.25f * p.d[t]);
    }
    float4* o = reinterpret_cast<float4*>(p.out + o0);
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

hipError_t launch_dequant(const DequantParams& p, hipStream_t s) {
  const int64_t nb = p.rows * (p.cols / 16);
  if (nb <= 0) return hipSuccess;
  int64_t blocks = (nb + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  switch (p.grid) {
    case kGridE1M2: hipLaunchKernelGGL(ufp4_dequant_kernel<kGridE1M2>, dim3((unsigned)blocks), dim3(256), 0, s, p); break;
    case kGridINT4: hipLaunchKernelGGL(ufp4_dequant_kernel<kGridINT4>, dim3((unsigned)blocks), dim3(256), 0, s, p); break;
    case kGridE2M1: hipLaunchKernelGGL(ufp4_dequant_kernel<kGridE2M1>, dim3((unsigned)blocks), dim3(256), 0, s, p); break;
    case kGridE2M1C: hipLaunchKernelGGL(ufp4_dequant_kernel<kGridE2M1C>, dim3((unsigned)blocks), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- statistics
// One thread per scale block; binary64 sums per thread, reduced per
// workgroup into a partial; the host adds the partials in workgroup order.
template <int GRID>
__global__ __launch_bounds__(256) void ufp4_stats_kernel(StatsParams p) {
  __shared__ double red[256];
  __shared__ uint32_t hist[16];
  const int B = p.mx ? 32 : 16;
  const int64_t lines = p.layout == 0 ? p.rows : p.cols;
  const int64_t len = p.layout == 0 ? p.cols : p.rows;
  const int64_t per_line = len / B;
  const int64_t nb = lines * per_line;
  const float qmax = grid_qmax<GRID>();
  const float S = p.mx ? 1.0f : p.ts[0];
  double a_v2 = 0, a_e2 = 0, a_vx = 0, a_se = 0, a_seg = 0, a_max = 0;
  uint64_t n = 0, n_grid = 0, n_zero = 0, n_sat = 0, n_nf = 0;
  if (threadIdx.x < 16) hist[threadIdx.x] = 0u;
  __syncthreads();
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb;
       b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t l = b / per_line, j0 = (b % per_line) * B;
    const int64_t o0 = l * len + j0;
    const uint32_t s = p.scales[o0 / B];
    const float d = p.mx ? ldexpf(1.0f, (int)s - 127) : e4m3_decode_full(s) * S;
    const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
    for (int h = 0; h < B; h += 16) {
      float v[16], xin[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int64_t j = j0 + h + t;
        const uint16_t raw = p.layout == 0 ? p.x[l * p.ld + j] : p.x[j * p.ld + l];
        xin[t] = __uint_as_float((uint32_t)raw << 16);
        v[t] = xin[t];
      }
      if (p.rht) {
        fwht16_inlane(v, p.sg);
#pragma unroll
        for (int t = 0; t < 16; ++t) v[t] = v[t] * p.sg.fin;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int64_t o = o0 + h + t;
        const uint32_t code = (p.codes[o >> 1] >> (4 * (o & 1))) & 15u;
        const float xh = code_value<GRID>(code) * d;
        const float y = v[t] * inv;
        ++n;
        atomicAdd(&hist[code], 1u);
        if (!isfinite(xin[t])) ++n_nf;
        if (fabsf(y) > qmax) ++n_sat;
        const double dv = (double)v[t], dx = (double)xh, diff = dx - dv;
        const double sg = dv > 0 ? 1.0 : (dv < 0 ? -1.0 : 0.0);
        a_max = fmax(a_max, fabs(dv));
        a_v2 += dv * dv;
        a_e2 += diff * diff;
        a_vx += dv * dx;
        a_se += sg * diff;
        if (d != 0.0f) {
          a_seg += sg * diff / (double)d;
          ++n_grid;
        } else {
          ++n_zero;
        }
      }
    }
  }
  double vals[11] = {a_v2, a_e2, a_vx, a_se, a_seg, a_max, (double)n, (double)n_grid,
                     (double)n_zero, (double)n_sat, (double)n_nf};
  double* out = p.part + (int64_t)blockIdx.x * kStatsSlots;
  for (int q = 0; q < 11; ++q) {
    red[threadIdx.x] = vals[q];
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
      if ((int)threadIdx.x < st) {
        red[threadIdx.x] = (q == 5) ? fmax(red[threadIdx.x], red[threadIdx.x + st])
                                    : red[threadIdx.x] + red[threadIdx.x + st];
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) out[q] = red[0];
    __syncthreads();
  }
  if (threadIdx.x < 16) out[11 + threadIdx.x] = (double)hist[threadIdx.x];
}

hipError_t launch_stats(const StatsParams& p, hipStream_t s) {
  switch (p.grid) {
    case kGridE1M2: hipLaunchKernelGGL(ufp4_stats_kernel<kGridE1M2>, dim3(p.n_wg), dim3(256), 0, s, p); break;
    case kGridINT4: hipLaunchKernelGGL(ufp4_stats_kernel<kGridINT4>, dim3(p.n_wg), dim3(256), 0, s, p); break;
    case kGridE2M1: hipLaunchKernelGGL(ufp4_stats_kernel<kGridE2M1>, dim3(p.n_wg), dim3(256), 0, s, p); break;
    case kGridE2M1C: hipLaunchKernelGGL(ufp4_stats_kernel<kGridE2M1C>, dim3(p.n_wg), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- rounding hook
template <int GRID, bool SR>
__global__ __launch_bounds__(256) void ufp4_round_kernel(const float* y, int64_t n, uint32_t k0,
                                                         uint32_t k1, uint8_t* codes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t r = 0u;
    if (SR) {
      const Ctr4 c = sr_words4((uint64_t)i >> 2, 0u, k0, k1);
      const uint32_t q = (uint32_t)(i & 3);
      r = q == 0 ? c.x : (q == 1 ? c.y : (q == 2 ? c.z : c.w));
    }
    codes[i] = (uint8_t)quantize_code<GRID, SR>(y[i], r);
  }
}

template <int GRID>
static void launch_round_grid(const float* y, int64_t n, bool sr, uint32_t k0, uint32_t k1,
                              uint8_t* codes, int64_t blocks, hipStream_t s) {
  if (sr)
    hipLaunchKernelGGL((ufp4_round_kernel<GRID, true>), dim3((unsigned)blocks), dim3(256), 0, s, y, n, k0, k1, codes);
  else
    hipLaunchKernelGGL((ufp4_round_kernel<GRID, false>), dim3((unsigned)blocks), dim3(256), 0, s, y, n, k0, k1, codes);
}

hipError_t launch_round(const float* y, int64_t n, int32_t grid, int32_t rounding, uint64_t seed,
                        uint8_t* codes, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const bool sr = rounding != 0;
  switch (grid) {
    case kGridE1M2: launch_round_grid<kGridE1M2>(y, n, sr, k0, k1, codes, blocks, s); break;
    case kGridINT4: launch_round_grid<kGridINT4>(y, n, sr, k0, k1, codes, blocks, s); break;
    case kGridE2M1: launch_round_grid<kGridE2M1>(y, n, sr, k0, k1, codes, blocks, s); break;
    case kGridE2M1C: launch_round_grid<kGridE2M1C>(y, n, sr, k0, k1, codes, blocks, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 -> bf16
// Round to nearest, ties to even, on the bit pattern; NaN stays a quiet NaN
// with its sign.  Four values per thread (16-byte load, 8-byte store) when
// both pointers allow it, one otherwise.
__global__ __launch_bounds__(256) void ufp4_to_bf16_kernel(const float* in, int64_t n, uint16_t* out, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  auto rne = [](uint32_t u) -> uint32_t {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  };
  if (vec) {
    const int64_t n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
      const uint4 u = reinterpret_cast<const uint4*>(in)[i];
      reinterpret_cast<uint2*>(out)[i] = make_uint2(rne(u.x) | (rne(u.y) << 16), rne(u.z) | (rne(u.w) << 16));
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
      out[i] = (uint16_t)rne(__float_as_uint(in[i]));
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
      out[i] = (uint16_t)rne(__float_as_uint(in[i]));
  }
}

hipError_t launch_to_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int vec = ((uintptr_t)in % 16 == 0 && (uintptr_t)out % 8 == 0) ? 1 : 0;
  int64_t blocks = ((vec ? n / 4 : n) + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(ufp4_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, n, out, vec);
  return hipGetLastError();
}

}  // namespace ufp4
