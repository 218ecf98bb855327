// ufp4_device.hpp -- device primitives of the gfx950 quantization kernels.
//
// Sources, by title and section:
//   [Z] "Shrinkage Bias: The Hidden Geometric Trap in FP4 Training ... and the
//       UFP4 Fix", "Key points" (grids, RHT, fused RHT+quantization).
//   [A] "UFP4 Eliminates Shrinkage Bias in FP4 LLM Pretraining ...",
//       "The UFP4 Recipe" (E1M2/INT4, RHT everywhere, SR on dY only).
//   [H] "Rethinking Shrinkage Bias in LLM FP4 Pretraining ...", technical
//       approach (NVFP4/MXFP4 comparison formats, RTNE).
//   Philox4x32-10: Salmon et al., SC'11.  E4M3/E8M0: OCP FP8 and MX v1.0.
//
// All floating-point steps are single IEEE binary32 operations with
// round-to-nearest-even (the library is built with -ffp-contract=off; the
// only fused multiply-adds are explicit fmaf calls whose product is exact).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ufp4 {

// E2M1C: E2M1 codes limited to the uniformly spaced magnitudes {0, 0.5, 1,
// 1.5, 2} (E2M1 with its range clamped to imitate a uniform grid).
constexpr int kGridE1M2 = 0, kGridINT4 = 1, kGridE2M1 = 2, kGridE2M1C = 3;

// ---------------------------------------------------------------- bf16
// A dword holds two bf16 values; each is the upper half of a binary32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- Philox4x32-10
struct Ctr4 {
  uint32_t x, y, z, w;
};

// Full 64-bit product of two 32-bit words in one v_mad_u64_u32 (the plain
// C++ product compiles to a low and a high multiply: two quarter-rate
// instructions instead of one).
__device__ __forceinline__ uint64_t mul_wide(uint32_t a, uint32_t m) {
  uint64_t r, carry;
  asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(r), "=s"(carry) : "v"(a), "s"(m));
  return r;
}

// N rounds of Philox4x32 from counter c under key (k0, k1) (the key of the
// first of these rounds).
template <int N>
__device__ __forceinline__ Ctr4 philox_rounds(Ctr4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < N; ++r) {
    const uint64_t p0 = mul_wide(c.x, 0xD2511F53u), p1 = mul_wide(c.z, 0xCD9E8D57u);
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // a ^ b ^ k as one three-input bitwise op (truth table 0x96)
    c = Ctr4{(uint32_t)__builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96), lo1,
             (uint32_t)__builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96), lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ Ctr4 philox10(Ctr4 c, uint32_t k0, uint32_t k1) { return philox_rounds<10>(c, k0, k1); }

// Four consecutive stochastic-rounding words for flat output indices
// 4q .. 4q+3 of output stream `stream`: Philox4x32-10 of the counter
// (lo(q), hi(q), stream, 0).  The first round is written out: its product of
// the stream word is a constant at every call site (a plain product, which
// the compiler folds), and the zero fourth word drops out of its xor.
__device__ __forceinline__ Ctr4 sr_words4(uint64_t q, uint32_t stream, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = mul_wide((uint32_t)q, 0xD2511F53u);
  const uint64_t p1 = (uint64_t)stream * 0xCD9E8D57u;
  const Ctr4 c{(uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), (uint32_t)(q >> 32), k0, 0x96),
               (uint32_t)p1, (uint32_t)(p0 >> 32) ^ k1, (uint32_t)p0};
  return philox_rounds<9>(c, k0 + 0x9E3779B9u, k1 + 0xBB67AE85u);
}

// ---------------------------------------------------------------- FWHT
// Butterfly with the random signs folded in.  With sigma_j the sign carried by
// value j, the pair (sigma_a a, sigma_b b) maps to sigma_a (a + q b) and
// sigma_a (a - q b) with q = sigma_a sigma_b = +-1; fma(b, q, a) rounds a + q b
// once, exactly like the butterfly's add/sub, so every output equals the
// transform of the sign-flipped input up to a known sign.
__device__ __forceinline__ void bfly(float& a, float& b, float q) {
  const float s = fmaf(b, q, a);
  const float d = fmaf(b, -q, a);
  a = s;
  b = d;
}

// Folded signs of the transform (uniform per call).  For stage half-width h
// and a butterfly whose lower element is j: q = d[j & ~(h-1)] * d[(j+h) & ~(h-1)];
// after the four stages every value carries the sign d[0].
struct RhtSigns {
  float q1[8];  // stage h=1, pair p = (2p, 2p+1)
  float q2[4];  // stage h=2, group g = 4g..4g+3
  float q3[2];  // stage h=4, group g = 8g..8g+7
  float q4;     // stage h=8
  float fin;    // 0.25 * d[0]
};

// Full 16-point transform of v[0..15] held in one lane (column-wise blocks).
__device__ __forceinline__ void fwht16_inlane(float v[16], const RhtSigns& S) {
#pragma unroll
  for (int p = 0; p < 8; ++p) bfly(v[2 * p], v[2 * p + 1], S.q1[p]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    bfly(v[4 * g + 0], v[4 * g + 2], S.q2[g]);
    bfly(v[4 * g + 1], v[4 * g + 3], S.q2[g]);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bfly(v[8 * g + j], v[8 * g + j + 4], S.q3[g]);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) bfly(v[j], v[j + 8], S.q4);
}

// First three stages on the 8 values of one half block (positions 8*half ..
// 8*half+7), with the half's own folded signs (per-lane values).
struct HalfSigns {
  float q1[4], q2[2], q3;
};

__device__ __forceinline__ void fwht8_half(float v[8], const HalfSigns& S) {
#pragma unroll
  for (int p = 0; p < 4; ++p) bfly(v[2 * p], v[2 * p + 1], S.q1[p]);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    bfly(v[4 * g + 0], v[4 * g + 2], S.q2[g]);
    bfly(v[4 * g + 1], v[4 * g + 3], S.q2[g]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) bfly(v[j], v[j + 4], S.q3);
}

// Cross-lane value of the lane whose index differs in bit 0 (DPP quad_perm
// [1,0,3,2]) and in bit 1 ([2,3,0,1]).
// (Every lane has a source lane in these permutations, so bound_ctrl does not
// change the result; setting it lets the compiler fold the move into the
// consuming instruction as a DPP operand.)
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}

// ---------------------------------------------------------------- E4M3 / E8M0
// OCP E4M3FN encode of q in [0, 448] with round-to-nearest-even: the gfx950
// conversion instruction (matches an exhaustive software RNE encode for every
// non-negative binary32 below 464; larger inputs would become NaN, hence the
// clamp, which is the saturation of the scale).
__device__ __forceinline__ uint32_t e4m3_encode_sat(float q) {
  const float c = fminf(q, 448.0f);
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
  return (q == q) ? code : 0x7Fu;  // NaN stays NaN
}

__device__ __forceinline__ float e4m3_decode_pos(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
}

// emax of the element format (floor(log2(Qmax))) for the E8M0 exponent.
template <int GRID>
__device__ __forceinline__ int grid_emax() { return (GRID == kGridE1M2 || GRID == kGridE2M1C) ? 1 : 2; }

template <int GRID>
__device__ __forceinline__ constexpr float grid_qmax() {
  return GRID == kGridE1M2 ? 3.5f : (GRID == kGridINT4 ? 7.0f : (GRID == kGridE2M1 ? 6.0f : 2.0f));
}

// Largest magnitude index of the grid.
template <int GRID>
__device__ __forceinline__ constexpr uint32_t grid_top() { return GRID == kGridE2M1C ? 4u : 7u; }

__device__ __forceinline__ float qmax_of(int grid) {
  return grid == kGridE1M2 ? 3.5f : (grid == kGridINT4 ? 7.0f : (grid == kGridE2M1 ? 6.0f : 2.0f));
}

// MX32 scale of a block: exponent X = clamp(floor(log2 amax) - emax, -127, 127)
// (-127 for a zero block); byte X + 127; quantization multiplier 2^-X.
template <int GRID>
__device__ __forceinline__ void mx_scale(float amax_b, uint32_t& byte, float& inv) {
  int X = -127;
  if (amax_b > 0.0f) {
    X = __builtin_amdgcn_frexp_expf(amax_b) - 1 - grid_emax<GRID>();
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    if (!(amax_b <= 3.40282347e38f)) X = 127;  // infinite block maximum
  }
  if (amax_b != amax_b) X = 127;
  byte = (uint32_t)(X + 127);
  inv = ldexpf(1.0f, -X);
}

// ---------------------------------------------------------------- rounding
// Code layout: E1M2/E2M1 sign<<3 | magnitude index; INT4 two's complement.
// A zero magnitude is always code 0.
template <int GRID>
__device__ __forceinline__ uint32_t make_code(uint32_t k, float y) {
  if (GRID == kGridINT4) return (y < 0.0f || (__float_as_uint(y) >> 31)) ? ((16u - k) & 15u) : k;
  return k ? (k | ((__float_as_uint(y) >> 28) & 8u)) : 0u;
}

// Round-to-nearest-even onto the grid at unit scale (ties to the even
// magnitude index), saturating at Qmax; NaN -> 0.
template <int GRID>
__device__ __forceinline__ uint32_t round_rtne(float y) {
  const float a = fabsf(y);
  uint32_t k;
  if (GRID == kGridE1M2 || GRID == kGridE2M1C) {
    k = (uint32_t)__builtin_rintf(fminf(a + a, (float)grid_top<GRID>()));
  } else if (GRID == kGridINT4) {
    k = (uint32_t)__builtin_rintf(fminf(a, 7.0f));
  } else {
    // E2M1: the hardware conversion (OCP E2M1, round to nearest even,
    // saturating at +-6) writes sign | magnitude index, the layout of these
    // codes; it matches the nearest-even search on every finite input
    // except that it keeps the sign of a zero result, so a zero magnitude is
    // mapped to code 0 here, and NaN is mapped to 0 before the conversion.
    const uint32_t c =
        (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, (a == a) ? y : 0.0f, 0.0f, 1.0f, 0) & 15u;
    return (c & 7u) ? c : 0u;
  }
  k = (a == a) ? k : 0u;
  return k ? make_code<GRID>(k, y) : 0u;
}

// Stochastic rounding: with lo <= |y| < hi adjacent grid magnitudes and
// frac = (|y| - lo) / (hi - lo) (exact), round up iff r < ceil(frac * 2^32).
//
// Uniform grids (E1M2, E2M1C: step 1/2; INT4: step 1): t = |y| / step is
// exact, lo = floor(t), frac = t - floor(t).  t is clamped to [0, top] by
// one median (a NaN operand makes v_med3_f32 return the smallest of the
// three, 0 here, so NaN gives index 0; +inf and everything at or above the
// top give the top with frac 0).  Both return the magnitude index.
//
// sr_steps takes s = y / step (any sign), which must not be a signaling NaN
// (the median treats one otherwise; the result of arithmetic never is one).
template <int GRID>
__device__ __forceinline__ uint32_t sr_steps(float s, uint32_t r) {
  const float t = __builtin_amdgcn_fmed3f(fabsf(s), 0.0f, (float)grid_top<GRID>());
  const uint32_t lo = (uint32_t)t;
  const uint32_t thr = (uint32_t)ceilf(__builtin_amdgcn_fractf(t) * 4294967296.0f);
  return lo + (r < thr ? 1u : 0u);
}

// sr_uniform_index takes y itself and quiets a signaling NaN first (free
// when y is the result of arithmetic).
template <int GRID>
__device__ __forceinline__ uint32_t sr_uniform_index(float y, uint32_t r) {
  constexpr float kInvStep = GRID == kGridINT4 ? 1.0f : 2.0f;
  return sr_steps<GRID>(__builtin_canonicalizef(y * kInvStep), r);
}

// E2M1, the same rule: the magnitudes 0, 1/2, 1, 3/2 | 2, 3 | 4, 6 are
// uniform within [0, 2) (step 1/2), [2, 4) (step 1) and [4, 6] (step 2), so
// a = |y| clamped to [0, 6] (NaN to 0) gives s = 2a, a - 2 or a/2 - 2 (each
// exact) and the index is the range's first index + floor(s), plus one iff
// r < ceil(fract(s) * 2^32), with fract(s) the bucket fraction (a - lo) /
// (hi - lo).  y must not be a signaling NaN.
__device__ __forceinline__ uint32_t sr_e2m1_index(float y, uint32_t r) {
  const float a = __builtin_amdgcn_fmed3f(fabsf(y), 0.0f, 6.0f);
  const bool r0 = a < 2.0f, r1 = a < 4.0f;
  const float s = r0 ? a + a : (r1 ? a - 2.0f : fmaf(a, 0.5f, -2.0f));
  const uint32_t base = r0 ? 0u : (r1 ? 4u : 6u);
  const uint32_t thr = (uint32_t)ceilf(__builtin_amdgcn_fractf(s) * 4294967296.0f);
  return base + (uint32_t)s + (r < thr ? 1u : 0u);
}

template <int GRID>
__device__ __forceinline__ uint32_t round_sr(float y, uint32_t r) {
  uint32_t k;
  if (GRID == kGridE2M1) {
    const float a = fabsf(y);
    if (!(a == a)) return 0u;
    if (a >= grid_qmax<GRID>()) {
      k = grid_top<GRID>();
    } else {
      const uint32_t i = (uint32_t)(a >= 0.5f) + (uint32_t)(a >= 1.0f) + (uint32_t)(a >= 1.5f) +
                         (uint32_t)(a >= 2.0f) + (uint32_t)(a >= 3.0f) + (uint32_t)(a >= 4.0f);
      const float lo = i < 4u ? 0.5f * (float)i : (i == 4u ? 2.0f : (i == 5u ? 3.0f : 4.0f));
      const float rw = i < 4u ? 2.0f : (i == 6u ? 0.5f : 1.0f);  // 1 / bucket width
      const float frac = (a - lo) * rw;
      const uint32_t thr = (uint32_t)ceilf(frac * 4294967296.0f);
      k = i + (r < thr ? 1u : 0u);
    }
  } else {
    k = sr_uniform_index<GRID>(y, r);
  }
  return k ? make_code<GRID>(k, y) : 0u;
}

template <int GRID, bool SR>
__device__ __forceinline__ uint32_t quantize_code(float y, uint32_t r) {
  if (SR) return round_sr<GRID>(y, r);
  return round_rtne<GRID>(y);
}

template <int GRID>
__device__ __forceinline__ float code_value(uint32_t c) {
  c &= 15u;
  if (GRID == kGridINT4) return (float)((int)c - (c >= 8u ? 16 : 0));
  const uint32_t k = c & 7u;
  float m;
  if (GRID == kGridE1M2) {
    m = 0.5f * (float)k;
  } else {
    m = k < 4u ? 0.5f * (float)k : (k == 4u ? 2.0f : (k == 5u ? 3.0f : (k == 6u ? 4.0f : 6.0f)));
  }
  return (c & 8u) ? -m : m;
}

}  // namespace ufp4
