/*
 * ufp4_oracle.c -- plain, slow, single-threaded CPU oracle (TEST INFRASTRUCTURE).
 *
 * Only the tests, the package smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares nothing with the HIP path.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (binary32 arithmetic, round-to-nearest-even, no FMA contraction).
 *
 * Source titles are abbreviated [Z], [A], [H] as in ufp4_oracle.h.
 *
 * What the method computes, step by step, per 16-element block along the
 * GEMM reduction dimension ([Z] "Key points": the RHT paradox and the fix;
 * [A] "The UFP4 Recipe"; [H] technical approach):
 *   1. widen bf16 to fp32 (exact);
 *   2. random Hadamard transform: multiply by seeded random signs, run a
 *      16-point Walsh-Hadamard butterfly, scale by 1/4;
 *   3. per-block and per-tensor absolute maxima;
 *   4. two-level scale (per-tensor fp32, per-block E4M3; NVFP4-style) or one
 *      power-of-two E8M0 scale per 32 elements (MXFP4-style) -- the pages
 *      name NVFP4 and MXFP4 as the comparison formats ([H] technical
 *      approach; [Z] "Key points": the symptom);
 *   5. scale each value and round it onto a 4-bit grid: uniform E1M2
 *      ([Z] "Key points": the fix), symmetric INT4 ([A] "The UFP4 Recipe"),
 *      or the E2M1 baseline ([Z] "Key points": the cause); round to nearest
 *      even ([H] core idea names RTNE) or stochastic rounding, which the
 *      recipe uses for the output gradient only ([A] "The UFP4 Recipe");
 *   6. encode and pack two codes per byte.
 *
 * Parity pins (see the tests): every function here is pinned by a test that
 * does not re-use its code -- exhaustive brute-force grid search, a library
 * E4M3 conversion, rocRAND's Philox4x32-10 engine, Hadamard closed forms,
 * the page's -0.125 bucket bias, binomial bounds for stochastic rounding.
 */
#include "ufp4_oracle.h"
#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 -> fp32: bf16 is the upper half of a binary32, so widening is exact. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, as defined in Salmon et al. (SC'11): ten rounds of the
 * Philox-4x32 S-box on a 128-bit counter under a 64-bit key; the key is
 * advanced by the Weyl constants between rounds.                            */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Random signs of the RHT.  Reading: one 16-sign vector per seed, shared by
 * every block, layout and tensor (both operands of a GEMM must use the same
 * signs along their common reduction dimension for the transform to cancel).
 * d_j = -1 where bit j of word 0 of Philox(key = seed, counter = (0,0,2,0)). */
void orc_rht_signs(uint64_t rht_seed, int8_t signs[16]) {
  uint32_t key[2] = {(uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)};
  uint32_t ctr[4] = {0u, 0u, 2u, 0u};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  for (int j = 0; j < 16; ++j) signs[j] = ((w[0] >> j) & 1u) ? (int8_t)-1 : (int8_t)1;
}

/* Random word for stochastic rounding of output element `index` of the
 * output stream `stream` (0 row-wise, 1 column-wise): Philox keyed by the
 * seed, counter (lo32(index/4), hi32(index/4), stream, 0), word index%4.    */
uint32_t orc_sr_word(uint64_t sr_seed, uint64_t index, uint32_t stream) {
  uint32_t key[2] = {(uint32_t)sr_seed, (uint32_t)(sr_seed >> 32)};
  uint64_t q = index >> 2;
  uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), stream, 0u};
  uint32_t w[4];
  orc_philox4x32_10(ctr, key, w);
  return w[index & 3u];
}

/* ------------------------------------------------------------------------ */
/* 16-point fast Walsh-Hadamard transform, Sylvester order, stages with
 * half-width h = 1, 2, 4, 8 in that order; each butterfly maps the pair
 * (a at the lower index, b) to (a + b, a - b), each operation rounded.      */
void orc_fwht16_stages(float v[16]) {
  for (int h = 1; h < 16; h *= 2) {
    for (int i = 0; i < 16; i += 2 * h) {
      for (int j = i; j < i + h; ++j) {
        float a = v[j];
        float b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

/* v = (1/4) H16 D x : signs first, then the butterfly, then the 1/4 that
 * makes the transform orthonormal (reading: the scaling comes last).         */
void orc_rht16(const float x[16], const int8_t signs[16], float v[16]) {
  for (int j = 0; j < 16; ++j) v[j] = signs[j] < 0 ? -x[j] : x[j];
  orc_fwht16_stages(v);
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

/* Inverse: x = D (1/4) H16 v, since H16 H16 = 16 I and D D = I.              */
void orc_inverse_rht16(const float v[16], const int8_t signs[16], float x[16]) {
  float t[16];
  for (int j = 0; j < 16; ++j) t[j] = v[j];
  orc_fwht16_stages(t);
  for (int j = 0; j < 16; ++j) {
    float u = t[j] * 0.25f;
    x[j] = signs[j] < 0 ? -u : u;
  }
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; subnormal step
 * 2^-9; largest finite 448; 0x7F/0xFF are NaN, there is no infinity.
 * Encode a non-negative value with round-to-nearest-even, saturating at 448. */
uint8_t orc_e4m3_encode(float q) {
  if (q != q) return 0x7F;
  if (!(q > 0.0f)) return 0x00;
  if (q >= 448.0f) return 0x7E;
  int e2;
  (void)frexp((double)q, &e2);           /* q = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;                        /* q in [2^e, 2^(e+1)) */
  if (e < -6) {                          /* below the smallest normal 2^-6 */
    double m = rint(ldexp((double)q, 9)); /* multiples of 2^-9, ties to even */
    return (uint8_t)m;                   /* m == 8 is exactly the code of 2^-6 */
  }
  double m = rint(ldexp((double)q, 3 - e)) - 8.0; /* 3-bit mantissa, RNE */
  int mant = (int)m;
  int bexp = e + 7;
  if (mant == 8) { mant = 0; bexp += 1; }
  int code = (bexp << 3) | mant;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)code;
}

void orc_e4m3_encode_n(const float* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(q[i]);
}

float orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return (float)(s ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* The 4-bit grids: magnitudes indexed by the 3 magnitude bits.  The clamped
 * E2M1 grid keeps E2M1's codes but only its uniformly spaced part, indices
 * 0..4 ({0, 0.5, 1, 1.5, 2}): E2M1 with its range clamped to imitate a
 * uniform grid, the alternative [Z] "Key points" (validation results) reports
 * as not recovering the uniform grid's accuracy.                           */
static const float kE1M2[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 2.5f, 3.0f, 3.5f};
static const float kINT4[8] = {0.0f, 1.0f, 2.0f, 3.0f, 4.0f, 5.0f, 6.0f, 7.0f};
static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static const float* grid_mags(int32_t grid) {
  return grid == ORC_GRID_INT4 ? kINT4 : (grid == ORC_GRID_E2M1 || grid == ORC_GRID_E2M1_CLAMP) ? kE2M1 : kE1M2;
}

/* Largest magnitude index the grid uses. */
static int grid_top(int32_t grid) { return grid == ORC_GRID_E2M1_CLAMP ? 4 : 7; }

float orc_grid_qmax(int32_t grid) { return grid_mags(grid)[grid_top(grid)]; }

/* emax of the element format, used by the E8M0 shared exponent (OCP MX):
 * floor(log2(Qmax)).                                                        */
static int grid_emax(int32_t grid) {
  return (grid == ORC_GRID_E1M2 || grid == ORC_GRID_E2M1_CLAMP) ? 1 : 2;
}

/* Code layout.  E1M2 and E2M1: sign << 3 | magnitude index (the magnitude
 * index equals the format's own bit pattern).  INT4: 4-bit two's complement.
 * Reading: a result of magnitude zero is always code 0 (+0).               */
static uint8_t encode_code(int k, int neg, int32_t grid) {
  if (k == 0) return 0;
  if (grid == ORC_GRID_INT4) return (uint8_t)(neg ? ((16 - k) & 15) : k);
  return (uint8_t)((neg ? 8 : 0) | k);
}

float orc_code_value(uint8_t code, int32_t grid) {
  code &= 15;
  if (grid == ORC_GRID_INT4) {
    int s = code >= 8 ? (int)code - 16 : (int)code;
    return (float)s;
  }
  float m = grid_mags(grid)[code & 7];
  return (code & 8) ? -m : m;
}

/* Round y (already divided by its scale) onto the grid.
 * RTNE: nearest magnitude; a tie goes to the even magnitude index.
 * SR: with lo <= |y| < hi adjacent magnitudes and frac = (|y|-lo)/(hi-lo),
 *     round up iff r32 < ceil(frac * 2^32).
 * |y| >= Qmax saturates to Qmax; NaN gives code 0.                         */
uint8_t orc_round_to_code(float y, int32_t grid, int32_t rounding, uint32_t r32) {
  if (y != y) return 0;
  const float* g = grid_mags(grid);
  const int top = grid_top(grid);
  float a = fabsf(y);
  int neg = signbit(y) ? 1 : 0;
  int k;
  if (a >= g[top]) {
    k = top;
  } else {
    int i = 0;
    while (i < top - 1 && g[i + 1] <= a) ++i;   /* g[i] <= a < g[i+1] */
    float lo = g[i], hi = g[i + 1];
    if (rounding == ORC_ROUND_SR) {
      /* a - lo is exact (lo == 0, or lo <= a <= hi <= 2 lo); hi - lo is a
       * power of two, so frac and frac * 2^32 are exact.                  */
      float frac = (a - lo) / (hi - lo);
      double thr = ceil((double)frac * 4294967296.0);
      k = ((double)r32 < thr) ? i + 1 : i;
    } else {
      float mid = (lo + hi) * 0.5f;        /* exact for these grids */
      if (a > mid) k = i + 1;
      else if (a < mid) k = i;
      else k = (i % 2 == 0) ? i : i + 1;
    }
  }
  return encode_code(k, neg, grid);
}

int orc_round_f32(const float* y, int64_t n, int32_t grid, int32_t rounding,
                  uint64_t sr_seed, uint8_t* codes) {
  if (n < 0 || (n > 0 && (!y || !codes))) return 1;
  if (grid < 0 || grid > 3 || rounding < 0 || rounding > 1) return 1;
  for (int64_t i = 0; i < n; ++i) {
    uint32_t r = rounding == ORC_ROUND_SR ? orc_sr_word(sr_seed, (uint64_t)i, 0u) : 0u;
    codes[i] = orc_round_to_code(y[i], grid, rounding, r);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* A set of "lines" quantized under one tensor scale.  Element j of line l is
 * x[l*xl + j*xj] for j < valid, and 0 for valid <= j < len (zero padding of a
 * grouped segment).  Its flat output index is o = l*ol + obase + j: code
 * nibble o (low nibble for even o), scale entry o/B, and stochastic-rounding
 * index o in output stream `stream`.                                        */
typedef struct {
  const uint16_t* x;
  int64_t xl, xj;
  int64_t lines, len, valid;
  int64_t ol, obase;
  uint32_t stream;
} lineset;

static int block_len(const orc_config* cfg) { return cfg->scaling == ORC_SCALE_MX32 ? 32 : 16; }

/* Post-transform values of the 16 elements starting at j0 of line l.        */
static void load_v16(const lineset* L, const orc_config* cfg, const int8_t signs[16],
                     int64_t l, int64_t j0, float v[16]) {
  float xs[16];
  for (int t = 0; t < 16; ++t) {
    int64_t j = j0 + t;
    xs[t] = (j < L->valid) ? orc_bf16_to_f32(L->x[l * L->xl + j * L->xj]) : 0.0f;
  }
  if (cfg->rht) {
    orc_rht16(xs, signs, v);
  } else {
    for (int t = 0; t < 16; ++t) v[t] = xs[t];
  }
}

/* Block maximum of |v|; NaN is skipped (a comparison with NaN is false).   */
static float abs_max(const float* v, int n, float m) {
  for (int t = 0; t < n; ++t) {
    float a = fabsf(v[t]);
    if (a > m) m = a;
  }
  return m;
}

static float lineset_amax(const lineset* L, const orc_config* cfg, const int8_t signs[16]) {
  float m = 0.0f;
  float v[16];
  for (int64_t l = 0; l < L->lines; ++l)
    for (int64_t j0 = 0; j0 < L->len; j0 += 16) {
      load_v16(L, cfg, signs, l, j0, v);
      m = abs_max(v, 16, m);
    }
  return m;
}

/* Scale of one block: the stored byte, the dequantization factor d_b and the
 * quantization multiplier inv_b.
 * NV16 (two-level): S_t = amax_t / (Qmax*448); s_b = E4M3(amax_b / (Qmax*S_t));
 *   d_b = s_b * S_t; inv_b = 1 / d_b (0 when d_b == 0).
 * MX32: X = clamp(floor(log2 amax_b) - emax, -127, 127) (X = -127 for a zero
 *   block); byte X + 127; d_b = 2^X; inv_b = 2^-X.                          */
static void block_scale(const orc_config* cfg, float S_t, float amax_b,
                        uint8_t* byte, float* d_b, float* inv_b) {
  if (cfg->scaling == ORC_SCALE_MX32) {
    int X;
    if (!(amax_b > 0.0f)) {
      X = -127;
    } else if (isinf(amax_b) || isnan(amax_b)) {
      X = 127;
    } else {
      int e2;
      (void)frexp((double)amax_b, &e2);
      X = (e2 - 1) - grid_emax(cfg->grid);
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    *byte = (uint8_t)(X + 127);
    *d_b = (float)ldexp(1.0, X);
    *inv_b = (float)ldexp(1.0, -X);
    return;
  }
  float qmax = orc_grid_qmax(cfg->grid);
  float denom = qmax * S_t;              /* fl(Qmax * S_t) */
  float q = amax_b / denom;
  uint8_t s = orc_e4m3_encode(q);
  float d = orc_e4m3_decode(s) * S_t;
  *byte = s;
  *d_b = d;
  *inv_b = (d == 0.0f) ? 0.0f : 1.0f / d;
}

static float tensor_scale_from_amax(const orc_config* cfg, float amax_t) {
  if (cfg->scaling == ORC_SCALE_MX32) return 1.0f;
  if (!(amax_t > 0.0f)) return 1.0f;      /* all-zero tensor: S_t = 1 */
  float qmax448 = orc_grid_qmax(cfg->grid) * 448.0f;  /* 1568, 3136, 2688, 896: exact */
  return amax_t / qmax448;
}

static void put_nibble(uint8_t* codes, int64_t o, uint8_t code) {
  uint8_t* p = &codes[o >> 1];
  if (o & 1) *p = (uint8_t)((*p & 0x0F) | (code << 4));
  else *p = (uint8_t)((*p & 0xF0) | (code & 0x0F));
}

static uint8_t get_nibble(const uint8_t* codes, int64_t o) {
  uint8_t b = codes[o >> 1];
  return (o & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
}

/* Quantize a lineset: pass 1 finds the tensor amax, pass 2 scales, rounds
 * and packs every block (recomputing the transform).  With amax_given, the
 * tensor scale comes from that maximum instead (delayed scaling): blocks
 * whose maximum exceeds it saturate, their E4M3 scale at 448 and their
 * codes at +-Qmax.  *amax_seen (if given) receives the lineset's own
 * maximum either way.                                                       */
static float quantize_lineset_amax(const lineset* L, const orc_config* cfg, uint8_t* codes,
                                   uint8_t* scales, const float* amax_given, float* amax_seen) {
  int8_t signs[16];
  orc_rht_signs(cfg->rht_seed, signs);
  float amax_t = lineset_amax(L, cfg, signs);
  if (amax_seen) *amax_seen = amax_t;
  float amax_s = amax_t;
  if (amax_given) {
    /* a provided maximum that is not a positive finite number counts as 0 */
    amax_s = (*amax_given > 0.0f && !isinf(*amax_given)) ? *amax_given : 0.0f;
  }
  float S_t = tensor_scale_from_amax(cfg, amax_s);
  int B = block_len(cfg);
  float v[32];
  for (int64_t l = 0; l < L->lines; ++l) {
    for (int64_t j0 = 0; j0 < L->len; j0 += B) {
      for (int h = 0; h < B; h += 16) load_v16(L, cfg, signs, l, j0 + h, v + h);
      float amax_b = abs_max(v, B, 0.0f);
      uint8_t sbyte;
      float d_b, inv_b;
      block_scale(cfg, S_t, amax_b, &sbyte, &d_b, &inv_b);
      int64_t o0 = l * L->ol + L->obase + j0;
      scales[o0 / B] = sbyte;
      for (int t = 0; t < B; ++t) {
        float y = v[t] * inv_b;
        int64_t o = o0 + t;
        uint32_t r = cfg->rounding == ORC_ROUND_SR ? orc_sr_word(cfg->sr_seed, (uint64_t)o, L->stream) : 0u;
        put_nibble(codes, o, orc_round_to_code(y, cfg->grid, cfg->rounding, r));
      }
    }
  }
  return S_t;
}


static int check_cfg(const orc_config* cfg) {
  if (!cfg) return 1;
  if (cfg->grid < 0 || cfg->grid > 3) return 1;
  if (cfg->rounding < 0 || cfg->rounding > 1) return 1;
  if (cfg->scaling < 0 || cfg->scaling > 1) return 1;
  return 0;
}

static int quantize_layout(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                           const orc_config* cfg, int32_t layout, const float* amax_given,
                           uint8_t* codes, uint8_t* scales, float* tensor_scale, float* amax_seen) {
  if (check_cfg(cfg) || rows < 0 || cols < 0 || ld < cols) return 1;
  int B = block_len(cfg);
  lineset L;
  L.x = x;
  L.obase = 0;
  if (layout == ORC_LAYOUT_ROW) {
    if (cols % B) return 2;
    L.xl = ld; L.xj = 1; L.lines = rows; L.len = cols; L.valid = cols; L.ol = cols; L.stream = 0;
  } else if (layout == ORC_LAYOUT_COL) {
    if (rows % B) return 2;
    L.xl = 1; L.xj = ld; L.lines = cols; L.len = rows; L.valid = rows; L.ol = rows; L.stream = 1;
  } else {
    return 1;
  }
  *tensor_scale = quantize_lineset_amax(&L, cfg, codes, scales, amax_given, amax_seen);
  return 0;
}

int orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                 const orc_config* cfg, int32_t layout,
                 uint8_t* codes, uint8_t* scales, float* tensor_scale) {
  return quantize_layout(x, rows, cols, ld, cfg, layout, NULL, codes, scales, tensor_scale, NULL);
}

int orc_quantize_given_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            const orc_config* cfg, int32_t layout, float amax_given,
                            uint8_t* codes, uint8_t* scales, float* tensor_scale, float* amax_seen) {
  if (cfg && cfg->scaling != ORC_SCALE_NV16) return 1;
  return quantize_layout(x, rows, cols, ld, cfg, layout, &amax_given, codes, scales, tensor_scale,
                         amax_seen);
}

int orc_grouped_col_offsets(const int64_t* offsets, int32_t num_groups, int32_t block,
                            int64_t* col_offsets) {
  if (num_groups < 0 || block <= 0) return 1;
  col_offsets[0] = 0;
  for (int32_t e = 0; e < num_groups; ++e) {
    int64_t m = offsets[e + 1] - offsets[e];
    if (m < 0) return 1;
    int64_t padded = (m + block - 1) / block * block;
    col_offsets[e + 1] = col_offsets[e] + padded;
  }
  return 0;
}

/* Grouped driver: segment e is one lineset per layout.  With amax_given,
 * segment e's tensor scales come from amax_given[2e] (row-wise) and
 * amax_given[2e+1] (column-wise) (delayed scaling per segment); amax_seen
 * receives each segment's own maxima in the same layout.                   */
static int quantize_grouped_impl(const uint16_t* x, int64_t total_rows, int64_t cols,
                                 const int64_t* offsets, int32_t num_groups, const orc_config* cfg,
                                 const float* amax_given, float* amax_seen,
                                 uint8_t* row_codes, uint8_t* row_scales, float* row_tensor_scale,
                                 uint8_t* col_codes, uint8_t* col_scales, float* col_tensor_scale) {
  if (check_cfg(cfg) || num_groups < 0 || cols < 0) return 1;
  int B = block_len(cfg);
  if (cols % B) return 2;
  if (offsets[0] != 0 || offsets[num_groups] != total_rows) return 1;
  int64_t col_off[num_groups + 1];
  if (orc_grouped_col_offsets(offsets, num_groups, B, col_off)) return 1;
  int64_t R_pad = col_off[num_groups];
  for (int32_t e = 0; e < num_groups; ++e) {
    int64_t r0 = offsets[e], m = offsets[e + 1] - offsets[e];
    if (row_codes) {
      lineset L = {x + r0 * cols, cols, 1, m, cols, cols, cols, r0 * cols, 0u};
      row_tensor_scale[e] = quantize_lineset_amax(&L, cfg, row_codes, row_scales,
                                                  amax_given ? &amax_given[2 * e] : NULL,
                                                  amax_seen ? &amax_seen[2 * e] : NULL);
    }
    if (col_codes) {
      int64_t P = col_off[e + 1] - col_off[e];
      lineset L = {x + r0 * cols, 1, cols, cols, P, m, R_pad, col_off[e], 1u};
      col_tensor_scale[e] = quantize_lineset_amax(&L, cfg, col_codes, col_scales,
                                                  amax_given ? &amax_given[2 * e + 1] : NULL,
                                                  amax_seen ? &amax_seen[2 * e + 1] : NULL);
    }
  }
  return 0;
}

int orc_quantize_grouped(const uint16_t* x, int64_t total_rows, int64_t cols,
                         const int64_t* offsets, int32_t num_groups, const orc_config* cfg,
                         uint8_t* row_codes, uint8_t* row_scales, float* row_tensor_scale,
                         uint8_t* col_codes, uint8_t* col_scales, float* col_tensor_scale) {
  return quantize_grouped_impl(x, total_rows, cols, offsets, num_groups, cfg, NULL, NULL, row_codes, row_scales,
                               row_tensor_scale, col_codes, col_scales, col_tensor_scale);
}

int orc_quantize_grouped_given_amax(const uint16_t* x, int64_t total_rows, int64_t cols,
                                    const int64_t* offsets, int32_t num_groups, const orc_config* cfg,
                                    const float* amax_given, float* amax_seen,
                                    uint8_t* row_codes, uint8_t* row_scales, float* row_tensor_scale,
                                    uint8_t* col_codes, uint8_t* col_scales, float* col_tensor_scale) {
  if (!cfg || cfg->scaling != ORC_SCALE_NV16 || !amax_given) return 1;
  return quantize_grouped_impl(x, total_rows, cols, offsets, num_groups, cfg, amax_given, amax_seen, row_codes,
                               row_scales, row_tensor_scale, col_codes, col_scales, col_tensor_scale);
}

/* ------------------------------------------------------------------------ */
/* Dequantize: xhat = value(code) * d_b (one rounding); optional inverse RHT. */
int orc_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                   int64_t rows, int64_t cols, const orc_config* cfg, int32_t inverse_rht,
                   float* out) {
  if (check_cfg(cfg) || rows < 0 || cols < 0) return 1;
  int B = block_len(cfg);
  if (cols % B) return 2;
  float S_t = tensor_scale[0];
  int8_t signs[16];
  orc_rht_signs(cfg->rht_seed, signs);
  for (int64_t l = 0; l < rows; ++l) {
    for (int64_t j0 = 0; j0 < cols; j0 += B) {
      int64_t o0 = l * cols + j0;
      uint8_t s = scales[o0 / B];
      float d_b = cfg->scaling == ORC_SCALE_MX32 ? (float)ldexp(1.0, (int)s - 127)
                                                 : orc_e4m3_decode(s) * S_t;
      for (int t = 0; t < B; ++t) out[o0 + t] = orc_code_value(get_nibble(codes, o0 + t), cfg->grid) * d_b;
      if (inverse_rht) {
        for (int h = 0; h < B; h += 16) {
          float xr[16];
          orc_inverse_rht16(&out[o0 + h], signs, xr);
          for (int t = 0; t < 16; ++t) out[o0 + h + t] = xr[t];
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Diagnostics of a quantization (all sums in binary64, in element order):
 *   SQNR (dB) = 10 log10( sum v^2 / sum (v - xhat)^2 )
 *   mean signed error = sum sign(v) (xhat - v) / N: negative means values are
 *     pulled toward zero, the shrinkage the pages measure per rounding bucket
 *     ([Z] "Key points": the cause);
 *   the same in grid units, (xhat - v)/d_b, skipping zero-scale blocks;
 *   alpha = <v, xhat> / <v, v>, the projection gain of the decomposition of a
 *     quantized operand into a scaled copy plus an orthogonal residual
 *     ([Z] "Key points": compounding decay);
 *   the code histogram (bucket utilisation, [H] abstract);
 *   saturations (|y| > Qmax) and non-finite inputs.                         */
int orc_compute_stats(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                      int32_t layout, const orc_config* cfg, const uint8_t* codes,
                      const uint8_t* scales, const float* tensor_scale, orc_stats* out) {
  if (check_cfg(cfg) || rows < 0 || cols < 0 || ld < cols || !out) return 1;
  int B = block_len(cfg);
  lineset L;
  L.x = x;
  L.obase = 0;
  if (layout == ORC_LAYOUT_ROW) {
    if (cols % B) return 2;
    L.xl = ld; L.xj = 1; L.lines = rows; L.len = cols; L.valid = cols; L.ol = cols; L.stream = 0;
  } else if (layout == ORC_LAYOUT_COL) {
    if (rows % B) return 2;
    L.xl = 1; L.xj = ld; L.lines = cols; L.len = rows; L.valid = rows; L.ol = rows; L.stream = 1;
  } else {
    return 1;
  }
  int8_t signs[16];
  orc_rht_signs(cfg->rht_seed, signs);
  float qmax = orc_grid_qmax(cfg->grid);
  float S_t = tensor_scale[0];
  double sum_v2 = 0, sum_e2 = 0, sum_vx = 0, sum_se = 0, sum_seg = 0;
  uint64_t n = 0, n_grid = 0, n_zero = 0, n_sat = 0, n_nonfinite = 0;
  uint64_t hist[16];
  memset(hist, 0, sizeof hist);
  float amax = 0.0f;
  float v[32];
  for (int64_t l = 0; l < L.lines; ++l) {
    for (int64_t j0 = 0; j0 < L.len; j0 += B) {
      for (int h = 0; h < B; h += 16) load_v16(&L, cfg, signs, l, j0 + h, v + h);
      int64_t o0 = l * L.ol + j0;
      uint8_t s = scales[o0 / B];
      float d_b = cfg->scaling == ORC_SCALE_MX32 ? (float)ldexp(1.0, (int)s - 127)
                                                 : orc_e4m3_decode(s) * S_t;
      float inv_b = (d_b == 0.0f) ? 0.0f : 1.0f / d_b;
      for (int t = 0; t < B; ++t) {
        int64_t j = j0 + t;
        float xin = orc_bf16_to_f32(L.x[l * L.xl + j * L.xj]);
        if (!isfinite(xin)) ++n_nonfinite;
        uint8_t code = get_nibble(codes, o0 + t);
        float xh = orc_code_value(code, cfg->grid) * d_b;
        float y = v[t] * inv_b;
        ++n;
        ++hist[code];
        if (fabsf(y) > qmax) ++n_sat;
        float av = fabsf(v[t]);
        if (av > amax) amax = av;
        double dv = (double)v[t], dx = (double)xh, diff = dx - dv;
        double sg = dv > 0 ? 1.0 : (dv < 0 ? -1.0 : 0.0);
        sum_v2 += dv * dv;
        sum_e2 += diff * diff;
        sum_vx += dv * dx;
        sum_se += sg * diff;
        if (d_b != 0.0f) {
          sum_seg += sg * diff / (double)d_b;
          ++n_grid;
        } else {
          ++n_zero;
        }
      }
    }
  }
  out->n = n;
  memcpy(out->code_hist, hist, sizeof hist);
  out->n_saturated = n_sat;
  out->n_nonfinite = n_nonfinite;
  out->n_zero_scale = n_zero;
  out->amax = (double)amax;
  out->sqnr_db = (sum_e2 > 0) ? 10.0 * log10(sum_v2 / sum_e2) : INFINITY;
  out->mean_signed_err = n ? sum_se / (double)n : 0.0;
  out->mean_signed_err_grid = n_grid ? sum_seg / (double)n_grid : 0.0;
  out->alpha = (sum_v2 > 0) ? sum_vx / sum_v2 : 1.0;
  return 0;
}
