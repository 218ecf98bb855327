/* oracle_driver.c -- runs every oracle function on small inputs under the
 * address and undefined-behaviour sanitizers: every configuration (grids,
 * roundings, scalings, transform on and off, given maxima), both layouts,
 * grouped segments that are empty, shorter than a block or ragged, and
 * inputs holding zeros, subnormals, huge values, infinities and NaNs.  Each
 * output buffer is allocated at its exact size, so a write past its end is
 * reported.  Exit status 0 when every call returned its expected status. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/ufp4_oracle.h"

static int g_fail = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static uint64_t g_state = 0x243F6A8885A308D3ull;
static uint32_t rnd32(void) { /* splitmix64 */
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

/* bf16 bit patterns: mostly moderate magnitudes, some specials */
static void fill(uint16_t* x, int64_t n, int specials) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t r = rnd32();
    uint16_t e = (uint16_t)(120 + (r >> 8) % 16), m = (uint16_t)(r & 0x7F), s = (uint16_t)((r >> 16) & 1);
    x[i] = (uint16_t)((s << 15) | (e << 7) | m);
    if (specials) {
      switch ((r >> 20) % 64) {
        case 0: x[i] = 0; break;
        case 1: x[i] = 0x8000; break;
        case 2: x[i] = (uint16_t)(r & 0x7F); break;       /* subnormal */
        case 3: x[i] = 0x7F7F; break;                      /* largest finite */
        case 4: if (specials > 1) x[i] = 0x7F80; break;   /* +inf */
        case 5: if (specials > 1) x[i] = 0x7FC1; break;   /* NaN */
        default: break;
      }
    }
  }
}

static void run_dense(int64_t R, int64_t C, int64_t ld, int specials) {
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(R * ld));
  fill(x, R * ld, specials);
  for (int grid = 0; grid < 4; ++grid)
    for (int rnd = 0; rnd < 2; ++rnd)
      for (int scl = 0; scl < 2; ++scl)
        for (int rht = 0; rht < 2; ++rht) {
          orc_config cfg = {grid, rnd, scl, rht, 5, 6};
          int B = scl ? 32 : 16;
          for (int layout = 0; layout < 2; ++layout) {
            int64_t lines = layout ? C : R, len = layout ? R : C;
            int ok_shape = len % B == 0;
            uint8_t* codes = malloc((size_t)(lines * len / 2) + 1);
            uint8_t* scales = malloc((size_t)(lines * len / B) + 1);
            float* out = malloc(sizeof(float) * (size_t)(lines * len) + 1);
            float ts = 0.0f, seen = 0.0f;
            int rc = orc_quantize(x, R, C, ld, &cfg, layout, codes, scales, &ts);
            EXPECT((rc == 0) == ok_shape);
            if (rc) goto next;
            EXPECT(orc_dequantize(codes, scales, &ts, lines, len, &cfg, 0, out) == 0);
            EXPECT(orc_dequantize(codes, scales, &ts, lines, len, &cfg, 1, out) == 0);
            orc_stats st;
            EXPECT(orc_compute_stats(x, R, C, ld, layout, &cfg, codes, scales, &ts, &st) == 0);
            if (!scl) {
              const float given[4] = {1.0f, 0.0f, -1.0f, INFINITY};
              for (int g = 0; g < 4; ++g)
                EXPECT(orc_quantize_given_amax(x, R, C, ld, &cfg, layout, given[g], codes, scales, &ts, &seen) == 0);
            } else {
              EXPECT(orc_quantize_given_amax(x, R, C, ld, &cfg, layout, 1.0f, codes, scales, &ts, &seen) == 1);
            }
          next:
            free(codes);
            free(scales);
            free(out);
          }
        }
  free(x);
}

static void run_grouped(const int64_t* counts, int E, int64_t C) {
  int64_t* off = malloc(sizeof(int64_t) * (size_t)(E + 1));
  off[0] = 0;
  for (int e = 0; e < E; ++e) off[e + 1] = off[e] + counts[e];
  const int64_t R = off[E];
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(R * C) + 2);
  fill(x, R * C, 1);
  for (int scl = 0; scl < 2; ++scl)
    for (int rnd = 0; rnd < 2; ++rnd) {
      orc_config cfg = {0, rnd, scl, 1, 3, 4};
      int B = scl ? 32 : 16;
      int64_t* coff = malloc(sizeof(int64_t) * (size_t)(E + 1));
      EXPECT(orc_grouped_col_offsets(off, E, B, coff) == 0);
      const int64_t Rp = coff[E];
      uint8_t* rc = malloc((size_t)(R * C / 2) + 1);
      uint8_t* rs = malloc((size_t)(R * C / B) + 1);
      uint8_t* cc = malloc((size_t)(C * Rp / 2) + 1);
      uint8_t* cs = malloc((size_t)(C * Rp / B) + 1);
      float* rts = malloc(sizeof(float) * (size_t)E);
      float* cts = malloc(sizeof(float) * (size_t)E);
      EXPECT(orc_quantize_grouped(x, R, C, off, E, &cfg, rc, rs, rts, cc, cs, cts) == 0);
      EXPECT(orc_quantize_grouped(x, R, C, off, E, &cfg, rc, rs, rts, NULL, NULL, cts) == 0);
      EXPECT(orc_quantize_grouped(x, R, C, off, E, &cfg, NULL, NULL, rts, cc, cs, cts) == 0);
      free(coff);
      free(rc);
      free(rs);
      free(cc);
      free(cs);
      free(rts);
      free(cts);
    }
  int64_t bad[3] = {0, 9, 4};
  int64_t co[3];
  EXPECT(orc_grouped_col_offsets(bad, 2, 16, co) != 0);
  free(x);
  free(off);
}

int main(void) {
  /* primitives */
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, w[4];
  orc_philox4x32_10(ctr, key, w);
  int8_t signs[16];
  orc_rht_signs(0xFFFFFFFFFFFFFFFFull, signs);
  for (int j = 0; j < 16; ++j) EXPECT(signs[j] == 1 || signs[j] == -1);
  (void)orc_sr_word(7, 0xFFFFFFFFFFFFFFFFull, 1);
  float v[16], xb[16];
  for (int j = 0; j < 16; ++j) v[j] = (float)j - 7.5f;
  orc_rht16(v, signs, xb);
  orc_inverse_rht16(xb, signs, v);
  for (int c = 0; c < 256; ++c) (void)orc_e4m3_decode((uint8_t)c);
  const float q[8] = {0.0f, 1e-30f, 0.001953125f, 1.0f, 447.9f, 448.0f, 464.0f, 1e30f};
  uint8_t e8[8];
  orc_e4m3_encode_n(q, 8, e8);
  for (int g = 0; g < 4; ++g) {
    EXPECT(orc_grid_qmax(g) > 0.0f);
    for (int c = 0; c < 16; ++c) (void)orc_code_value((uint8_t)c, g);
  }
  /* the rounding hook over every bf16 pattern, every grid and rounding */
  float* y = malloc(sizeof(float) * 65536);
  uint8_t* codes = malloc(65536);
  for (int h = 0; h < 65536; ++h) y[h] = orc_bf16_to_f32((uint16_t)h);
  for (int g = 0; g < 4; ++g)
    for (int r = 0; r < 2; ++r) EXPECT(orc_round_f32(y, 65536, g, r, 99, codes) == 0);
  EXPECT(orc_round_f32(y, 4, 7, 0, 0, codes) != 0);
  free(y);
  free(codes);
  /* dense tensors: several tiles' worth of shapes, ragged ones, padded ld */
  run_dense(64, 64, 64, 1);
  run_dense(48, 96, 104, 2);
  run_dense(32, 40, 40, 1);   /* 40 columns: MX32 rejects, NV16 rejects */
  run_dense(0, 32, 32, 0);
  run_dense(16, 0, 0, 0);
  run_dense(1, 16, 16, 2);
  /* grouped: empty segments, segments shorter than a block, ragged ones */
  const int64_t c1[6] = {0, 5, 16, 37, 1, 0};
  run_grouped(c1, 6, 64);
  const int64_t c2[3] = {70, 0, 33};
  run_grouped(c2, 3, 32);
  if (g_fail) {
    fprintf(stderr, "%d oracle checks failed\n", g_fail);
    return 1;
  }
  printf("oracle sanitizer run passed\n");
  return 0;
}
