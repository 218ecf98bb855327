/*
 * ufp4_oracle.h -- plain, slow, single-threaded CPU oracle for the UFP4
 * quantization hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check
 * and the CPU-baseline leg of the benchmark may load or call this code.  The
 * product path (the HIP library) shares no code, header, table or constant
 * with it, and must never fall back to it.
 *
 * Sources (cited by title and section; all three describe one paper):
 *   [Z] "Shrinkage Bias: The Hidden Geometric Trap in FP4 Training ... and the
 *       UFP4 Fix" (zhichai.net forum mirror) -- sections "Key points",
 *       "Engineering implications".
 *   [A] "UFP4 Eliminates Shrinkage Bias in FP4 LLM Pretraining, Ant Group
 *       Research Finds" (autonainews.com) -- sections "Unveiling the Geometric
 *       Roots of Shrinkage Bias", "The UFP4 Recipe".
 *   [H] "Rethinking Shrinkage Bias in LLM FP4 Pretraining: Geometric Origin,
 *       Systemic Impact, and UFP4 Recipe" (hotpaper.ai summary) -- abstract,
 *       core idea, technical approach.
 *   Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *       Easy as 1, 2, 3", SC'11.  E4M3 / E8M0: OCP 8-bit floating point and
 *       OCP Microscaling (MX) v1.0 specifications.
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, no FMA contraction
 * (built with -ffp-contract=off, no -ffast-math); statistics in binary64.
 *
 * Parity status of each function is listed in the file's implementation
 * header and in the tests that pin it.
 */
#ifndef UFP4_ORACLE_H
#define UFP4_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_GRID_E1M2 = 0, ORC_GRID_INT4 = 1, ORC_GRID_E2M1 = 2, ORC_GRID_E2M1_CLAMP = 3 };
enum { ORC_ROUND_RTNE = 0, ORC_ROUND_SR = 1 };
enum { ORC_SCALE_NV16 = 0, ORC_SCALE_MX32 = 1 };
enum { ORC_LAYOUT_ROW = 0, ORC_LAYOUT_COL = 1 };

typedef struct {
  int32_t grid, rounding, scaling, rht;
  uint64_t rht_seed, sr_seed;
} orc_config;

typedef struct {
  double sqnr_db, mean_signed_err, mean_signed_err_grid, alpha, amax;
  uint64_t n, code_hist[16], n_saturated, n_nonfinite, n_zero_scale;
} orc_stats;

/* --- primitives ---------------------------------------------------------- */
float orc_bf16_to_f32(uint16_t h);
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void orc_rht_signs(uint64_t rht_seed, int8_t signs[16]);
uint32_t orc_sr_word(uint64_t sr_seed, uint64_t index, uint32_t stream);
void orc_fwht16_stages(float v[16]);                       /* 4 butterfly stages, no scaling */
void orc_rht16(const float x[16], const int8_t signs[16], float v[16]);
void orc_inverse_rht16(const float v[16], const int8_t signs[16], float x[16]);
uint8_t orc_e4m3_encode(float q);                          /* q >= 0; RNE; saturate at 448 */
void orc_e4m3_encode_n(const float* q, int64_t n, uint8_t* out);  /* batch form */
float orc_e4m3_decode(uint8_t c);
float orc_grid_qmax(int32_t grid);
float orc_code_value(uint8_t code, int32_t grid);
uint8_t orc_round_to_code(float y, int32_t grid, int32_t rounding, uint32_t r32);

/* Exhaustive-test hook: codes[i] = quantized y[i] at unit scale; SR word for
 * element i uses stream 0 and index i. */
int orc_round_f32(const float* y, int64_t n, int32_t grid, int32_t rounding,
                  uint64_t sr_seed, uint8_t* codes);

/* --- whole-tensor drivers ------------------------------------------------- */
/* Quantize one layout of a dense bf16 matrix x[rows][ld].
 * ORC_LAYOUT_ROW: blocks run along a row; codes[rows][cols/2],
 *                 scales[rows][cols/B] (B = 16 for NV16, 32 for MX32).
 * ORC_LAYOUT_COL: blocks run down a column; output is stored transposed:
 *                 codes[cols][rows/2], scales[cols][rows/B].
 * tensor_scale receives one float.  Returns 0, or a positive error code for a
 * shape the layout cannot block. */
int orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                 const orc_config* cfg, int32_t layout,
                 uint8_t* codes, uint8_t* scales, float* tensor_scale);

/* Padded column offsets of a grouped (per-expert) tensor: exclusive scan of
 * each segment's row count rounded up to the scale block. */
/* Delayed scaling (NV16 only): as orc_quantize, but the tensor scale comes
 * from amax_given, a maximum of the layout's transformed values supplied by
 * the caller (for instance the previous step's), instead of from this
 * tensor.  A given maximum that is not a positive finite number counts as
 * zero (S_t = 1).  Blocks above it saturate.  *amax_seen receives this
 * tensor's own maximum for the layout.  Returns 1 for MX32. */
int orc_quantize_given_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            const orc_config* cfg, int32_t layout, float amax_given,
                            uint8_t* codes, uint8_t* scales, float* tensor_scale, float* amax_seen);

int orc_grouped_col_offsets(const int64_t* offsets, int32_t num_groups, int32_t block,
                            int64_t* col_offsets);

/* Grouped quantization: rows [offsets[e], offsets[e+1]) form segment e, with
 * its own tensor scale.  Row output has the dense row shape; column output is
 * codes[cols][R_pad/2], scales[cols][R_pad/B], R_pad = col_offsets[E]. */
int orc_quantize_grouped(const uint16_t* x, int64_t total_rows, int64_t cols,
                         const int64_t* offsets, int32_t num_groups, const orc_config* cfg,
                         uint8_t* row_codes, uint8_t* row_scales, float* row_tensor_scale,
                         uint8_t* col_codes, uint8_t* col_scales, float* col_tensor_scale);

/* Grouped delayed scaling (NV16 only): as orc_quantize_grouped, but segment
 * e's tensor scales come from amax_given[2e] (row-wise) and amax_given[2e+1]
 * (column-wise), maxima of that segment's transformed values supplied by the
 * caller, with the same rules as orc_quantize_given_amax; amax_seen (may be
 * null) receives each segment's own maxima in the same layout (0 for an
 * empty segment).  Returns 1 for MX32. */
int orc_quantize_grouped_given_amax(const uint16_t* x, int64_t total_rows, int64_t cols,
                                    const int64_t* offsets, int32_t num_groups, const orc_config* cfg,
                                    const float* amax_given, float* amax_seen,
                                    uint8_t* row_codes, uint8_t* row_scales, float* row_tensor_scale,
                                    uint8_t* col_codes, uint8_t* col_scales, float* col_tensor_scale);

/* Dequantize one layout, in that layout's own orientation (rows = number of
 * block lines, cols = elements per line).  Optional inverse RHT per block. */
int orc_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                   int64_t rows, int64_t cols, const orc_config* cfg, int32_t inverse_rht,
                   float* out);

/* Quantization diagnostics over the quantizer's domain (post-RHT input v,
 * dequantized xhat without inverse RHT). */
int orc_compute_stats(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                      int32_t layout, const orc_config* cfg, const uint8_t* codes,
                      const uint8_t* scales, const float* tensor_scale, orc_stats* out);

#ifdef __cplusplus
}
#endif
#endif
