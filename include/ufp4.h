/*
 * ufp4.h -- C ABI of the MI355X (gfx950) library for fused random-Hadamard
 * transform + 4-bit block quantization, the operand-quantization step of the
 * UFP4 FP4-pretraining recipe.
 *
 * The method (sources cited by title and section):
 *   [Z] "Shrinkage Bias: The Hidden Geometric Trap in FP4 Training ... and the
 *       UFP4 Fix" (zhichai.net) -- "Key points": the E2M1 and E1M2 grids, the
 *       RHT paradox, the fix (uniform grid, RHT on all three GEMM paths,
 *       stochastic rounding, fused RHT+quantization kernels).
 *   [A] "UFP4 Eliminates Shrinkage Bias in FP4 LLM Pretraining, Ant Group
 *       Research Finds" (autonainews.com) -- "The UFP4 Recipe": uniform E1M2 or
 *       INT4 grids, RHT on the three training GEMMs, stochastic rounding only
 *       on the output gradient dY.
 *   [H] "Rethinking Shrinkage Bias in LLM FP4 Pretraining: Geometric Origin,
 *       Systemic Impact, and UFP4 Recipe" (hotpaper.ai) -- technical approach:
 *       RHT on FPROP/DGRAD/WGRAD, SR on dY, NVFP4 and MXFP4 as comparison
 *       formats; RTNE named as the rounding that exposes E2M1's bias.
 *
 * Per 16-element block along the GEMM reduction dimension the library
 *   1. multiplies by 16 seeded random signs, runs a 16-point fast
 *      Walsh-Hadamard butterfly (stages of half-width 1, 2, 4, 8) and scales
 *      by 1/4 (an orthonormal random Hadamard transform);
 *   2. scales the block by an FP8-E4M3 block scale under an FP32 per-tensor
 *      scale (NVFP4-style), or by a power-of-two E8M0 scale per 32 elements
 *      (MXFP4-style);
 *   3. rounds onto the uniform E1M2 grid {0, .5, ..., 3.5}, symmetric INT4
 *      {-7..7}, the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} or E2M1 clamped
 *      to its uniform part {0, .5, 1, 1.5, 2}, with round-to-nearest-even
 *      or Philox-driven stochastic rounding;
 *   4. packs two 4-bit codes per byte.
 * Outputs come in the row-wise layout (blocks along a row; the fwd_y and
 * bwd_dx operands) and the column-wise layout (blocks down a column, stored
 * transposed; the bwd_dw operands), for dense tensors and for ragged
 * per-expert (MoE) row segments.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Scratch memory is a caller-owned
 *     device workspace of ufp4_workspace_size() bytes.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns before it completes.  ufp4_stats and ufp4_workspace_status
 *     synchronize the stream.
 *   - Return value: UFP4_OK, or a UFP4_ERR_* code.  Argument errors are found
 *     on the host before anything is enqueued, and leave outputs untouched.
 *     Nothing throws across the ABI.
 *   - Results are deterministic for fixed inputs and configuration.
 *   - Calls that share one workspace must not run concurrently.
 *   - Quantization calls accept cols < 2^25 and rows < 2^25 (UFP4_ERR_SHAPE
 *     otherwise).
 */
#ifndef UFP4_H
#define UFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* ufp4_stream_t; /* hipStream_t */

enum ufp4_status {
  UFP4_OK = 0,
  UFP4_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad enum value, negative size */
  UFP4_ERR_SHAPE = 2,            /* a dimension is not a multiple of the block */
  UFP4_ERR_ALIGNMENT = 3,        /* a pointer or leading dimension is misaligned */
  UFP4_ERR_WORKSPACE = 4,        /* workspace null or smaller than required */
  UFP4_ERR_HIP = 5,              /* a HIP runtime call failed */
  UFP4_ERR_OFFSETS = 6,          /* grouped offsets were found invalid on the device */
  UFP4_ERR_SYNC = 7              /* a single-pass call's device-wide exchange did not
                                    complete within 2 s (a device fault); its outputs
                                    are incomplete; the workspace stays usable (the
                                    failed call advanced its generation) */
};

/* Code layouts: E1M2, E2M1 and E2M1C store sign | magnitude index (index 0..7,
 * 0..7, 0..4); INT4 stores the two's-complement integer.  E2M1C is E2M1 with
 * its range clamped to the uniformly spaced magnitudes {0, .5, 1, 1.5, 2}
 * (Qmax 2, MX32 element emax 1): the "simulated uniform" E2M1 alternative of
 * "Shrinkage Bias: The Hidden Geometric Trap in FP4 Training" (zhichai.net),
 * section "Key points", validation results. */
enum ufp4_grid { UFP4_GRID_E1M2 = 0, UFP4_GRID_INT4 = 1, UFP4_GRID_E2M1 = 2, UFP4_GRID_E2M1C = 3 };
enum ufp4_rounding { UFP4_ROUND_RTNE = 0, UFP4_ROUND_STOCHASTIC = 1 };
/* NV16: E4M3 scale per 16 elements + FP32 per-tensor scale.
 * MX32: E8M0 (power-of-two) scale per 32 elements, no tensor scale (1.0). */
enum ufp4_scaling { UFP4_SCALE_NV16 = 0, UFP4_SCALE_MX32 = 1 };

/* Quantization configuration ("tensor, grid, RHT on/off, rounding mode and seed").
 * rht_seed selects the 16 random signs (bit j of word 0 of
 * Philox4x32-10(key = rht_seed, counter = (0,0,2,0)) set => sign j is -1); both
 * operands of one GEMM must use the same rht_seed.  sr_seed keys the random
 * words of stochastic rounding: output element i of a layout uses word i%4 of
 * Philox4x32-10(key = sr_seed, counter = (lo32(i/4), hi32(i/4), stream, 0)),
 * stream 0 for the row-wise output and 1 for the column-wise output, with i the
 * element's flat index in that output. */
typedef struct {
  int32_t grid;     /* enum ufp4_grid */
  int32_t rounding; /* enum ufp4_rounding */
  int32_t scaling;  /* enum ufp4_scaling */
  int32_t rht;      /* 0 = off, 1 = random Hadamard transform on */
  uint64_t rht_seed;
  uint64_t sr_seed;
} ufp4_config;

/* One quantized layout.  All three pointers are device pointers; codes and
 * scales may be null when the output has no elements. */
typedef struct {
  uint8_t* codes;      /* packed codes, element 2k in the low nibble of byte k */
  uint8_t* scales;     /* one byte per scale block (E4M3 or E8M0) */
  float* tensor_scale; /* one float (E floats for grouped calls) */
} ufp4_qtensor;

/* Quantization diagnostics, computed over the quantizer's own domain (v = the
 * post-RHT input, xhat = the dequantized value before any inverse RHT), with
 * binary64 sums:
 *   sqnr_db = 10 log10(sum v^2 / sum (v - xhat)^2)
 *   mean_signed_err = mean of sign(v) (xhat - v); negative = shrinkage toward
 *     zero, the bias the pages measure per rounding bucket ([Z] "Key points").
 *   mean_signed_err_grid = the same in grid units (divided by the block's
 *     dequantization factor), over elements of blocks with a nonzero scale.
 *   alpha = <v, xhat> / <v, v>, the gain of the scaled-copy-plus-orthogonal-
 *     residual decomposition of a quantized operand ([Z] "Key points").
 *   code_hist = occurrences of each 4-bit code (bucket utilisation, [H]).
 *   n_saturated = elements with |v / d_b| > Qmax; n_nonfinite = non-finite
 *     inputs; n_zero_scale = elements in blocks whose scale is zero. */
typedef struct {
  double sqnr_db, mean_signed_err, mean_signed_err_grid, alpha, amax;
  uint64_t n, code_hist[16], n_saturated, n_nonfinite, n_zero_scale;
} ufp4_stats_t;

/* Static text for a status code. */
const char* ufp4_status_string(int status);

/* Bytes of device workspace needed by any call on a tensor of `rows` x `cols`
 * with `num_groups` segments (1 for dense tensors). */
size_t ufp4_workspace_size(int64_t rows, int64_t cols, int32_t num_groups);

/* Prepare a workspace before its first use (zeroes all ws_bytes with a fill
 * kernel: the status word and the synchronization words of the single-pass
 * schedule).  Every later call leaves it ready for the next one. */
int ufp4_workspace_init(void* ws, size_t ws_bytes, ufp4_stream_t stream);

/* Reads the status word the last call left in the workspace and writes it to
 * *status_out: UFP4_OK; UFP4_ERR_OFFSETS after a grouped call whose offsets
 * the device found invalid (no output written); UFP4_ERR_SYNC after a
 * single-pass call whose exchange timed out (outputs incomplete; the next
 * single-pass call clears it); UFP4_ERR_WORKSPACE if the word holds anything
 * else (a workspace never initialized, or overwritten).  Returns UFP4_OK when
 * the word was read.  Synchronizes the stream. */
int ufp4_workspace_status(const void* ws, size_t ws_bytes, int* status_out, ufp4_stream_t stream);

/* Row-wise quantization of x[rows][ld] (bf16 bit patterns), blocks along each
 * row: the operand layout of the forward GEMM and of dY in the input-gradient
 * GEMM.  Implements steps 1-4 above for one layout: the RHT of every block
 * ("Shrinkage Bias: The Hidden Geometric Trap in FP4 Training" (zhichai.net),
 * "Key points", the RHT paradox and the fix), the two-level scale (hotpaper.ai
 * summary, technical approach: NVFP4 / MXFP4 formats), rounding onto the
 * selected grid (zhichai.net "Key points": the E2M1 and E1M2 grids;
 * autonainews.com "The UFP4 Recipe": E1M2 or INT4, stochastic rounding).  cols must be a multiple of 16 (NV16) or 32 (MX32); rows may be any
 * size >= 0.  x must be 16-byte aligned with ld a multiple of 8 elements and
 * ld >= cols; output pointers 16-byte aligned.
 * Output: codes[rows][cols/2], scales[rows][cols/B] (B = 16 or 32),
 * tensor_scale[1] (S_t = amax/(Qmax*448) for NV16, 1.0 for MX32). */
int ufp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                  const ufp4_config* cfg, ufp4_qtensor row_out, void* ws, size_t ws_bytes,
                  ufp4_stream_t stream);

/* Row-wise and column-wise quantization of the same tensor in one call: the
 * fused RHT + quantization of a training-GEMM operand in both of the
 * orientations the three GEMMs read it in ("Shrinkage Bias: The Hidden
 * Geometric Trap in FP4 Training" (zhichai.net), "Key points": RHT on all
 * three GEMM paths, fused RHT+quantization kernels; autonainews.com "The UFP4
 * Recipe": fwd_y, bwd_dx and bwd_dw operands).  rows and cols must both be
 * multiples of B.  Column-wise output is stored
 * transposed: codes[cols][rows/2], scales[cols][rows/B], tensor_scale[1]
 * (its own per-tensor scale, from the column-wise transformed values). */
int ufp4_quantize_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                         const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out,
                         void* ws, size_t ws_bytes, ufp4_stream_t stream);

/* ufp4_quantize_rowcol for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and outputs, bit for bit, without a
 * workspace.  Scratch memory is a 1 MiB array the library holds on each GPU
 * it runs on until the process ends; its address is looked up (no
 * allocation) and the array zeroed by a fill kernel on `stream` at the first
 * call on each device.  Tensors whose workspace would exceed it (more than
 * about 106,000 tiles of 128 x 256 elements, 3.4e9 elements) give
 * UFP4_ERR_WORKSPACE; a failed symbol lookup gives UFP4_ERR_HIP.  All calls
 * on one GPU share the array: calls that overlap on one GPU (concurrent
 * streams, threads) race and must be serialized by the caller.  Calls no
 * hipMalloc, hipFree or other allocating routine. */
int ufp4_quantize_rowcol_noalloc(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                 const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out,
                                 ufp4_stream_t stream);

/* Grouped (MoE) quantization of x[total_rows][cols] whose rows are split into
 * num_groups ragged segments: segment e is rows [offsets[e], offsets[e+1]);
 * the per-expert operands of the mixture-of-experts models the recipe is
 * validated on ("Shrinkage Bias: The Hidden Geometric Trap in FP4 Training"
 * (zhichai.net), "Key points", validation results: MoE models; autonainews.com
 * "Empirical Validation and Hardware Implications").  Each segment is
 * quantized exactly as ufp4_quantize_rowcol would quantize it alone, its
 * column-wise blocks zero-padded.  The column-wise line length is passed as
 * padded_rows (a host value) rather than as a device array of column offsets:
 * the offsets follow from offsets_dev and the block, and the device derives
 * them, so the two can never disagree.
 * offsets_dev: device array of num_groups+1 int64 (1 <= num_groups <= 1024,
 * else UFP4_ERR_INVALID_ARGUMENT), offsets[0] = 0, non-decreasing,
 * offsets[E] = total_rows.  Each segment gets its own tensor scale
 * per layout.  Column-wise blocks restart at each segment start; a segment's
 * last block is zero-padded to B rows and all of its outputs are stored.
 * padded_rows = sum over segments of roundup(M_e, B) (ufp4_grouped_col_offsets
 * computes it); the column output is codes[cols][padded_rows/2],
 * scales[cols][padded_rows/B], segment e occupying positions
 * [col_offsets[e], col_offsets[e+1]).  Row output as ufp4_quantize.
 * row_out.tensor_scale / col_out.tensor_scale hold num_groups floats.  Either
 * output may be skipped by passing a qtensor whose pointers are all null.  If the device finds
 * the offsets inconsistent it writes nothing and ufp4_workspace_status
 * reports UFP4_ERR_OFFSETS. */
int ufp4_quantize_grouped(const uint16_t* x, int64_t total_rows, int64_t cols,
                          const int64_t* offsets_dev, int32_t num_groups, int64_t padded_rows,
                          const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out,
                          void* ws, size_t ws_bytes, ufp4_stream_t stream);

/* Dequantize one layout in its own orientation: `rows` lines of `cols`
 * elements (for a column-wise output: rows = tensor cols, cols = tensor rows):
 * the values the GEMM consumes, x_hat = value(code) * d_b, which the pages'
 * decomposition of a quantized operand into a scaled copy plus a residual is
 * about ("Shrinkage Bias: The Hidden Geometric Trap in FP4 Training"
 * (zhichai.net), "Key points": compounding decay).
 * out[rows][cols] = value(code) * d_b, one rounding, d_b = decode(scale) * S_t
 * (NV16) or 2^(scale-127) (MX32); with inverse_rht != 0 each 16-block is then
 * mapped back through the inverse transform (butterfly, x1/4, signs). */
int ufp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                    int64_t rows, int64_t cols, const ufp4_config* cfg, int32_t inverse_rht,
                    float* out, ufp4_stream_t stream);

/* Diagnostics (ufp4_stats_t) of one dense layout of x (layout 0 row-wise,
 * 1 column-wise), the quantities the pages reason with: SQNR (zhichai.net
 * "Key points", the RHT paradox), the per-bucket mean signed error that makes
 * E2M1 shrink (zhichai.net "Key points", the cause; autonainews.com
 * "Unveiling the Geometric Roots of Shrinkage Bias"), the gain alpha and the
 * bucket utilisation (hotpaper.ai summary, core idea), against its
 * quantization (codes/scales/tensor_scale as
 * written by ufp4_quantize / _rowcol).  Uses the workspace; synchronizes the
 * stream and fills *host_out. */
int ufp4_stats(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int32_t layout,
               const ufp4_config* cfg, const uint8_t* codes, const uint8_t* scales,
               const float* tensor_scale, void* ws, size_t ws_bytes, ufp4_stats_t* host_out,
               ufp4_stream_t stream);

/* --- consumer GEMM -------------------------------------------------------- */

/* c[m][n] = sum_k xa[m][k] * xb[n][k] (fp32, row-major with stride ldc), where
 * xa and xb are the dequantized values of a and b: row-wise layouts of an
 * M x K and an N x K matrix (codes [rows][K/2]; NV16: scales [rows][K/16]
 * and one tensor scale; MX32: E8M0 scales [rows][K/32], tensor scale 1),
 * blocks along K, the reduction dimension of the training GEMMs ("Shrinkage
 * Bias: The Hidden Geometric Trap in FP4 Training" (zhichai.net), "Key
 * points": the fix quantizes the operands of all three).  Operands quantized
 * with the same RHT signs give the product of the untransformed matrices
 * (the transform is orthonormal).  NV16: each dequantized value is exact in
 * fp16 and the products are summed on the fp16 MFMA in fp32.  MX32: the
 * codes (as FP4 for E2M1 and E2M1C, expanded to FP8 E4M3 for E1M2 and INT4)
 * and the E8M0 block scales feed the scaled f8f6f4 MFMA directly, fp32
 * accumulation.  Either way the products are exact and c differs from the
 * exact sum only by fp32 accumulation order (and, for MX32, by fp32 range:
 * scaled products below fp32's smallest subnormal are lost).
 * cfg: grid and scaling of both operands.  K % 32 == 0 (UFP4_ERR_SHAPE);
 * ldc >= N; codes 16-byte aligned.  M or N of 0 writes nothing; K of 0
 * writes zeros. */
int ufp4_gemm_nt(const ufp4_config* cfg, int64_t M, int64_t N, int64_t K, ufp4_qtensor a, ufp4_qtensor b,
                 float* c, int64_t ldc, ufp4_stream_t stream);

/* --- delayed scaling ------------------------------------------------------ */

/* Pairs of maxima a delayed call on a rows x cols tensor writes to amax_out
 * (one per 128 x 256 tile; 0 for an empty tensor). */
int64_t ufp4_amax_tiles(int64_t rows, int64_t cols);

/* Delayed-scaling quantization (NV16 only): as ufp4_quantize_rowcol (or
 * ufp4_quantize when col_out.tensor_scale is NULL), but the per-tensor
 * scales come from provided maxima instead of this tensor's own, so the
 * input is read once by one kernel.
 *   amax_in: device, n_in >= 1 pairs (row-wise, column-wise), each a maximum
 *     of |transformed value| (after the RHT's 1/4; of |x| without the RHT)
 *     for that layout.  The effective maximum of a layout is the largest
 *     entry, an entry that is not a positive finite number counting as zero
 *     (then S_t = 1).  S_t = max / (Qmax * 448).
 *   amax_out: device, ufp4_amax_tiles(rows, cols) pairs, or NULL: this
 *     call's exact tile maxima in the same units, to pass as the next call's
 *     amax_in (their largest entries are this tensor's maxima).  It must not
 *     overlap amax_in (UFP4_ERR_INVALID_ARGUMENT).
 *   Blocks whose maximum exceeds the provided one saturate: E4M3 scale 448,
 *   codes at +-Qmax.  With a provided maximum equal to the tensor's own the
 *   outputs equal ufp4_quantize_rowcol's bit for bit.
 * Shapes, alignment and layouts as ufp4_quantize_rowcol (rows % 16 == 0 only
 * with the column-wise layout); amax_in and amax_out 8-byte aligned.  No
 * workspace.  MX32 gives UFP4_ERR_INVALID_ARGUMENT (it has no tensor
 * scale).  This is a numerics choice (delayed scaling), not the pages'
 * recipe, which takes each tensor's own maximum. */
int ufp4_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                          const ufp4_config* cfg, const float* amax_in, int32_t n_in, float* amax_out,
                          ufp4_qtensor row_out, ufp4_qtensor col_out, ufp4_stream_t stream);

/* Delayed scaling of grouped (MoE) segments (NV16 only): as
 * ufp4_quantize_grouped, but segment e's tensor scales come from provided
 * maxima instead of the segment's own, so the input is read once by one
 * kernel (the mixture-of-experts operands of "Shrinkage Bias: The Hidden
 * Geometric Trap in FP4 Training" (zhichai.net), "Key points", validation
 * results; the maxima rules of ufp4_quantize_delayed, per segment).
 *   amax_in: device, num_groups pairs (row-wise, column-wise): maxima of
 *     |transformed value| (after the RHT's 1/4; of |x| without the RHT) of
 *     each segment's values in that layout.  An entry that is not a positive
 *     finite number counts as zero (S_t = 1).  S_t = max / (Qmax * 448).
 *   amax_out: device, num_groups pairs, or NULL: this call's own per-segment
 *     maxima in the same units (0 for an empty segment or a layout not
 *     requested), to pass as the next call's amax_in when the routing stays
 *     comparable.  Must not overlap amax_in (UFP4_ERR_INVALID_ARGUMENT).
 *   Blocks whose maximum exceeds the provided one saturate (E4M3 scale 448,
 *   codes at +-Qmax).  With each segment's own maxima provided, the outputs
 *   equal ufp4_quantize_grouped's bit for bit.
 * Shapes, layouts, offsets rules and workspace (its status word reports
 * offsets the device rejects) as ufp4_quantize_grouped; amax_in and amax_out
 * 8-byte aligned.  MX32 gives UFP4_ERR_INVALID_ARGUMENT.  A numerics choice
 * (delayed scaling), not the pages' recipe, which takes each tensor's own
 * maximum. */
int ufp4_quantize_grouped_delayed(const uint16_t* x, int64_t total_rows, int64_t cols,
                                  const int64_t* offsets_dev, int32_t num_groups, int64_t padded_rows,
                                  const ufp4_config* cfg, const float* amax_in, float* amax_out,
                                  ufp4_qtensor row_out, ufp4_qtensor col_out, void* ws, size_t ws_bytes,
                                  ufp4_stream_t stream);

/* --- schedule ------------------------------------------------------------ */

/* Dense NV16 calls need the tensor maximum before any code is written.
 * UFP4_SCHEDULE_TWO_PASS runs two kernels: tile maxima, then quantization
 * (the input is read twice).  UFP4_SCHEDULE_SINGLE_PASS runs one kernel
 * whose workgroups keep their tile on chip while the tile maxima are
 * exchanged through the workspace, so the input is read once; it applies to
 * tensors of at most 1024 tiles of 128 x 256 elements (others take two
 * passes).  It wants every tile resident at once; a workgroup that finds
 * some tile not started within 100 us leaves its tile to the workgroups that
 * did start, which reload and quantize it, so the call always completes
 * (slowly when the device is shared).  UFP4_SCHEDULE_AUTO (the default)
 * takes the single pass for row+column calls whose tiles the device holds
 * at once (two per compute unit; the faster schedule there on MI355X) and
 * two passes otherwise.  Results are bit-identical in every schedule.
 * Process-wide setting. */
enum ufp4_schedule { UFP4_SCHEDULE_AUTO = 0, UFP4_SCHEDULE_TWO_PASS = 1, UFP4_SCHEDULE_SINGLE_PASS = 2 };

/* Select the schedule.  left_stride (test hook, single-pass schedule only):
 * when > 1, every tile whose index is not a multiple of it is left to the
 * others as if it had found the device full; 0 or 1 leaves none.
 * UFP4_ERR_INVALID_ARGUMENT for an unknown schedule or a negative stride. */
int ufp4_set_schedule(int32_t schedule, int32_t left_stride);

/* The schedule a quantization call on a tensor of rows x cols with
 * num_groups segments and this configuration takes on the current device
 * under the current setting, for a call with both layouts (both_layouts != 0,
 * ufp4_quantize_rowcol) or one: UFP4_SCHEDULE_SINGLE_PASS or
 * UFP4_SCHEDULE_TWO_PASS (also for MX32, grouped and empty tensors, which
 * need no separate maxima pass or have their own).  Host only. */
int ufp4_schedule_of(int64_t rows, int64_t cols, int32_t num_groups, int32_t both_layouts,
                     const ufp4_config* cfg, int32_t* schedule_out);

/* --- training recipes ------------------------------------------------------ */

/* The quantization of each operand of the three training GEMMs under a
 * recipe.  The GEMMs of a linear layer Y = X W^T (X: tokens x in, W: out x in,
 * dY: tokens x out) and the operands ufp4_gemm_nt takes for them (a: M x K,
 * b: N x K, blocks along K, the reduction dimension):
 *   fwd_y  Y  = X W^T : a = X  row-wise,    b = W  row-wise     (K = in)
 *   bwd_dx dX = dY W  : a = dY row-wise,    b = W  column-wise  (K = out)
 *   bwd_dw dW = dY^T X: a = dY column-wise, b = X  column-wise  (K = tokens)
 * Recipes:
 *   UFP4: E1M2 grid, NV16 scales, RHT on all three GEMMs, stochastic
 *     rounding on dY only, RTNE elsewhere ("Shrinkage Bias: The Hidden
 *     Geometric Trap in FP4 Training" (zhichai.net), "Key points", the fix;
 *     "UFP4 Eliminates Shrinkage Bias ..." (autonainews.com), "The UFP4
 *     Recipe"; hotpaper.ai summary, technical approach).
 *   UFP4_INT4: the same with the symmetric INT4 grid (autonainews.com, "The
 *     UFP4 Recipe": E1M2 or INT4).
 *   NVFP4: the E2M1 baseline, RHT on bwd_dw only (zhichai.net, "Key points":
 *     the RHT paradox; practitioners on E2M1-only hardware restrict RHT to
 *     bwd_dw).  The pages do not say where the baseline rounds
 *     stochastically; it keeps UFP4's choice (dY only), so the two presets
 *     differ only in the grid and the RHT coverage.
 * Both operands of one GEMM must share rht_seed (the signs must match along
 * K); sr_seed is used only where the preset rounds stochastically (0 is
 * written otherwise).  Host only; UFP4_ERR_INVALID_ARGUMENT for an unknown
 * enum value or a null output. */
enum ufp4_recipe { UFP4_RECIPE_UFP4 = 0, UFP4_RECIPE_UFP4_INT4 = 1, UFP4_RECIPE_NVFP4 = 2 };
enum ufp4_gemm_path { UFP4_GEMM_FWD_Y = 0, UFP4_GEMM_BWD_DX = 1, UFP4_GEMM_BWD_DW = 2 };
enum ufp4_operand { UFP4_OPERAND_A = 0, UFP4_OPERAND_B = 1 };
enum ufp4_tensor_role { UFP4_TENSOR_X = 0, UFP4_TENSOR_W = 1, UFP4_TENSOR_DY = 2 };

/* Writes the configuration, the layout (0 row-wise, 1 column-wise) and the
 * tensor (enum ufp4_tensor_role) of operand `operand` of GEMM `gemm` under
 * `recipe`. */
int ufp4_recipe_config(int32_t recipe, int32_t gemm, int32_t operand, uint64_t rht_seed, uint64_t sr_seed,
                       ufp4_config* cfg_out, int32_t* layout_out, int32_t* tensor_out);

/* --- diagnostic hooks (not on the hot path) ------------------------------ */

/* out_dev[i] = in_dev[i] rounded to bf16 (nearest, ties to even; NaN stays a
 * quiet NaN): the conversion between the layers of a chain of quantized
 * GEMMs, whose fp32 outputs feed the next layer's bf16 quantizer (the
 * compounding of the GEMM gain through layers, "Shrinkage Bias: The Hidden
 * Geometric Trap in FP4 Training" (zhichai.net), "Key points").  Device
 * pointers, in_dev 4-byte and out_dev 2-byte aligned (UFP4_ERR_ALIGNMENT);
 * n < 0 gives UFP4_ERR_INVALID_ARGUMENT. */
int ufp4_f32_to_bf16(const float* in_dev, int64_t n, uint16_t* out_dev, ufp4_stream_t stream);

/* codes_dev[i] = 4-bit code (one per byte) of y_dev[i] rounded at unit scale
 * onto `grid`, with the stochastic-rounding word of index i in stream 0.
 * +-inf saturates to +-Qmax; NaN gives code 0. */
int ufp4_round_f32(const float* y_dev, int64_t n, int32_t grid, int32_t rounding,
                   uint64_t sr_seed, uint8_t* codes_dev, ufp4_stream_t stream);

/* Measurement hook (not part of the quantization path): one
 * ufp4_quantize_rowcol call with NV16 scaling on `stream`, whose kernels are
 * launched with start/stop hipEvents that the runtime stamps with each
 * kernel's own start and end.  Synchronizes the stream and writes the kernel
 * durations in milliseconds to host memory: the tensor-maximum kernel's in
 * *ms_amax_host and the quantization kernel's in *ms_quant_host (under the
 * single-pass schedule, 0 and the one kernel's).  Other arguments and outputs exactly as ufp4_quantize_rowcol.
 * rows or cols of 0, MX32 scaling or a null duration pointer give
 * UFP4_ERR_INVALID_ARGUMENT.  Not for use under stream capture. */
int ufp4_time_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                     const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out,
                     void* ws, size_t ws_bytes, ufp4_stream_t stream, float* ms_amax_host,
                     float* ms_quant_host);

/* Measurement hook (not part of the quantization path): the memory traffic
 * of a dense NV16 ufp4_quantize_rowcol call on the same tensor with no
 * arithmetic, for the bandwidth this access pattern attains.  Reads the
 * rows x cols bf16 tensor x (ld = cols) with the quantization kernels' tile
 * walk and 16-byte loads, and writes every byte of both layouts' codes and
 * block scales (row_out: rows x cols, col_out: cols x rows, as
 * ufp4_quantize_rowcol) with coalesced 16-byte stores (column-wise scales:
 * 8-byte); tensor scales are not
 * touched.  The bytes written are zero unless a lane's 64 input words xor to
 * one fixed constant.  rows must be a multiple of 128 and cols of 256
 * (UFP4_ERR_SHAPE); x, the codes and the row-wise scales 16-byte and the
 * column-wise scales 8-byte aligned (UFP4_ERR_ALIGNMENT); null pointers give
 * UFP4_ERR_INVALID_ARGUMENT.  Asynchronous on `stream`. */
int ufp4_roof_rowcol(const uint16_t* x, int64_t rows, int64_t cols, ufp4_qtensor row_out, ufp4_qtensor col_out,
                     ufp4_stream_t stream);

/* The 16 signs (+1/-1) selected by rht_seed (host memory). */
int ufp4_rht_signs(uint64_t rht_seed, int8_t signs_host[16]);

/* Host helper: col_offsets[e] = sum over e' < e of roundup(offsets[e+1]-offsets[e], block),
 * for e = 0..num_groups (col_offsets[num_groups] = padded_rows). */
int ufp4_grouped_col_offsets(const int64_t* offsets_host, int32_t num_groups, int32_t block,
                             int64_t* col_offsets_host);

#ifdef __cplusplus
}
#endif
#endif /* UFP4_H */
