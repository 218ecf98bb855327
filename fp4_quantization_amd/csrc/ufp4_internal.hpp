// ufp4_internal.hpp -- host/device shared parameter blocks and launchers of
// the gfx950 kernels (internal to the library; the public ABI is ufp4.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ufp4_device.hpp"

namespace ufp4 {

// Geometry of the quantization kernels.  A workgroup of 4 wavefronts covers a
// tile of kTileRows x kBandCols elements: each wavefront a 32-row strip (two
// 16-row halves, one per 32-lane half of the wavefront), each lane 16 rows x 8
// columns (one 16-byte load per row).
constexpr int kThreads = 256;
constexpr int kBandCols = 256;
constexpr int kTileRows = 128;
constexpr int kMaxGroups = 1024;
constexpr int kNumXcd = 8;

struct QuantParams {
  const uint16_t* x;
  int64_t rows, cols, ld;
  const int64_t* offsets;  // grouped: device offsets[E+1]; dense: null
  int32_t num_groups;      // E (1 for a dense tensor)
  int32_t block;           // 16 (NV16) or 32 (MX32)
  int64_t padded_rows;     // length of a column-wise output line
  uint8_t* row_codes;
  uint8_t* row_scales;
  float* row_ts;
  uint8_t* col_codes;
  uint8_t* col_scales;
  float* col_ts;
  int32_t do_row, do_col, rht, mx, grid, sr;
  uint32_t sr_k0, sr_k1;
  RhtSigns sg;        // folded signs for in-lane (column-wise) blocks
  HalfSigns hs[2];    // folded signs for the two 8-column halves of a row block
  float s4[2];        // stage-4 multiplier of the partner value, per lane parity
  float fin_lane[2];  // output multiplier per lane parity (row-wise blocks)
  int32_t n_band;     // column bands of kBandCols
  int32_t n_tiles;    // row tiles per band (upper bound for grouped)
  int32_t n_work;     // n_band * n_tiles (workgroups beyond this are idle)
  // workspace
  uint32_t* ws_status;  // grouped calls: 0, or UFP4_ERR_OFFSETS
  float2* ws_part;      // [n_work]: per tile, max |transform| (row-wise, column-wise)
  // delayed scaling: provided maxima in, this call's tile maxima out
  const float2* amax_in;  // [n_in] (row-wise, column-wise) maxima of the transformed values
  int32_t n_in;
  float2* amax_out;       // [n_work], or null
  // single-pass schedule
  uint32_t* fs_gen;          // call generation, advanced once per call
  uint64_t* fs_words;        // generation-tagged words: start words, tile maxima, aggregators' results
  int32_t fs_orphan_stride;  // > 1: tiles whose index is not a multiple leave their work to others
};

// Workspace layout (bytes): a 256-byte header (status word at 4, call
// generation at 128), the single-pass schedule's generation-tagged words
// (start words in kFsReplicas copies, tile maxima and the aggregators'
// results, up to kMaxFusedTiles tiles; nothing else is
// ever stored there, so a stale word carries an older generation), then one
// float2 partial per tile for the two-pass schedule.
constexpr size_t kWsHeader = 256;
constexpr size_t kWsGenOffset = 128;
constexpr int kMaxFusedTiles = 1024;
// The single-pass start words are written in kFsReplicas copies and each
// workgroup reads one of them, so that no memory line has more than
// 1/kFsReplicas of the workgroups reading it.
constexpr int kFsReplicas = 8;
constexpr size_t kWsFusedWords = ((size_t)(kFsReplicas + 2) * kMaxFusedTiles + 64 * 16) * sizeof(uint64_t);
constexpr size_t kWsPartOffset = kWsHeader + kWsFusedWords;

void fill_rht_signs(uint64_t seed, QuantParams& p);
uint32_t rht_sign_mask(uint64_t seed);

int64_t grid_size_quant(int64_t rows, int64_t cols, int32_t groups, int32_t block, int32_t* n_band,
                        int32_t* n_tiles);

// With non-null events the kernel's start and end are recorded in them.
hipError_t launch_amax(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0 = nullptr,
                       hipEvent_t t1 = nullptr);
hipError_t launch_quant(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);
// Delayed scaling (dense NV16): one kernel, tensor scales from p.amax_in.
hipError_t launch_delayed(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0 = nullptr,
                          hipEvent_t t1 = nullptr);
// Delayed scaling of grouped (MoE) segments (NV16): one kernel, per-segment
// tensor scales from p.amax_in[e], per-segment maxima folded into
// p.amax_out[e] (zeroed beforehand) when it is not null.
hipError_t launch_grouped_delayed(const QuantParams& p, int64_t grid, hipStream_t s);
hipError_t launch_roof(const QuantParams& p, int64_t grid, hipStream_t s);
// The single-pass schedule (dense NV16 tensors of at most kMaxFusedTiles
// tiles): one kernel, every tile kept in registers across a device-wide
// exchange of the tile maxima.
hipError_t launch_fused(const QuantParams& p, int64_t grid, hipStream_t s, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);
hipError_t launch_fill(uint32_t* p, int64_t n, uint32_t value, hipStream_t s);

struct DequantParams {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  int64_t rows, cols;
  int32_t grid, mx, inverse;
  float d[16];  // signs of the inverse transform
  float* out;
};
hipError_t launch_dequant(const DequantParams& p, hipStream_t s);

struct StatsParams {
  const uint16_t* x;
  int64_t rows, cols, ld;
  int32_t layout, grid, mx, rht;
  RhtSigns sg;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  double* part;  // per workgroup: 5 doubles + 20 counters (as double-size slots)
  int32_t n_wg;
};
constexpr int kStatsSlots = 32;  // 8-byte slots per workgroup partial
hipError_t launch_stats(const StatsParams& p, hipStream_t s);

hipError_t launch_round(const float* y, int64_t n, int32_t grid, int32_t rounding, uint64_t seed,
                        uint8_t* codes, hipStream_t s);

// Consumer GEMM of two NV16 row-wise layouts along K (codes [rows][K/2],
// scales [rows][K/16], one tensor scale each); C row-major with stride ldc.
struct GemmParams {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_ts;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_ts;
  float* c;
  int64_t M, N, K, ldc;
  int32_t grid;
  int32_t mx;  // MX32 operands (E8M0 scales per 32), else NV16
};
hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
hipError_t launch_to_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s);

}  // namespace ufp4
