// launch_stubs.cpp -- stand-ins for the kernel launchers, linked instead of
// the device code into a sanitized host build of the C ABI.  Each checks the
// launch geometry and the parameter block the ABI prepared, counts the
// call, and returns success (so the ABI's host path runs to its end) or the
// error the driver asked for.  No GPU is touched.
#include <stdio.h>
#include <stdlib.h>

#include "../../fp4_quantization_amd/csrc/ufp4_internal.hpp"

namespace ufp4 {

int g_stub_calls = 0;
hipError_t g_stub_result = hipSuccess;

static void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launch stub: %s\n", what);
    abort();
  }
}

static hipError_t quant_launch(const QuantParams& p, int64_t grid, const char* kind) {
  ++g_stub_calls;
  require(p.x != nullptr, kind);
  require(p.rows > 0 && p.cols > 0 && p.ld >= p.cols, "shape");
  require(p.n_band > 0 && p.n_tiles > 0 && p.n_work == p.n_band * p.n_tiles, "work items");
  require(grid >= p.n_work && grid % kNumXcd == 0 && grid <= 0x7FFFFFFF, "grid");
  require(p.block == 16 || p.block == 32, "block");
  require(p.do_row || p.do_col, "no layout");
  if (p.do_row) require(p.row_ts != nullptr && p.row_codes && p.row_scales, "row outputs");
  if (p.do_col) require(p.col_ts != nullptr && p.col_codes && p.col_scales && p.padded_rows >= p.rows, "col outputs");
  require(p.num_groups >= 1 && p.num_groups <= kMaxGroups, "groups");
  return g_stub_result;
}

hipError_t launch_amax(const QuantParams& p, int64_t grid, hipStream_t, hipEvent_t, hipEvent_t) {
  require(p.ws_part != nullptr && !p.mx, "amax partials");
  return quant_launch(p, grid, "amax");
}
hipError_t launch_quant(const QuantParams& p, int64_t grid, hipStream_t, hipEvent_t, hipEvent_t) {
  require(p.mx || p.ws_part != nullptr, "quant partials");
  return quant_launch(p, grid, "quant");
}
hipError_t launch_delayed(const QuantParams& p, int64_t grid, hipStream_t, hipEvent_t, hipEvent_t) {
  require(p.amax_in != nullptr && p.n_in >= 1 && !p.mx && p.offsets == nullptr, "delayed");
  return quant_launch(p, grid, "delayed");
}
hipError_t launch_grouped_delayed(const QuantParams& p, int64_t grid, hipStream_t) {
  require(p.amax_in != nullptr && p.n_in == p.num_groups && p.offsets != nullptr && !p.mx && p.ws_status, "grouped delayed");
  return quant_launch(p, grid, "grouped delayed");
}
hipError_t launch_fused(const QuantParams& p, int64_t grid, hipStream_t, hipEvent_t, hipEvent_t) {
  require(p.fs_gen != nullptr && p.fs_words != nullptr && p.n_work <= kMaxFusedTiles && !p.mx, "single pass");
  return quant_launch(p, grid, "single pass");
}
hipError_t launch_roof(const QuantParams& p, int64_t grid, hipStream_t) {
  ++g_stub_calls;
  require(p.x && p.row_codes && p.row_scales && p.col_codes && p.col_scales, "roof outputs");
  require(p.rows % kTileRows == 0 && p.cols % kBandCols == 0 && p.padded_rows == p.rows && p.ld == p.cols, "roof shape");
  require(p.n_work == p.n_band * p.n_tiles && grid >= p.n_work && grid % kNumXcd == 0, "roof grid");
  return g_stub_result;
}
hipError_t launch_fill(uint32_t* ptr, int64_t n, uint32_t, hipStream_t) {
  ++g_stub_calls;
  require(ptr != nullptr && n >= 0, "fill");
  return g_stub_result;
}
hipError_t launch_dequant(const DequantParams& p, hipStream_t) {
  ++g_stub_calls;
  require(p.codes && p.scales && p.out && p.rows > 0 && p.cols > 0, "dequant");
  return g_stub_result;
}
hipError_t launch_stats(const StatsParams& p, hipStream_t) {
  ++g_stub_calls;
  require(p.x && p.codes && p.scales && p.part && p.n_wg >= 1, "stats");
  // the partials must not be read back after a failed launch
  return hipErrorNoDevice;
}
hipError_t launch_round(const float* y, int64_t n, int32_t, int32_t, uint64_t, uint8_t* c, hipStream_t) {
  ++g_stub_calls;
  require(y && c && n > 0, "round");
  return g_stub_result;
}
hipError_t launch_gemm(const GemmParams& p, hipStream_t) {
  ++g_stub_calls;
  require(p.M > 0 && p.N > 0 && p.K >= 0 && p.K % 32 == 0 && p.ldc >= p.N && p.c, "gemm");
  require(p.mx == 0 || p.mx == 1, "gemm scaling");
  return g_stub_result;
}
hipError_t launch_to_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t) {
  ++g_stub_calls;
  require(n == 0 || (in && out), "to_bf16");
  return g_stub_result;
}

}  // namespace ufp4
