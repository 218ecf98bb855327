// ufp4_api.hip -- the C ABI (include/ufp4.h): argument checks, workspace
// layout and launches.  Every check runs on the host before anything is
// enqueued; nothing here allocates device memory.
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/ufp4.h"
#include "ufp4_internal.hpp"

using namespace ufp4;

namespace {

constexpr int kStatsMaxWg = 1024;
constexpr int64_t kMaxDim = (int64_t)1 << 25;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_cfg(const ufp4_config* cfg) {
  if (!cfg) return UFP4_ERR_INVALID_ARGUMENT;
  if (cfg->grid < 0 || cfg->grid > 3) return UFP4_ERR_INVALID_ARGUMENT;
  if (cfg->rounding < 0 || cfg->rounding > 1) return UFP4_ERR_INVALID_ARGUMENT;
  if (cfg->scaling < 0 || cfg->scaling > 1) return UFP4_ERR_INVALID_ARGUMENT;
  if (cfg->rht != 0 && cfg->rht != 1) return UFP4_ERR_INVALID_ARGUMENT;
  return UFP4_OK;
}

int block_of(const ufp4_config* cfg) { return cfg->scaling == UFP4_SCALE_MX32 ? 32 : 16; }

size_t quant_ws_bytes(int64_t rows, int64_t cols, int32_t groups) {
  int32_t nb, nt;
  const int64_t g16 = grid_size_quant(rows, cols, groups, 16, &nb, &nt);
  const int64_t g32 = grid_size_quant(rows, cols, groups, 32, &nb, &nt);
  const int64_t g = g16 > g32 ? g16 : g32;
  return kWsPartOffset + (size_t)g * sizeof(float2);
}

// Schedule of dense NV16 calls (ufp4_set_schedule).
std::atomic<int> g_schedule{UFP4_SCHEDULE_AUTO};
std::atomic<int> g_left_stride{0};

size_t stats_ws_bytes() { return kWsPartOffset + (size_t)kStatsMaxWg * kStatsSlots * sizeof(double); }

// Workspace of ufp4_quantize_rowcol_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` only
// names the symbol; its device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)1 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of the scratch array, zeroed (by a fill kernel
// on `stream`) before its first use; null if the runtime call fails.
void* scratch_for_current_device(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    if (launch_fill(static_cast<uint32_t*>(ptr), (int64_t)(kScratchBytes / 4), 0u, stream) != hipSuccess)
      return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// An empty output (no elements) may pass null codes/scales; the tensor
// scale is always written.
int check_qtensor(const ufp4_qtensor& q, bool empty) {
  if (!q.tensor_scale) return UFP4_ERR_INVALID_ARGUMENT;
  if (!empty && (!q.codes || !q.scales)) return UFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(q.codes, 16) || !aligned(q.tensor_scale, 4)) return UFP4_ERR_ALIGNMENT;
  return UFP4_OK;
}

// Common setup of the quantization parameters.
void base_params(QuantParams& p, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                 const ufp4_config* cfg, void* ws) {
  memset(&p, 0, sizeof p);
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld = ld;
  p.num_groups = 1;
  p.block = block_of(cfg);
  p.padded_rows = rows;
  p.rht = cfg->rht;
  p.mx = cfg->scaling == UFP4_SCALE_MX32;
  p.grid = cfg->grid;
  p.sr = cfg->rounding == UFP4_ROUND_STOCHASTIC;
  p.sr_k0 = (uint32_t)cfg->sr_seed;
  p.sr_k1 = (uint32_t)(cfg->sr_seed >> 32);
  fill_rht_signs(cfg->rht_seed, p);
  p.ws_status = ws ? reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + 4) : nullptr;
}

// Workgroups of the single-pass kernels the current device holds at once
// (two per compute unit), 0 if it cannot be queried.
int64_t resident_tiles() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return 2 * (int64_t)cus;
}

// Whether a dense NV16 call of n_work tiles takes the single pass.  AUTO
// takes it for row+column calls whose tiles the device holds at once (on
// MI355X the 8192 x 2048 row+column call takes 26.0 us against 27.9 us in
// two passes, and reads its input once instead of twice); single-layout
// calls keep the two-pass schedule.
bool single_pass(bool grouped, bool mx, bool both, int64_t n_work) {
  if (grouped || mx || n_work > kMaxFusedTiles) return false;
  const int mode = g_schedule.load(std::memory_order_relaxed);
  if (mode == UFP4_SCHEDULE_SINGLE_PASS) return true;
  return mode == UFP4_SCHEDULE_AUTO && both && n_work <= resident_tiles();
}

// Start and end events of the two kernels of one call.
struct KernelTimer {
  hipEvent_t ev[4];
  bool single = false;  // the call ran as one kernel (events 2 and 3 only)
};

int run_quant(QuantParams& p, void* ws, size_t ws_bytes, hipStream_t stream, KernelTimer* tm = nullptr) {
  // per-lane output offsets inside a tile are 32-bit
  if (p.cols >= kMaxDim || p.padded_rows >= kMaxDim) return UFP4_ERR_SHAPE;
  if (p.rows == 0 || p.cols == 0) {
    // nothing to quantize: every per-tensor scale is 1 (a zero tensor)
    if (p.do_row && p.row_ts &&
        launch_fill(reinterpret_cast<uint32_t*>(p.row_ts), p.num_groups, 0x3F800000u, stream) != hipSuccess)
      return UFP4_ERR_HIP;
    if (p.do_col && p.col_ts &&
        launch_fill(reinterpret_cast<uint32_t*>(p.col_ts), p.num_groups, 0x3F800000u, stream) != hipSuccess)
      return UFP4_ERR_HIP;
    return UFP4_OK;
  }
  const int64_t grid = grid_size_quant(p.rows, p.cols, p.num_groups, p.block, &p.n_band, &p.n_tiles);
  p.n_work = p.n_band * p.n_tiles;
  if (grid > 0x7FFFFFFF) return UFP4_ERR_SHAPE;
  if (!p.mx) {
    const size_t need = quant_ws_bytes(p.rows, p.cols, p.num_groups);
    if (!ws || ws_bytes < need || !aligned(ws, 256)) return UFP4_ERR_WORKSPACE;
    p.ws_part = reinterpret_cast<float2*>(static_cast<uint8_t*>(ws) + kWsPartOffset);
    if (single_pass(p.offsets != nullptr, false, p.do_row && p.do_col, p.n_work)) {
      const int mode = g_schedule.load(std::memory_order_relaxed);
      // every tile fits on the device at once: one pass over the input
      uint8_t* base = static_cast<uint8_t*>(ws);
      p.fs_gen = reinterpret_cast<uint32_t*>(base + kWsGenOffset);
      p.fs_words = reinterpret_cast<uint64_t*>(base + kWsHeader);
      p.fs_orphan_stride = mode == UFP4_SCHEDULE_SINGLE_PASS ? g_left_stride.load(std::memory_order_relaxed) : 0;
      if (tm) tm->single = true;  // no separate maxima kernel
      if (launch_fused(p, grid, stream, tm ? tm->ev[2] : nullptr, tm ? tm->ev[3] : nullptr) != hipSuccess)
        return UFP4_ERR_HIP;
      return UFP4_OK;
    }
    if (launch_amax(p, grid, stream, tm ? tm->ev[0] : nullptr, tm ? tm->ev[1] : nullptr) != hipSuccess)
      return UFP4_ERR_HIP;
  } else if (p.offsets) {
    if (!ws || ws_bytes < kWsHeader || !aligned(ws, 256)) return UFP4_ERR_WORKSPACE;
  }
  if (launch_quant(p, grid, stream, tm ? tm->ev[2] : nullptr, tm ? tm->ev[3] : nullptr) != hipSuccess)
    return UFP4_ERR_HIP;
  return UFP4_OK;
}

}  // namespace

extern "C" {

const char* ufp4_status_string(int status) {
  switch (status) {
    case UFP4_OK: return "ok";
    case UFP4_ERR_INVALID_ARGUMENT: return "invalid argument";
    case UFP4_ERR_SHAPE: return "shape is not a multiple of the block";
    case UFP4_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case UFP4_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case UFP4_ERR_HIP: return "HIP runtime error";
    case UFP4_ERR_OFFSETS: return "grouped offsets invalid";
    case UFP4_ERR_SYNC: return "single-pass device-wide exchange did not complete";
    default: return "unknown status";
  }
}

size_t ufp4_workspace_size(int64_t rows, int64_t cols, int32_t num_groups) {
  if (rows < 0 || cols < 0 || num_groups < 1) return 0;
  const size_t a = quant_ws_bytes(rows, cols, num_groups), b = stats_ws_bytes();
  return a > b ? a : b;
}

int ufp4_workspace_init(void* ws, size_t ws_bytes, ufp4_stream_t stream) {
  if (!ws || ws_bytes < kWsHeader || !aligned(ws, 256)) return UFP4_ERR_WORKSPACE;
  if (launch_fill(static_cast<uint32_t*>(ws), (int64_t)(ws_bytes / 4), 0u, (hipStream_t)stream) != hipSuccess)
    return UFP4_ERR_HIP;
  return UFP4_OK;
}

int ufp4_gemm_nt(const ufp4_config* cfg, int64_t M, int64_t N, int64_t K, ufp4_qtensor a, ufp4_qtensor b,
                 float* c, int64_t ldc, ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (M < 0 || N < 0 || K < 0 || ldc < N) return UFP4_ERR_INVALID_ARGUMENT;
  if (K % 32) return UFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return UFP4_OK;
  if (!c || !a.tensor_scale || !b.tensor_scale) return UFP4_ERR_INVALID_ARGUMENT;
  if (K > 0 && (!a.codes || !a.scales || !b.codes || !b.scales)) return UFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(a.codes, 16) || !aligned(b.codes, 16) || !aligned(c, 4) || !aligned(a.tensor_scale, 4) ||
      !aligned(b.tensor_scale, 4))
    return UFP4_ERR_ALIGNMENT;
  // grid: (N / 256) x (M / 256) workgroups of 256 x 256 output tiles
  if ((M + 255) / 256 > 0xFFFF || (N + 255) / 256 > 0x7FFFFFFF) return UFP4_ERR_SHAPE;
  GemmParams p;
  p.a_codes = a.codes;
  p.a_scales = a.scales;
  p.a_ts = a.tensor_scale;
  p.b_codes = b.codes;
  p.b_scales = b.scales;
  p.b_ts = b.tensor_scale;
  p.c = c;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldc = ldc;
  p.grid = cfg->grid;
  p.mx = cfg->scaling == UFP4_SCALE_MX32;
  if (launch_gemm(p, (hipStream_t)stream) != hipSuccess) return UFP4_ERR_HIP;
  return UFP4_OK;
}

int64_t ufp4_amax_tiles(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  int32_t nb, nt;
  grid_size_quant(rows, cols, 1, 16, &nb, &nt);
  return (int64_t)nb * nt;
}

int ufp4_quantize_delayed(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const ufp4_config* cfg,
                          const float* amax_in, int32_t n_in, float* amax_out, ufp4_qtensor row_out,
                          ufp4_qtensor col_out, ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->scaling != UFP4_SCALE_NV16) return UFP4_ERR_INVALID_ARGUMENT;
  if (rows < 0 || cols < 0 || ld < cols || !amax_in || n_in < 1) return UFP4_ERR_INVALID_ARGUMENT;
  const bool do_col = col_out.tensor_scale != nullptr;
  if (cols % 16 || (do_col && rows % 16)) return UFP4_ERR_SHAPE;
  const bool empty = rows == 0 || cols == 0;
  if ((rc = check_qtensor(row_out, empty))) return rc;
  if (do_col && (rc = check_qtensor(col_out, empty))) return rc;
  if (!aligned(amax_in, 8) || !aligned(amax_out, 8)) return UFP4_ERR_ALIGNMENT;
  if (!empty) {
    if (!x) return UFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || ld % 8) return UFP4_ERR_ALIGNMENT;
  }
  const int64_t n_out = ufp4_amax_tiles(rows, cols);
  if (amax_out && n_out > 0) {
    // the kernel reads every provided maximum while it writes its own
    const uintptr_t a0 = (uintptr_t)amax_in, a1 = a0 + (uintptr_t)n_in * 2 * sizeof(float);
    const uintptr_t b0 = (uintptr_t)amax_out, b1 = b0 + (uintptr_t)n_out * 2 * sizeof(float);
    if (a0 < b1 && b0 < a1) return UFP4_ERR_INVALID_ARGUMENT;
  }
  QuantParams p;
  base_params(p, x, rows, cols, ld, cfg, nullptr);
  p.do_row = 1;
  p.do_col = do_col;
  p.row_codes = row_out.codes;
  p.row_scales = row_out.scales;
  p.row_ts = row_out.tensor_scale;
  if (do_col) {
    p.col_codes = col_out.codes;
    p.col_scales = col_out.scales;
    p.col_ts = col_out.tensor_scale;
  }
  hipStream_t s = (hipStream_t)stream;
  if (empty) {
    if (launch_fill(reinterpret_cast<uint32_t*>(p.row_ts), 1, 0x3F800000u, s) != hipSuccess) return UFP4_ERR_HIP;
    if (do_col && launch_fill(reinterpret_cast<uint32_t*>(p.col_ts), 1, 0x3F800000u, s) != hipSuccess)
      return UFP4_ERR_HIP;
    return UFP4_OK;
  }
  if (cols >= kMaxDim || rows >= kMaxDim) return UFP4_ERR_SHAPE;
  const int64_t grid = grid_size_quant(rows, cols, 1, 16, &p.n_band, &p.n_tiles);
  p.n_work = p.n_band * p.n_tiles;
  if (grid > 0x7FFFFFFF) return UFP4_ERR_SHAPE;
  p.amax_in = reinterpret_cast<const float2*>(amax_in);
  p.n_in = n_in;
  p.amax_out = reinterpret_cast<float2*>(amax_out);
  if (launch_delayed(p, grid, s) != hipSuccess) return UFP4_ERR_HIP;
  return UFP4_OK;
}

int ufp4_schedule_of(int64_t rows, int64_t cols, int32_t num_groups, int32_t both_layouts, const ufp4_config* cfg,
                     int32_t* schedule_out) {
  if (check_cfg(cfg) || !schedule_out || rows < 0 || cols < 0 || num_groups < 1)
    return UFP4_ERR_INVALID_ARGUMENT;
  int32_t nb, nt;
  grid_size_quant(rows, cols, num_groups, block_of(cfg), &nb, &nt);
  const bool one = rows > 0 && cols > 0 &&
                   single_pass(num_groups > 1, cfg->scaling == UFP4_SCALE_MX32, both_layouts != 0, (int64_t)nb * nt);
  *schedule_out = one ? UFP4_SCHEDULE_SINGLE_PASS : UFP4_SCHEDULE_TWO_PASS;
  return UFP4_OK;
}

int ufp4_set_schedule(int32_t schedule, int32_t left_stride) {
  if (schedule < UFP4_SCHEDULE_AUTO || schedule > UFP4_SCHEDULE_SINGLE_PASS || left_stride < 0)
    return UFP4_ERR_INVALID_ARGUMENT;
  g_left_stride.store(left_stride, std::memory_order_relaxed);
  g_schedule.store(schedule, std::memory_order_relaxed);
  return UFP4_OK;
}

int ufp4_workspace_status(const void* ws, size_t ws_bytes, int* status_out, ufp4_stream_t stream) {
  if (!ws || ws_bytes < kWsHeader || !status_out) return UFP4_ERR_INVALID_ARGUMENT;
  uint32_t st = 0;
  if (hipMemcpyAsync(&st, static_cast<const uint8_t*>(ws) + 4, 4, hipMemcpyDeviceToHost,
                     (hipStream_t)stream) != hipSuccess)
    return UFP4_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return UFP4_ERR_HIP;
  // the device writes 0, UFP4_ERR_OFFSETS (grouped offsets rejected) or
  // UFP4_ERR_SYNC (a single-pass exchange that did not complete); any other
  // word means the workspace was never initialized or was overwritten
  *status_out = (st == 0u || st == (uint32_t)UFP4_ERR_OFFSETS || st == (uint32_t)UFP4_ERR_SYNC) ? (int)st
                                                                                             : UFP4_ERR_WORKSPACE;
  return UFP4_OK;
}

int ufp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const ufp4_config* cfg,
                  ufp4_qtensor row_out, void* ws, size_t ws_bytes, ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (rows < 0 || cols < 0 || ld < cols) return UFP4_ERR_INVALID_ARGUMENT;
  if (cols % block_of(cfg)) return UFP4_ERR_SHAPE;
  if ((rc = check_qtensor(row_out, rows == 0 || cols == 0))) return rc;
  if (rows > 0 && cols > 0) {
    if (!x) return UFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || ld % 8) return UFP4_ERR_ALIGNMENT;
  }
  QuantParams p;
  base_params(p, x, rows, cols, ld, cfg, ws);
  p.do_row = 1;
  p.row_codes = row_out.codes;
  p.row_scales = row_out.scales;
  p.row_ts = row_out.tensor_scale;
  if (rows == 0 || cols == 0) cols = rows = 0;
  p.rows = rows;
  p.cols = cols;
  return run_quant(p, ws, ws_bytes, (hipStream_t)stream);
}

static int rowcol_impl(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const ufp4_config* cfg,
                       ufp4_qtensor row_out, ufp4_qtensor col_out, void* ws, size_t ws_bytes,
                       ufp4_stream_t stream, KernelTimer* tm) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (rows < 0 || cols < 0 || ld < cols) return UFP4_ERR_INVALID_ARGUMENT;
  const int B = block_of(cfg);
  if (cols % B || rows % B) return UFP4_ERR_SHAPE;
  if ((rc = check_qtensor(row_out, rows == 0 || cols == 0))) return rc;
  if ((rc = check_qtensor(col_out, rows == 0 || cols == 0))) return rc;
  if (rows > 0 && cols > 0) {
    if (!x) return UFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || ld % 8) return UFP4_ERR_ALIGNMENT;
  }
  QuantParams p;
  base_params(p, x, rows, cols, ld, cfg, ws);
  p.do_row = 1;
  p.do_col = 1;
  p.row_codes = row_out.codes;
  p.row_scales = row_out.scales;
  p.row_ts = row_out.tensor_scale;
  p.col_codes = col_out.codes;
  p.col_scales = col_out.scales;
  p.col_ts = col_out.tensor_scale;
  if (rows == 0 || cols == 0) p.rows = p.cols = 0;
  p.padded_rows = p.rows;
  return run_quant(p, ws, ws_bytes, (hipStream_t)stream, tm);
}

int ufp4_quantize_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                         const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out, void* ws,
                         size_t ws_bytes, ufp4_stream_t stream) {
  return rowcol_impl(x, rows, cols, ld, cfg, row_out, col_out, ws, ws_bytes, stream, nullptr);
}

int ufp4_quantize_rowcol_noalloc(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                 const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out,
                                 ufp4_stream_t stream) {
  // the same argument checks as the workspace variant come first (it reports
  // them before looking at the workspace)
  const int rc = check_cfg(cfg);
  if (rc) return rc;
  if (rows < 0 || cols < 0 || ld < cols) return UFP4_ERR_INVALID_ARGUMENT;
  if (quant_ws_bytes(rows, cols, 1) > kScratchBytes) return UFP4_ERR_WORKSPACE;
  void* ws = scratch_for_current_device((hipStream_t)stream);
  if (!ws) return UFP4_ERR_HIP;
  return rowcol_impl(x, rows, cols, ld, cfg, row_out, col_out, ws, kScratchBytes, stream, nullptr);
}

int ufp4_time_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const ufp4_config* cfg,
                     ufp4_qtensor row_out, ufp4_qtensor col_out, void* ws, size_t ws_bytes,
                     ufp4_stream_t stream, float* ms_amax_host, float* ms_quant_host) {
  if (!ms_amax_host || !ms_quant_host || !cfg || cfg->scaling != UFP4_SCALE_NV16 || rows <= 0 || cols <= 0)
    return UFP4_ERR_INVALID_ARGUMENT;
  KernelTimer tm;
  int made = 0, rc = UFP4_OK;
  for (; made < 4; ++made)
    if (hipEventCreate(&tm.ev[made]) != hipSuccess) {
      rc = UFP4_ERR_HIP;
      break;
    }
  if (rc == UFP4_OK) rc = rowcol_impl(x, rows, cols, ld, cfg, row_out, col_out, ws, ws_bytes, stream, &tm);
  if (rc == UFP4_OK) {
    *ms_amax_host = 0.0f;
    if (hipEventSynchronize(tm.ev[3]) != hipSuccess ||
        (!tm.single && hipEventElapsedTime(ms_amax_host, tm.ev[0], tm.ev[1]) != hipSuccess) ||
        hipEventElapsedTime(ms_quant_host, tm.ev[2], tm.ev[3]) != hipSuccess)
      rc = UFP4_ERR_HIP;
  }
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(tm.ev[i]);
  return rc;
}

int ufp4_roof_rowcol(const uint16_t* x, int64_t rows, int64_t cols, ufp4_qtensor row_out, ufp4_qtensor col_out,
                     ufp4_stream_t stream) {
  if (!x || !row_out.codes || !row_out.scales || !col_out.codes || !col_out.scales) return UFP4_ERR_INVALID_ARGUMENT;
  if (rows <= 0 || cols <= 0 || rows % kTileRows || cols % kBandCols || rows >= kMaxDim || cols >= kMaxDim)
    return UFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(row_out.codes, 16) || !aligned(row_out.scales, 16) ||
      !aligned(col_out.codes, 16) || !aligned(col_out.scales, 8))
    return UFP4_ERR_ALIGNMENT;
  QuantParams p = {};
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld = cols;
  p.num_groups = 1;
  p.block = 16;
  p.padded_rows = rows;
  p.row_codes = row_out.codes;
  p.row_scales = row_out.scales;
  p.col_codes = col_out.codes;
  p.col_scales = col_out.scales;
  const int64_t grid = grid_size_quant(rows, cols, 1, 16, &p.n_band, &p.n_tiles);
  p.n_work = p.n_band * p.n_tiles;
  if (grid > 0x7FFFFFFF) return UFP4_ERR_SHAPE;
  return launch_roof(p, grid, (hipStream_t)stream) == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
}

int ufp4_quantize_grouped(const uint16_t* x, int64_t total_rows, int64_t cols,
                          const int64_t* offsets_dev, int32_t num_groups, int64_t padded_rows,
                          const ufp4_config* cfg, ufp4_qtensor row_out, ufp4_qtensor col_out, void* ws,
                          size_t ws_bytes, ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (total_rows < 0 || cols < 0 || num_groups < 1 || num_groups > kMaxGroups) return UFP4_ERR_INVALID_ARGUMENT;
  if (!offsets_dev) return UFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(offsets_dev, 8)) return UFP4_ERR_ALIGNMENT;
  const int B = block_of(cfg);
  if (cols % B) return UFP4_ERR_SHAPE;
  const bool do_row = row_out.tensor_scale != nullptr, do_col = col_out.tensor_scale != nullptr;
  if (!do_row && !do_col) return UFP4_ERR_INVALID_ARGUMENT;
  const bool empty = total_rows == 0 || cols == 0;
  if (do_row && (rc = check_qtensor(row_out, empty))) return rc;
  if (do_col) {
    if ((rc = check_qtensor(col_out, empty))) return rc;
    if (padded_rows < total_rows || padded_rows % B ||
        padded_rows > total_rows + (int64_t)(B - 1) * num_groups)
      return UFP4_ERR_SHAPE;
  }
  if (total_rows > 0 && cols > 0) {
    if (!x) return UFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || cols % 8) return UFP4_ERR_ALIGNMENT;
  }
  QuantParams p;
  base_params(p, x, total_rows, cols, cols, cfg, ws);
  p.offsets = offsets_dev;
  p.num_groups = num_groups;
  p.padded_rows = do_col ? padded_rows : 0;
  p.do_row = do_row;
  p.do_col = do_col;
  p.row_codes = row_out.codes;
  p.row_scales = row_out.scales;
  p.row_ts = row_out.tensor_scale;
  p.col_codes = col_out.codes;
  p.col_scales = col_out.scales;
  p.col_ts = col_out.tensor_scale;
  return run_quant(p, ws, ws_bytes, (hipStream_t)stream);
}

int ufp4_quantize_grouped_delayed(const uint16_t* x, int64_t total_rows, int64_t cols,
                                  const int64_t* offsets_dev, int32_t num_groups, int64_t padded_rows,
                                  const ufp4_config* cfg, const float* amax_in, float* amax_out,
                                  ufp4_qtensor row_out, ufp4_qtensor col_out, void* ws, size_t ws_bytes,
                                  ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->scaling != UFP4_SCALE_NV16) return UFP4_ERR_INVALID_ARGUMENT;
  if (total_rows < 0 || cols < 0 || num_groups < 1 || num_groups > kMaxGroups || !amax_in)
    return UFP4_ERR_INVALID_ARGUMENT;
  if (!offsets_dev) return UFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(offsets_dev, 8) || !aligned(amax_in, 8) || !aligned(amax_out, 8)) return UFP4_ERR_ALIGNMENT;
  if (cols % 16) return UFP4_ERR_SHAPE;
  const bool do_row = row_out.tensor_scale != nullptr, do_col = col_out.tensor_scale != nullptr;
  if (!do_row && !do_col) return UFP4_ERR_INVALID_ARGUMENT;
  if (amax_out) {
    // the kernel reads the provided maxima while it folds in its own
    const uintptr_t a0 = (uintptr_t)amax_in, a1 = a0 + (uintptr_t)num_groups * 2 * sizeof(float);
    const uintptr_t b0 = (uintptr_t)amax_out, b1 = b0 + (uintptr_t)num_groups * 2 * sizeof(float);
    if (a0 < b1 && b0 < a1) return UFP4_ERR_INVALID_ARGUMENT;
  }
  const bool empty = total_rows == 0 || cols == 0;
  if (do_row && (rc = check_qtensor(row_out, empty))) return rc;
  if (do_col) {
    if ((rc = check_qtensor(col_out, empty))) return rc;
    if (padded_rows < total_rows || padded_rows % 16 || padded_rows > total_rows + 15 * (int64_t)num_groups)
      return UFP4_ERR_SHAPE;
  }
  if (!empty) {
    if (!x) return UFP4_ERR_INVALID_ARGUMENT;
    if (!aligned(x, 16) || cols % 8) return UFP4_ERR_ALIGNMENT;
  }
  if (!ws || ws_bytes < kWsHeader || !aligned(ws, 256)) return UFP4_ERR_WORKSPACE;
  QuantParams p;
  base_params(p, x, total_rows, cols, cols, cfg, ws);
  p.offsets = offsets_dev;
  p.num_groups = num_groups;
  p.padded_rows = do_col ? padded_rows : 0;
  p.do_row = do_row;
  p.do_col = do_col;
  p.row_codes = row_out.codes;
  p.row_scales = row_out.scales;
  p.row_ts = row_out.tensor_scale;
  p.col_codes = col_out.codes;
  p.col_scales = col_out.scales;
  p.col_ts = col_out.tensor_scale;
  p.amax_in = reinterpret_cast<const float2*>(amax_in);
  p.n_in = num_groups;
  p.amax_out = reinterpret_cast<float2*>(amax_out);
  hipStream_t s = (hipStream_t)stream;
  // this call's maxima are folded into zeroed entries (empty segments stay 0)
  if (amax_out && launch_fill(reinterpret_cast<uint32_t*>(amax_out), 2 * (int64_t)num_groups, 0u, s) != hipSuccess)
    return UFP4_ERR_HIP;
  if (empty) {
    if (do_row && launch_fill(reinterpret_cast<uint32_t*>(p.row_ts), num_groups, 0x3F800000u, s) != hipSuccess)
      return UFP4_ERR_HIP;
    if (do_col && launch_fill(reinterpret_cast<uint32_t*>(p.col_ts), num_groups, 0x3F800000u, s) != hipSuccess)
      return UFP4_ERR_HIP;
    return UFP4_OK;
  }
  if (p.cols >= kMaxDim || p.padded_rows >= kMaxDim) return UFP4_ERR_SHAPE;
  const int64_t grid = grid_size_quant(total_rows, cols, num_groups, 16, &p.n_band, &p.n_tiles);
  p.n_work = p.n_band * p.n_tiles;
  if (grid > 0x7FFFFFFF) return UFP4_ERR_SHAPE;
  if (launch_grouped_delayed(p, grid, s) != hipSuccess) return UFP4_ERR_HIP;
  return UFP4_OK;
}

int ufp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t rows,
                    int64_t cols, const ufp4_config* cfg, int32_t inverse_rht, float* out,
                    ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (rows < 0 || cols < 0) return UFP4_ERR_INVALID_ARGUMENT;
  if (cols % block_of(cfg)) return UFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return UFP4_OK;
  if (!codes || !scales || !out || (!tensor_scale && cfg->scaling == UFP4_SCALE_NV16))
    return UFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(codes, 8) || !aligned(out, 16)) return UFP4_ERR_ALIGNMENT;
  DequantParams p;
  memset(&p, 0, sizeof p);
  p.codes = codes;
  p.scales = scales;
  p.ts = tensor_scale;
  p.rows = rows;
  p.cols = cols;
  p.grid = cfg->grid;
  p.mx = cfg->scaling == UFP4_SCALE_MX32;
  p.inverse = inverse_rht ? 1 : 0;
  const uint32_t mask = rht_sign_mask(cfg->rht_seed);
  for (int j = 0; j < 16; ++j) p.d[j] = ((mask >> j) & 1u) ? -1.0f : 1.0f;
  p.out = out;
  return launch_dequant(p, (hipStream_t)stream) == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
}

int ufp4_stats(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int32_t layout,
               const ufp4_config* cfg, const uint8_t* codes, const uint8_t* scales,
               const float* tensor_scale, void* ws, size_t ws_bytes, ufp4_stats_t* host_out,
               ufp4_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!host_out || rows < 0 || cols < 0 || ld < cols || (layout != 0 && layout != 1))
    return UFP4_ERR_INVALID_ARGUMENT;
  const int B = block_of(cfg);
  if ((layout == 0 ? cols : rows) % B) return UFP4_ERR_SHAPE;
  if (!ws || ws_bytes < stats_ws_bytes() || !aligned(ws, 256)) return UFP4_ERR_WORKSPACE;
  memset(host_out, 0, sizeof *host_out);
  const int64_t nblk = rows * cols / B;
  if (nblk == 0) {
    host_out->sqnr_db = __builtin_inf();
    host_out->alpha = 1.0;
    return UFP4_OK;
  }
  if (!x || !codes || !scales || (!tensor_scale && cfg->scaling == UFP4_SCALE_NV16))
    return UFP4_ERR_INVALID_ARGUMENT;
  StatsParams p;
  memset(&p, 0, sizeof p);
  p.x = x;
  p.rows = rows;
  p.cols = cols;
  p.ld = ld;
  p.layout = layout;
  p.grid = cfg->grid;
  p.mx = cfg->scaling == UFP4_SCALE_MX32;
  p.rht = cfg->rht;
  QuantParams tmp;
  memset(&tmp, 0, sizeof tmp);
  fill_rht_signs(cfg->rht_seed, tmp);
  p.sg = tmp.sg;
  p.codes = codes;
  p.scales = scales;
  p.ts = tensor_scale;
  int64_t wg = (nblk + 255) / 256;
  if (wg > kStatsMaxWg) wg = kStatsMaxWg;
  p.n_wg = (int32_t)wg;
  p.part = reinterpret_cast<double*>(static_cast<uint8_t*>(ws) + kWsPartOffset);
  hipStream_t s = (hipStream_t)stream;
  if (launch_stats(p, s) != hipSuccess) return UFP4_ERR_HIP;
  static thread_local double host[kStatsMaxWg * kStatsSlots];
  if (hipMemcpyAsync(host, p.part, (size_t)wg * kStatsSlots * sizeof(double), hipMemcpyDeviceToHost, s) !=
      hipSuccess)
    return UFP4_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return UFP4_ERR_HIP;
  double v2 = 0, e2 = 0, vx = 0, se = 0, seg = 0, amax = 0;
  double n = 0, n_grid = 0, n_zero = 0, n_sat = 0, n_nf = 0;
  double hist[16] = {0};
  for (int64_t i = 0; i < wg; ++i) {
    const double* q = host + i * kStatsSlots;
    v2 += q[0]; e2 += q[1]; vx += q[2]; se += q[3]; seg += q[4];
    amax = q[5] > amax ? q[5] : amax;
    n += q[6]; n_grid += q[7]; n_zero += q[8]; n_sat += q[9]; n_nf += q[10];
    for (int c = 0; c < 16; ++c) hist[c] += q[11 + c];
  }
  host_out->n = (uint64_t)n;
  for (int c = 0; c < 16; ++c) host_out->code_hist[c] = (uint64_t)hist[c];
  host_out->n_saturated = (uint64_t)n_sat;
  host_out->n_nonfinite = (uint64_t)n_nf;
  host_out->n_zero_scale = (uint64_t)n_zero;
  host_out->amax = amax;
  host_out->sqnr_db = e2 > 0 ? 10.0 * __builtin_log10(v2 / e2) : __builtin_inf();
  host_out->mean_signed_err = n > 0 ? se / n : 0.0;
  host_out->mean_signed_err_grid = n_grid > 0 ? seg / n_grid : 0.0;
  host_out->alpha = v2 > 0 ? vx / v2 : 1.0;
  return UFP4_OK;
}

int ufp4_round_f32(const float* y_dev, int64_t n, int32_t grid, int32_t rounding, uint64_t sr_seed,
                   uint8_t* codes_dev, ufp4_stream_t stream) {
  if (n < 0 || grid < 0 || grid > 3 || rounding < 0 || rounding > 1) return UFP4_ERR_INVALID_ARGUMENT;
  if (n == 0) return UFP4_OK;
  if (!y_dev || !codes_dev) return UFP4_ERR_INVALID_ARGUMENT;
  if (!aligned(y_dev, 4)) return UFP4_ERR_ALIGNMENT;
  return launch_round(y_dev, n, grid, rounding, sr_seed, codes_dev, (hipStream_t)stream) == hipSuccess
             ? UFP4_OK
             : UFP4_ERR_HIP;
}

int ufp4_recipe_config(int32_t recipe, int32_t gemm, int32_t operand, uint64_t rht_seed, uint64_t sr_seed,
                       ufp4_config* cfg_out, int32_t* layout_out, int32_t* tensor_out) {
  if (!cfg_out || !layout_out || !tensor_out) return UFP4_ERR_INVALID_ARGUMENT;
  if (recipe < UFP4_RECIPE_UFP4 || recipe > UFP4_RECIPE_NVFP4 || gemm < UFP4_GEMM_FWD_Y ||
      gemm > UFP4_GEMM_BWD_DW || (operand != UFP4_OPERAND_A && operand != UFP4_OPERAND_B))
    return UFP4_ERR_INVALID_ARGUMENT;
  // operand tensors and layouts: the reduction dimension of each product
  // runs along the quantization blocks
  static const int32_t kTensor[3][2] = {{UFP4_TENSOR_X, UFP4_TENSOR_W},
                                        {UFP4_TENSOR_DY, UFP4_TENSOR_W},
                                        {UFP4_TENSOR_DY, UFP4_TENSOR_X}};
  static const int32_t kLayout[3][2] = {{0, 0}, {0, 1}, {1, 1}};
  const int32_t tensor = kTensor[gemm][operand];
  ufp4_config c;
  c.grid = recipe == UFP4_RECIPE_UFP4 ? UFP4_GRID_E1M2 : recipe == UFP4_RECIPE_UFP4_INT4 ? UFP4_GRID_INT4
                                                                                          : UFP4_GRID_E2M1;
  c.scaling = UFP4_SCALE_NV16;
  c.rht = recipe == UFP4_RECIPE_NVFP4 ? (gemm == UFP4_GEMM_BWD_DW ? 1 : 0) : 1;
  c.rounding = tensor == UFP4_TENSOR_DY ? UFP4_ROUND_STOCHASTIC : UFP4_ROUND_RTNE;
  c.rht_seed = rht_seed;
  c.sr_seed = c.rounding == UFP4_ROUND_STOCHASTIC ? sr_seed : 0u;
  *cfg_out = c;
  *layout_out = kLayout[gemm][operand];
  *tensor_out = tensor;
  return UFP4_OK;
}

int ufp4_f32_to_bf16(const float* in_dev, int64_t n, uint16_t* out_dev, ufp4_stream_t stream) {
  if (n < 0 || (n > 0 && (!in_dev || !out_dev))) return UFP4_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)in_dev % 4 || (uintptr_t)out_dev % 2) return UFP4_ERR_ALIGNMENT;
  return launch_to_bf16(in_dev, n, out_dev, (hipStream_t)stream) == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
}

int ufp4_rht_signs(uint64_t rht_seed, int8_t signs_host[16]) {
  if (!signs_host) return UFP4_ERR_INVALID_ARGUMENT;
  const uint32_t mask = rht_sign_mask(rht_seed);
  for (int j = 0; j < 16; ++j) signs_host[j] = ((mask >> j) & 1u) ? (int8_t)-1 : (int8_t)1;
  return UFP4_OK;
}

int ufp4_grouped_col_offsets(const int64_t* offsets_host, int32_t num_groups, int32_t block,
                             int64_t* col_offsets_host) {
  if (!offsets_host || !col_offsets_host || num_groups < 1 || (block != 16 && block != 32))
    return UFP4_ERR_INVALID_ARGUMENT;
  if (offsets_host[0] != 0) return UFP4_ERR_INVALID_ARGUMENT;
  col_offsets_host[0] = 0;
  for (int32_t e = 0; e < num_groups; ++e) {
    const int64_t m = offsets_host[e + 1] - offsets_host[e];
    if (m < 0) return UFP4_ERR_INVALID_ARGUMENT;
    col_offsets_host[e + 1] = col_offsets_host[e] + (m + block - 1) / block * block;
  }
  return UFP4_OK;
}

}  // extern "C"
