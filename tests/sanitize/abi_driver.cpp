// abi_driver.cpp -- runs the host side of every C-ABI entry point under the
// address and undefined-behaviour sanitizers, with the kernel launchers
// replaced by the checking stubs of launch_stubs.cpp.  Device pointers are
// addresses inside an inaccessible (PROT_NONE) mapping: the host code may do
// arithmetic on them but any host read or write through one crashes the run.
// Exit status 0 when every call returned the expected status.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/mman.h>

#include "../../include/ufp4.h"

namespace ufp4 {
extern int g_stub_calls;
}

static int g_fail = 0;
static uint8_t* g_dev = nullptr;

#define EXPECT(call, want)                                                                     \
  do {                                                                                         \
    const int got_ = (call);                                                                   \
    if (got_ != (want)) {                                                                      \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, \
              (int)(want));                                                                    \
      ++g_fail;                                                                                \
    }                                                                                          \
  } while (0)

template <typename T>
static T* dev(size_t off) {
  return reinterpret_cast<T*>(g_dev + off);
}

static ufp4_config cfg(int grid, int rnd, int scl, int rht) {
  ufp4_config c;
  c.grid = grid;
  c.rounding = rnd;
  c.scaling = scl;
  c.rht = rht;
  c.rht_seed = 1;
  c.sr_seed = 2;
  return c;
}

static ufp4_qtensor qt(size_t codes, size_t scales, size_t ts) {
  ufp4_qtensor q;
  q.codes = codes ? dev<uint8_t>(codes) : nullptr;
  q.scales = scales ? dev<uint8_t>(scales) : nullptr;
  q.tensor_scale = ts ? dev<float>(ts) : nullptr;
  return q;
}

int main() {
  const size_t kSpan = (size_t)1 << 34;
  void* m = mmap(nullptr, kSpan, PROT_NONE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
  if (m == MAP_FAILED) return 2;
  g_dev = static_cast<uint8_t*>(m);
  const uint16_t* x = dev<uint16_t>(1 << 20);
  void* ws = dev<void>(1 << 30);
  const size_t wsb = ufp4_workspace_size(8192, 2048, 1);
  const ufp4_qtensor row = qt((size_t)2 << 30, (size_t)3 << 30, (size_t)4 << 30), col = qt((size_t)5 << 30, (size_t)6 << 30, (size_t)7 << 30);
  const ufp4_qtensor none = qt(0, 0, 0);
  const ufp4_config ok = cfg(0, 0, 0, 1), mx = cfg(0, 0, 1, 1), sr = cfg(0, 1, 0, 1);

  // status strings and sizes
  for (int s = -1; s < 10; ++s) EXPECT(ufp4_status_string(s) != nullptr, 1);
  EXPECT(ufp4_workspace_size(-1, 16, 1) == 0, 1);
  EXPECT(ufp4_workspace_size(16, 16, 0) == 0, 1);
  EXPECT(wsb >= 256, 1);
  EXPECT(ufp4_amax_tiles(0, 16) == 0, 1);
  EXPECT(ufp4_amax_tiles(8192, 2048) == 512, 1);
  EXPECT(ufp4_workspace_init(nullptr, 1024, nullptr), UFP4_ERR_WORKSPACE);
  EXPECT(ufp4_workspace_init(dev<uint8_t>(1 << 30) + 8, 1024, nullptr), UFP4_ERR_WORKSPACE);
  EXPECT(ufp4_workspace_init(ws, wsb, nullptr), UFP4_OK);
  int st = 0;
  EXPECT(ufp4_workspace_status(nullptr, wsb, &st, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_workspace_status(ws, wsb, nullptr, nullptr), UFP4_ERR_INVALID_ARGUMENT);

  // ufp4_quantize
  ufp4_config bad = ok;
  bad.grid = 9;
  EXPECT(ufp4_quantize(x, 64, 64, 64, nullptr, row, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize(x, 64, 64, 64, &bad, row, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize(x, -1, 64, 64, &ok, row, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize(x, 64, 64, 32, &ok, row, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize(x, 64, 72, 72, &ok, row, ws, wsb, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_quantize(x, 64, 48, 48, &mx, row, ws, wsb, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_quantize(x, 64, 64, 64, &ok, none, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize(x, 64, 64, 64, &ok, qt(((size_t)2 << 30) + 1, (size_t)3 << 30, (size_t)4 << 30), ws, wsb, nullptr),
         UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_quantize(x + 1, 64, 64, 64, &ok, row, ws, wsb, nullptr), UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_quantize(x, 64, 64, 68, &ok, row, ws, wsb, nullptr), UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_quantize(nullptr, 64, 64, 64, &ok, row, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize(x, 64, 64, 64, &ok, row, nullptr, 0, nullptr), UFP4_ERR_WORKSPACE);
  EXPECT(ufp4_quantize(x, 8192, 2048, 2048, &ok, row, ws, 300, nullptr), UFP4_ERR_WORKSPACE);
  EXPECT(ufp4_quantize(x, (int64_t)1 << 25, 16, 16, &ok, row, ws, (size_t)1 << 30, nullptr), UFP4_ERR_SHAPE);
  int before = ufp4::g_stub_calls;
  EXPECT(ufp4_quantize(x, 8192, 2048, 2048, &ok, row, ws, wsb, nullptr), UFP4_OK);
  EXPECT(ufp4::g_stub_calls > before, 1);
  EXPECT(ufp4_quantize(x, 1000, 2048, 4096, &sr, row, ws, wsb, nullptr), UFP4_OK);
  EXPECT(ufp4_quantize(x, 1000, 2048, 2048, &mx, row, nullptr, 0, nullptr), UFP4_OK);  // MX32: no workspace
  EXPECT(ufp4_quantize(nullptr, 0, 64, 64, &ok, qt(0, 0, (size_t)4 << 30), nullptr, 0, nullptr), UFP4_OK);

  // ufp4_quantize_rowcol and the single-pass schedule
  EXPECT(ufp4_quantize_rowcol(x, 8200, 2048, 2048, &ok, row, col, ws, wsb, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_quantize_rowcol(x, 8192, 2048, 2048, &ok, row, none, ws, wsb, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_rowcol(x, 8192, 2048, 2048, &ok, row, col, ws, wsb, nullptr), UFP4_OK);
  for (int sched = 0; sched <= 2; ++sched) {
    EXPECT(ufp4_set_schedule(sched, sched == 2 ? 3 : 0), UFP4_OK);
    int32_t which = -1;
    EXPECT(ufp4_schedule_of(8192, 2048, 1, 0, &ok, &which), UFP4_OK);
    EXPECT(which == (sched == 2 ? 2 : 1), 1);  // one layout: two passes unless forced
    EXPECT(ufp4_schedule_of(8192, 2048, 1, 1, &ok, &which), UFP4_OK);
    EXPECT(which == 1 || which == 2, 1);  // AUTO: single pass if the device (none here) holds every tile
    EXPECT(ufp4_quantize_rowcol(x, 8192, 2048, 2048, &ok, row, col, ws, wsb, nullptr), UFP4_OK);
    EXPECT(ufp4_quantize_rowcol(x, 65536, 4096, 4096, &ok, row, col, ws, ufp4_workspace_size(65536, 4096, 1),
                                nullptr),
           UFP4_OK);  // too many tiles for one pass: two passes
  }
  EXPECT(ufp4_set_schedule(3, 0), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_set_schedule(0, -1), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_set_schedule(0, 0), UFP4_OK);
  int32_t which = 0;
  EXPECT(ufp4_schedule_of(16, 16, 1, 1, nullptr, &which), UFP4_ERR_INVALID_ARGUMENT);
  float ta = 0, tq = 0;
  EXPECT(ufp4_time_rowcol(x, 8192, 2048, 2048, &mx, row, col, ws, wsb, nullptr, &ta, &tq), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_time_rowcol(x, 8192, 2048, 2048, &ok, row, col, ws, wsb, nullptr, nullptr, &tq),
         UFP4_ERR_INVALID_ARGUMENT);

  // bandwidth roof hook: full tiles only
  EXPECT(ufp4_roof_rowcol(x, 8192, 2048, row, col, nullptr), UFP4_OK);
  EXPECT(ufp4_roof_rowcol(x, 8192 + 16, 2048, row, col, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_roof_rowcol(x, 8192, 2048 + 16, row, col, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_roof_rowcol(x, 0, 2048, row, col, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_roof_rowcol(nullptr, 8192, 2048, row, col, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_roof_rowcol(x + 1, 8192, 2048, row, col, nullptr), UFP4_ERR_ALIGNMENT);

  // the no-allocation variant: argument errors first, then the size limit;
  // a valid call needs the device's scratch array, which a GPU-less run
  // cannot look up (UFP4_ERR_HIP), or runs to the stubbed launches
  EXPECT(ufp4_quantize_rowcol_noalloc(x, 64, 64, 64, nullptr, row, col, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_rowcol_noalloc(x, 64, 64, 32, &ok, row, col, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_rowcol_noalloc(x, (int64_t)1 << 24, 16384, 16384, &ok, row, col, nullptr),
         UFP4_ERR_WORKSPACE);
  {
    const int r = ufp4_quantize_rowcol_noalloc(x, 8192, 2048, 2048, &ok, row, col, nullptr);
    EXPECT(r == UFP4_ERR_HIP || r == UFP4_OK, 1);
  }

  // ufp4_quantize_grouped
  const int64_t* off = dev<int64_t>((size_t)8 << 30);
  const size_t gwsb = ufp4_workspace_size(65536, 4096, 64);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 0, 65536, &ok, row, col, ws, gwsb, nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 1025, 65536, &ok, row, col, ws, gwsb, nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, nullptr, 64, 65536, &ok, row, col, ws, gwsb, nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off + 0, 64, 65536, &ok, none, none, ws, gwsb, nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, reinterpret_cast<const int64_t*>(g_dev + ((size_t)8 << 30) + 4), 64,
                               65536, &ok, row, col, ws, gwsb, nullptr),
         UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 65530, &ok, row, col, ws, gwsb, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 65536 + 16 * 64, &ok, row, col, ws, gwsb, nullptr),
         UFP4_ERR_SHAPE);
  // within the host's bounds; the device checks it against the offsets
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 65536 + 15 * 64, &ok, row, col, ws, gwsb, nullptr),
         UFP4_OK);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 65536 + 16 * 60, &ok, row, col, ws, gwsb, nullptr),
         UFP4_OK);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 0, &ok, row, none, ws, gwsb, nullptr), UFP4_OK);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 65536, &ok, none, col, ws, 64, nullptr), UFP4_ERR_WORKSPACE);
  EXPECT(ufp4_quantize_grouped(x, 65536, 4096, off, 64, 65536, &mx, row, col, ws, 256, nullptr), UFP4_OK);

  // grouped delayed scaling
  {
    const float* gin = dev<float>((size_t)12 << 30);
    float* gout = dev<float>((size_t)13 << 30);
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 65536, &mx, gin, gout, row, col, ws, gwsb, nullptr),
           UFP4_ERR_INVALID_ARGUMENT);
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 65536, &ok, nullptr, gout, row, col, ws, gwsb,
                                         nullptr),
           UFP4_ERR_INVALID_ARGUMENT);
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 65536, &ok, gin, const_cast<float*>(gin) + 2, row,
                                         col, ws, gwsb, nullptr),
           UFP4_ERR_INVALID_ARGUMENT);  // overlapping maxima
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 65536, &ok, gin + 1, gout, row, col, ws, gwsb,
                                         nullptr),
           UFP4_ERR_ALIGNMENT);
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 65536, &ok, gin, gout, row, col, nullptr, 0, nullptr),
           UFP4_ERR_WORKSPACE);
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 65536 + 16 * 60, &ok, gin, gout, row, col, ws, 256,
                                         nullptr),
           UFP4_OK);
    EXPECT(ufp4_quantize_grouped_delayed(x, 65536, 4096, off, 64, 0, &sr, gin, nullptr, row, none, ws, 256, nullptr),
           UFP4_OK);
    EXPECT(ufp4_quantize_grouped_delayed(nullptr, 0, 4096, off, 64, 0, &ok, gin, gout, row, col, ws, 256, nullptr),
           UFP4_OK);
  }

  // ufp4_dequantize and ufp4_stats
  EXPECT(ufp4_dequantize(row.codes, row.scales, row.tensor_scale, 64, 72, &ok, 1, dev<float>((size_t)9 << 30), nullptr),
         UFP4_ERR_SHAPE);
  EXPECT(ufp4_dequantize(nullptr, row.scales, row.tensor_scale, 64, 64, &ok, 1, dev<float>((size_t)9 << 30), nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_dequantize(row.codes, row.scales, nullptr, 64, 64, &ok, 1, dev<float>((size_t)9 << 30), nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_dequantize(row.codes, row.scales, nullptr, 64, 64, &mx, 1, dev<float>((size_t)9 << 30), nullptr), UFP4_OK);
  EXPECT(ufp4_dequantize(row.codes, row.scales, row.tensor_scale, 64, 64, &ok, 0, dev<float>(((size_t)9 << 30) + 4),
                         nullptr),
         UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_dequantize(row.codes, row.scales, row.tensor_scale, 0, 64, &ok, 0, nullptr, nullptr), UFP4_OK);
  ufp4_stats_t stt;
  EXPECT(ufp4_stats(x, 64, 64, 64, 2, &ok, row.codes, row.scales, row.tensor_scale, ws, wsb, &stt, nullptr),
         UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_stats(x, 64, 64, 64, 0, &ok, row.codes, row.scales, row.tensor_scale, ws, 512, &stt, nullptr),
         UFP4_ERR_WORKSPACE);
  EXPECT(ufp4_stats(x, 0, 64, 64, 0, &ok, nullptr, nullptr, nullptr, ws, wsb, &stt, nullptr), UFP4_OK);
  EXPECT(stt.alpha == 1.0 && stt.n == 0, 1);
  EXPECT(ufp4_stats(x, 64, 64, 64, 1, &ok, row.codes, row.scales, row.tensor_scale, ws, wsb, &stt, nullptr),
         UFP4_ERR_HIP);  // the stub launch fails; nothing is read back

  // rounding hook, bf16 conversion, GEMM, delayed scaling
  EXPECT(ufp4_round_f32(dev<float>((size_t)9 << 30), 10, 4, 0, 0, row.codes, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_round_f32(dev<float>((size_t)9 << 30), 0, 0, 0, 0, nullptr, nullptr), UFP4_OK);
  EXPECT(ufp4_round_f32(dev<float>(((size_t)9 << 30) + 2), 10, 0, 0, 0, row.codes, nullptr), UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_round_f32(dev<float>((size_t)9 << 30), 10, 3, 1, 5, row.codes, nullptr), UFP4_OK);
  EXPECT(ufp4_f32_to_bf16(dev<float>((size_t)9 << 30), -1, dev<uint16_t>((size_t)10 << 30), nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_f32_to_bf16(dev<float>(((size_t)9 << 30) + 1), 4, dev<uint16_t>((size_t)10 << 30), nullptr), UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_f32_to_bf16(dev<float>((size_t)9 << 30), 4, dev<uint16_t>((size_t)10 << 30), nullptr), UFP4_OK);
  float* c = dev<float>((size_t)11 << 30);
  EXPECT(ufp4_gemm_nt(&ok, 256, 256, 48, row, row, c, 256, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_gemm_nt(&mx, 256, 256, 64, row, row, c, 256, nullptr), UFP4_OK);  // MX32: scaled-MFMA path
  EXPECT(ufp4_gemm_nt(&mx, 256, 256, 48, row, row, c, 256, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_gemm_nt(&ok, 256, 256, 64, row, row, c, 128, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_gemm_nt(&ok, (int64_t)0x10000 * 256, 256, 64, row, row, c, 256, nullptr), UFP4_ERR_SHAPE);
  EXPECT(ufp4_gemm_nt(&ok, 0, 256, 64, row, row, c, 256, nullptr), UFP4_OK);
  EXPECT(ufp4_gemm_nt(&ok, 8192, 8192, 2048, row, col, c, 8192, nullptr), UFP4_OK);
  const float* ain = dev<float>((size_t)12 << 30);
  float* aout = dev<float>((size_t)13 << 30);
  EXPECT(ufp4_quantize_delayed(x, 8192, 2048, 2048, &mx, ain, 1, aout, row, col, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_delayed(x, 8192, 2048, 2048, &ok, ain, 0, aout, row, col, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_quantize_delayed(x, 8192, 2048, 2048, &ok, ain, 600, const_cast<float*>(ain) + 8, row, col, nullptr),
         UFP4_ERR_INVALID_ARGUMENT);  // overlapping maxima
  EXPECT(ufp4_quantize_delayed(x, 8192, 2048, 2048, &ok, ain + 1, 1, aout, row, col, nullptr), UFP4_ERR_ALIGNMENT);
  EXPECT(ufp4_quantize_delayed(x, 8192, 2048, 2048, &ok, ain, 512, aout, row, col, nullptr), UFP4_OK);
  EXPECT(ufp4_quantize_delayed(x, 8192, 2048, 2048, &sr, ain, 1, nullptr, row, none, nullptr), UFP4_OK);
  EXPECT(ufp4_quantize_delayed(nullptr, 0, 2048, 2048, &ok, ain, 1, aout, row, col, nullptr), UFP4_OK);

  // host helpers and recipes
  int8_t signs[16];
  EXPECT(ufp4_rht_signs(7, nullptr), UFP4_ERR_INVALID_ARGUMENT);
  for (uint64_t s = 0; s < 64; ++s) {
    EXPECT(ufp4_rht_signs(s * 0x9E3779B97F4A7C15ull, signs), UFP4_OK);
    for (int j = 0; j < 16; ++j) EXPECT(signs[j] == 1 || signs[j] == -1, 1);
  }
  int64_t offs[6] = {0, 5, 5, 37, 100, 101}, coff[6];
  EXPECT(ufp4_grouped_col_offsets(offs, 5, 16, coff), UFP4_OK);
  EXPECT(coff[5] == 16 + 0 + 32 + 64 + 16, 1);
  EXPECT(ufp4_grouped_col_offsets(offs, 5, 24, coff), UFP4_ERR_INVALID_ARGUMENT);
  int64_t bad_offs[3] = {0, 9, 4};
  EXPECT(ufp4_grouped_col_offsets(bad_offs, 2, 16, coff), UFP4_ERR_INVALID_ARGUMENT);
  for (int r = 0; r < 3; ++r)
    for (int g = 0; g < 3; ++g)
      for (int o = 0; o < 2; ++o) {
        ufp4_config rc;
        int32_t lay, ten;
        EXPECT(ufp4_recipe_config(r, g, o, 3, 4, &rc, &lay, &ten), UFP4_OK);
        EXPECT(rc.scaling == UFP4_SCALE_NV16 && (lay == 0 || lay == 1) && ten >= 0 && ten <= 2, 1);
      }
  ufp4_config rc;
  int32_t lay, ten;
  EXPECT(ufp4_recipe_config(3, 0, 0, 3, 4, &rc, &lay, &ten), UFP4_ERR_INVALID_ARGUMENT);
  EXPECT(ufp4_recipe_config(0, 0, 0, 3, 4, nullptr, &lay, &ten), UFP4_ERR_INVALID_ARGUMENT);

  munmap(m, kSpan);
  if (g_fail) {
    fprintf(stderr, "%d unexpected results\n", g_fail);
    return 1;
  }
  printf("abi host checks passed (%d stubbed launches)\n", ufp4::g_stub_calls);
  return 0;
}
