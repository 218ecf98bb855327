"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/ufp4.h, rejects bad arguments on the host before any
launch, and its host helpers agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ufp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ufp4_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def F():
    import fp4_quantization_amd as F
    return F


def test_exports_every_declared_symbol(F):
    names = declared_functions()
    assert len(names) >= 12
    raw = ctypes.CDLL(F.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(F._lib.EXPORTED)


def test_status_strings(F):
    for s in range(8):
        assert F.lib.ufp4_status_string(s) != b"unknown status"
    assert b"exchange" in F.lib.ufp4_status_string(7)
    assert F.lib.ufp4_status_string(99) == b"unknown status"


def test_host_signs_and_offsets_match_oracle(F, orc):
    for seed in (0, 1, 2, 3, 4, 77, 2**63 + 5):
        np.testing.assert_array_equal(F.ufp4_rht_signs(seed), orc.rht_signs(seed))
    rng = np.random.default_rng(0)
    for block in (16, 32):
        counts = rng.integers(0, 100, size=40)
        off = np.concatenate([[0], np.cumsum(counts)])
        np.testing.assert_array_equal(F.ufp4_grouped_col_offsets(off, block),
                                      orc.grouped_col_offsets(off, block))


def test_workspace_size(F):
    assert F.lib.ufp4_workspace_size(8192, 2048, 1) > 0
    assert F.lib.ufp4_workspace_size(-1, 16, 1) == 0
    assert F.lib.ufp4_workspace_size(16, 16, 0) == 0
    assert F.lib.ufp4_workspace_size(65536, 4096, 64) >= F.lib.ufp4_workspace_size(65536, 4096, 1)


def test_delayed_arguments(F):
    # host-side checks only (fake device pointers are never dereferenced)
    cfg = F.config()
    mx = F.config(scaling=F.SCALE_MX32)
    q = F.ufp4_qtensor(ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288))
    none = F.ufp4_qtensor(None, None, None)
    x, a_in, a_out = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), ctypes.c_void_p(1 << 22)
    call = F.lib.ufp4_quantize_delayed
    assert F.lib.ufp4_amax_tiles(8192, 2048) == 512
    assert F.lib.ufp4_amax_tiles(0, 2048) == 0
    assert call(x, 64, 64, 64, ctypes.byref(mx), a_in, 1, a_out, q, q, None) == 1    # MX32
    assert call(x, 64, 64, 64, ctypes.byref(cfg), None, 1, a_out, q, q, None) == 1   # no maxima
    assert call(x, 64, 64, 64, ctypes.byref(cfg), a_in, 0, a_out, q, q, None) == 1   # n_in 0
    assert call(x, 64, 40, 64, ctypes.byref(cfg), a_in, 1, a_out, q, q, None) == 2   # cols % 16
    assert call(x, 40, 64, 64, ctypes.byref(cfg), a_in, 1, a_out, q, q, None) == 2   # rows % 16, col layout
    assert call(x, 64, 64, 64, ctypes.byref(cfg), ctypes.c_void_p((1 << 21) + 4), 1, a_out, q, q, None) == 3
    assert call(x, 64, 64, 64, ctypes.byref(cfg), a_in, 1, a_in, q, q, None) == 1    # overlap
    assert call(x, 64, 64, 64, ctypes.byref(cfg), a_in, 1, a_out, none, q, None) == 1  # row output needed


def test_gemm_arguments(F):
    cfg, mx = F.config(), F.config(scaling=F.SCALE_MX32)
    q = F.ufp4_qtensor(ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288))
    c = ctypes.c_void_p(1 << 20)
    g = F.lib.ufp4_gemm_nt
    assert g(ctypes.byref(mx), 16, 16, 48, q, q, c, 16, None) == 2    # MX32: K % 32 as well
    assert g(ctypes.byref(cfg), 16, 16, 48, q, q, c, 16, None) == 2   # K % 32
    assert g(ctypes.byref(cfg), 16, 16, 32, q, q, c, 8, None) == 1    # ldc < N
    assert g(ctypes.byref(cfg), -1, 16, 32, q, q, c, 16, None) == 1
    assert g(ctypes.byref(cfg), 16, 16, 32, q, q, None, 16, None) == 1
    bad = F.ufp4_qtensor(ctypes.c_void_p(4100), ctypes.c_void_p(8192), ctypes.c_void_p(12288))
    assert g(ctypes.byref(cfg), 16, 16, 32, bad, q, c, 16, None) == 3
    assert g(ctypes.byref(cfg), 0, 16, 32, q, q, c, 16, None) == 0    # nothing to do


def test_set_schedule_arguments(F):
    assert F.lib.ufp4_set_schedule(3, 0) == 1
    assert F.lib.ufp4_set_schedule(-1, 0) == 1
    assert F.lib.ufp4_set_schedule(2, -1) == 1
    for mode in (1, 2, 0):
        assert F.lib.ufp4_set_schedule(mode, 0) == 0
    assert F.lib.ufp4_set_schedule(0, 0) == 0


# Argument errors are detected on the host before anything is enqueued, so
# these calls are safe with fake (never dereferenced) pointers and no GPU.
FAKE = 1 << 40  # 16-byte aligned, never touched


def q(F, codes=FAKE, scales=FAKE, ts=FAKE):
    return F.ufp4_qtensor(codes, scales, ts)


def call_quant(F, rows=64, cols=64, ld=64, cfg=None, out=None, ws=FAKE, ws_bytes=1 << 30, x=FAKE):
    cfg = cfg or F.config()
    return F.lib.ufp4_quantize(ctypes.c_void_p(x), rows, cols, ld, ctypes.byref(cfg), out or q(F),
                               ctypes.c_void_p(ws), ws_bytes, None)


def test_quantize_argument_errors(F):
    assert call_quant(F, cfg=F.config(grid=4)) == 1
    assert call_quant(F, cfg=F.config(rounding=2)) == 1
    assert call_quant(F, cfg=F.config(scaling=5)) == 1
    assert call_quant(F, cfg=F.config(rht=2)) == 1
    assert F.lib.ufp4_quantize(ctypes.c_void_p(FAKE), 64, 64, 64, None, q(F), None, 0, None) == 1
    assert call_quant(F, rows=-1) == 1
    assert call_quant(F, ld=32) == 1
    assert call_quant(F, cols=24) == 2                      # not a multiple of 16
    assert call_quant(F, cols=48, ld=48, cfg=F.config(scaling=1)) == 2  # MX32 needs 32
    assert call_quant(F, x=FAKE + 2) == 3
    assert call_quant(F, ld=68) == 3
    assert call_quant(F, out=q(F, codes=FAKE + 4)) == 3
    assert call_quant(F, out=q(F, codes=0)) == 1
    assert call_quant(F, x=0) == 1
    assert call_quant(F, ws=0) == 4
    assert call_quant(F, ws_bytes=16) == 4
    assert call_quant(F, ws=FAKE + 16) == 4


def test_rowcol_and_grouped_argument_errors(F):
    cfg = F.config()
    rc = F.lib.ufp4_quantize_rowcol(ctypes.c_void_p(FAKE), 40, 64, 64, ctypes.byref(cfg), q(F), q(F),
                                    ctypes.c_void_p(FAKE), 1 << 30, None)
    assert rc == 2  # rows not a multiple of 16
    rc = F.lib.ufp4_quantize_rowcol(ctypes.c_void_p(FAKE), 64, 64, 64, ctypes.byref(cfg), q(F),
                                    q(F, scales=0), ctypes.c_void_p(FAKE), 1 << 30, None)
    assert rc == 1

    def grouped(E=4, padded=None, offsets=FAKE, row=None, col=None, cols=64, rows=100):
        return F.lib.ufp4_quantize_grouped(ctypes.c_void_p(FAKE), rows, cols, ctypes.c_void_p(offsets), E,
                                           padded if padded is not None else 128, ctypes.byref(cfg),
                                           row or q(F), col or q(F), ctypes.c_void_p(FAKE), 1 << 30, None)
    assert grouped(E=0) == 1
    assert grouped(E=1025) == 1
    assert grouped(offsets=0) == 1
    assert grouped(offsets=FAKE + 4) == 3
    assert grouped(padded=96) == 2          # fewer than total rows
    assert grouped(padded=120) == 2         # not a multiple of 16
    assert grouped(padded=100 + 15 * 4 + 16) == 2  # more than any segmentation allows
    assert grouped(row=q(F, codes=0, scales=0, ts=0), col=q(F, codes=0, scales=0, ts=0)) == 1
    assert grouped(row=q(F, codes=0)) == 1
    assert grouped(cols=40) == 2


def test_other_entry_point_errors(F):
    cfg = F.config()
    assert F.lib.ufp4_dequantize(None, None, None, 16, 24, ctypes.byref(cfg), 0, None, None) == 2
    assert F.lib.ufp4_dequantize(None, None, None, 16, 32, ctypes.byref(cfg), 0, None, None) == 1
    assert F.lib.ufp4_dequantize(None, None, None, 0, 32, ctypes.byref(cfg), 0, None, None) == 0
    st = F.ufp4_stats_t()
    assert F.lib.ufp4_stats(None, 16, 16, 16, 2, ctypes.byref(cfg), None, None, None, None, 0,
                            ctypes.byref(st), None) == 1
    assert F.lib.ufp4_stats(None, 16, 16, 16, 0, ctypes.byref(cfg), None, None, None, None, 0,
                            ctypes.byref(st), None) == 4
    assert F.lib.ufp4_round_f32(None, 10, 0, 0, 0, None, None) == 1
    assert F.lib.ufp4_round_f32(None, 10, 4, 0, 0, None, None) == 1
    assert F.lib.ufp4_round_f32(None, 0, 0, 0, 0, None, None) == 0
    assert F.lib.ufp4_rht_signs(0, None) == 1
    assert F.lib.ufp4_workspace_init(None, 0, None) == 4
    assert F.lib.ufp4_grouped_col_offsets(None, 1, 16, None) == 1
    ms = ctypes.c_float()
    for c, rows, a, b in ((cfg, 64, None, ctypes.byref(ms)), (cfg, 64, ctypes.byref(ms), None),
                          (F.config(scaling=1), 64, ctypes.byref(ms), ctypes.byref(ms)),
                          (cfg, 0, ctypes.byref(ms), ctypes.byref(ms))):
        assert F.lib.ufp4_time_rowcol(ctypes.c_void_p(FAKE), rows, 64, 64, ctypes.byref(c), q(F), q(F),
                                      ctypes.c_void_p(FAKE), 1 << 30, None, a, b) == 1


# The recipes as the pages state them ("Shrinkage Bias: The Hidden Geometric
# Trap in FP4 Training" (zhichai.net), "Key points"; "UFP4 Eliminates
# Shrinkage Bias ..." (autonainews.com), "The UFP4 Recipe"): UFP4 puts the RHT
# on all three GEMMs and rounds stochastically on dY only; the NVFP4 baseline
# keeps the RHT to bwd_dw.
RECIPE_EXPECT = {0: (0, {0, 1, 2}), 1: (1, {0, 1, 2}), 2: (2, {2})}  # recipe: (grid, GEMMs with RHT)


def test_recipe_presets(F):
    T, I, O = 48, 80, 112  # tokens, in, out: X [T][I], W [O][I], dY [T][O]
    shape = {F.TENSOR_X: (T, I), F.TENSOR_W: (O, I), F.TENSOR_DY: (T, O)}
    out_shape = {F.GEMM_FWD_Y: (T, O), F.GEMM_BWD_DX: (T, I), F.GEMM_BWD_DW: (O, I)}
    for recipe, (grid, rht_gemms) in RECIPE_EXPECT.items():
        for gemm in (F.GEMM_FWD_Y, F.GEMM_BWD_DX, F.GEMM_BWD_DW):
            lines, lengths, seeds = [], [], set()
            for operand in (F.OPERAND_A, F.OPERAND_B):
                cfg, layout, tensor = F.ufp4_recipe_config(recipe, gemm, operand, rht_seed=77, sr_seed=5)
                assert cfg.grid == grid and cfg.scaling == F.SCALE_NV16
                assert cfg.rht == (1 if gemm in rht_gemms else 0)
                sr = tensor == F.TENSOR_DY
                assert cfg.rounding == (F.ROUND_STOCHASTIC if sr else F.ROUND_RTNE)
                assert cfg.sr_seed == (5 if sr else 0)
                seeds.add(cfg.rht_seed)
                R, C = shape[tensor]
                # the layout's lines and block length: row-wise R x C, column-wise C x R
                ln, lg = (R, C) if layout == 0 else (C, R)
                lines.append(ln)
                lengths.append(lg)
            # a: M x K, b: N x K, C = a b^T has the GEMM's output shape
            assert lengths[0] == lengths[1], (recipe, gemm)
            assert tuple(lines) == out_shape[gemm], (recipe, gemm)
            assert seeds == {77}
    # the reduction dimensions: in, out, tokens
    for gemm, k in ((F.GEMM_FWD_Y, I), (F.GEMM_BWD_DX, O), (F.GEMM_BWD_DW, T)):
        _, layout, tensor = F.ufp4_recipe_config(0, gemm, F.OPERAND_A)
        R, C = shape[tensor]
        assert (C if layout == 0 else R) == k
    for bad in ((3, 0, 0), (-1, 0, 0), (0, 3, 0), (0, 0, 2)):
        with pytest.raises(F.Ufp4Error):
            F.ufp4_recipe_config(*bad)


def test_bench_algorithmic_bytes():
    # bf16 read once (2 B), codes of both layouts (2 x 0.5 B) and E4M3 scales
    # of both layouts (2 x 1/16 B) per element, plus two fp32 tensor scales
    import bench
    assert bench.algorithmic_bytes(8192, 2048) == 52_428_808
    n = 8192 * 2048
    assert bench.algorithmic_bytes(8192, 2048) == int(n * (2 + 0.5 + 0.5 + 1 / 16 + 1 / 16)) + 8


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: --gpus 2 exits with status 2 and a message, before any
    # device work
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
