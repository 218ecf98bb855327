"""ctypes binding of the C ABI in include/ufp4.h (argument marshalling only).

Every computation runs in the HIP library ``libufp4.so`` built for gfx950;
there is no Python or CPU fallback.  Importing the binding when the library
is missing raises ``ImportError``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libufp4.so")

UFP4_OK = 0
STATUS_NAMES = {0: "UFP4_OK", 1: "UFP4_ERR_INVALID_ARGUMENT", 2: "UFP4_ERR_SHAPE",
                3: "UFP4_ERR_ALIGNMENT", 4: "UFP4_ERR_WORKSPACE", 5: "UFP4_ERR_HIP",
                6: "UFP4_ERR_OFFSETS", 7: "UFP4_ERR_SYNC"}

GRID_E1M2, GRID_INT4, GRID_E2M1, GRID_E2M1C = 0, 1, 2, 3
ROUND_RTNE, ROUND_STOCHASTIC = 0, 1
SCALE_NV16, SCALE_MX32 = 0, 1
SCHEDULE_AUTO, SCHEDULE_TWO_PASS, SCHEDULE_SINGLE_PASS = 0, 1, 2
RECIPE_UFP4, RECIPE_UFP4_INT4, RECIPE_NVFP4 = 0, 1, 2
GEMM_FWD_Y, GEMM_BWD_DX, GEMM_BWD_DW = 0, 1, 2
OPERAND_A, OPERAND_B = 0, 1
TENSOR_X, TENSOR_W, TENSOR_DY = 0, 1, 2

EXPORTED = ["ufp4_status_string", "ufp4_workspace_size", "ufp4_workspace_init",
            "ufp4_workspace_status", "ufp4_quantize", "ufp4_quantize_rowcol",
            "ufp4_quantize_grouped", "ufp4_dequantize", "ufp4_stats", "ufp4_round_f32",
            "ufp4_rht_signs", "ufp4_grouped_col_offsets", "ufp4_time_rowcol", "ufp4_set_schedule",
            "ufp4_schedule_of", "ufp4_amax_tiles", "ufp4_quantize_delayed", "ufp4_gemm_nt",
            "ufp4_recipe_config", "ufp4_f32_to_bf16", "ufp4_quantize_rowcol_noalloc",
            "ufp4_quantize_grouped_delayed", "ufp4_roof_rowcol"]


class Ufp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")


class ufp4_config(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("scaling", ctypes.c_int32), ("rht", ctypes.c_int32),
                ("rht_seed", ctypes.c_uint64), ("sr_seed", ctypes.c_uint64)]


class ufp4_qtensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class ufp4_stats_t(ctypes.Structure):
    _fields_ = [("sqnr_db", ctypes.c_double), ("mean_signed_err", ctypes.c_double),
                ("mean_signed_err_grid", ctypes.c_double), ("alpha", ctypes.c_double),
                ("amax", ctypes.c_double), ("n", ctypes.c_uint64),
                ("code_hist", ctypes.c_uint64 * 16), ("n_saturated", ctypes.c_uint64),
                ("n_nonfinite", ctypes.c_uint64), ("n_zero_scale", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_ if k != "code_hist"}
        d["code_hist"] = list(self.code_hist)
        return d


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    cfgp = ctypes.POINTER(ufp4_config)
    L.ufp4_status_string.restype = ctypes.c_char_p
    L.ufp4_status_string.argtypes = [ctypes.c_int]
    L.ufp4_workspace_size.restype = sz
    L.ufp4_workspace_size.argtypes = [i64, i64, i32]
    L.ufp4_workspace_init.restype = ctypes.c_int
    L.ufp4_workspace_init.argtypes = [P, sz, P]
    L.ufp4_workspace_status.restype = ctypes.c_int
    L.ufp4_workspace_status.argtypes = [P, sz, ctypes.POINTER(ctypes.c_int), P]
    L.ufp4_quantize.restype = ctypes.c_int
    L.ufp4_quantize.argtypes = [P, i64, i64, i64, cfgp, ufp4_qtensor, P, sz, P]
    L.ufp4_quantize_rowcol.restype = ctypes.c_int
    L.ufp4_quantize_rowcol.argtypes = [P, i64, i64, i64, cfgp, ufp4_qtensor, ufp4_qtensor, P, sz, P]
    L.ufp4_quantize_rowcol_noalloc.restype = ctypes.c_int
    L.ufp4_quantize_rowcol_noalloc.argtypes = [P, i64, i64, i64, cfgp, ufp4_qtensor, ufp4_qtensor, P]
    L.ufp4_quantize_grouped_delayed.restype = ctypes.c_int
    L.ufp4_quantize_grouped_delayed.argtypes = [P, i64, i64, P, i32, i64, cfgp, P, P, ufp4_qtensor, ufp4_qtensor,
                                                P, sz, P]
    L.ufp4_quantize_grouped.restype = ctypes.c_int
    L.ufp4_quantize_grouped.argtypes = [P, i64, i64, P, i32, i64, cfgp, ufp4_qtensor, ufp4_qtensor,
                                        P, sz, P]
    L.ufp4_dequantize.restype = ctypes.c_int
    L.ufp4_dequantize.argtypes = [P, P, P, i64, i64, cfgp, i32, P, P]
    L.ufp4_stats.restype = ctypes.c_int
    L.ufp4_stats.argtypes = [P, i64, i64, i64, i32, cfgp, P, P, P, P, sz,
                             ctypes.POINTER(ufp4_stats_t), P]
    L.ufp4_round_f32.restype = ctypes.c_int
    L.ufp4_round_f32.argtypes = [P, i64, i32, i32, u64, P, P]
    L.ufp4_time_rowcol.restype = ctypes.c_int
    L.ufp4_time_rowcol.argtypes = [P, i64, i64, i64, cfgp, ufp4_qtensor, ufp4_qtensor, P, sz, P,
                                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
    L.ufp4_roof_rowcol.restype = ctypes.c_int
    L.ufp4_roof_rowcol.argtypes = [P, i64, i64, ufp4_qtensor, ufp4_qtensor, P]
    L.ufp4_rht_signs.restype = ctypes.c_int
    L.ufp4_rht_signs.argtypes = [u64, P]
    L.ufp4_grouped_col_offsets.restype = ctypes.c_int
    L.ufp4_grouped_col_offsets.argtypes = [P, i32, i32, P]
    L.ufp4_set_schedule.restype = ctypes.c_int
    L.ufp4_set_schedule.argtypes = [i32, i32]
    L.ufp4_gemm_nt.restype = ctypes.c_int
    L.ufp4_gemm_nt.argtypes = [cfgp, i64, i64, i64, ufp4_qtensor, ufp4_qtensor, P, i64, P]
    L.ufp4_amax_tiles.restype = i64
    L.ufp4_amax_tiles.argtypes = [i64, i64]
    L.ufp4_quantize_delayed.restype = ctypes.c_int
    L.ufp4_quantize_delayed.argtypes = [P, i64, i64, i64, cfgp, P, i32, P, ufp4_qtensor, ufp4_qtensor, P]
    L.ufp4_f32_to_bf16.restype = ctypes.c_int
    L.ufp4_f32_to_bf16.argtypes = [P, i64, P, P]
    L.ufp4_recipe_config.restype = ctypes.c_int
    L.ufp4_recipe_config.argtypes = [i32, i32, i32, u64, u64, cfgp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.ufp4_schedule_of.restype = ctypes.c_int
    L.ufp4_schedule_of.argtypes = [i64, i64, i32, i32, cfgp, ctypes.POINTER(i32)]
    return L


lib = _load()


def check(fn: str, status: int) -> None:
    if status != UFP4_OK:
        raise Ufp4Error(fn, status)
