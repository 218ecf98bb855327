"""MI355X (gfx950) fused random-Hadamard transform + 4-bit block quantization.

Thin Python layer over the C ABI of ``libufp4.so`` (include/ufp4.h): the
functions below marshal torch device tensors into pointers and call the
entry point of the same name.  PyTorch only provides device memory and
streams; every step of the quantization runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import (GEMM_BWD_DW, GEMM_BWD_DX, GEMM_FWD_Y, OPERAND_A, OPERAND_B, RECIPE_NVFP4, RECIPE_UFP4,
                   RECIPE_UFP4_INT4, TENSOR_DY, TENSOR_W, TENSOR_X,
                   GRID_E1M2, GRID_E2M1, GRID_E2M1C, GRID_INT4, LIB_PATH, ROUND_RTNE, ROUND_STOCHASTIC,
                   SCALE_MX32, SCALE_NV16, SCHEDULE_AUTO, SCHEDULE_SINGLE_PASS, SCHEDULE_TWO_PASS, Ufp4Error, check, lib, ufp4_config, ufp4_qtensor,
                   ufp4_stats_t)

__all__ = ["GRID_E1M2", "GRID_INT4", "GRID_E2M1", "GRID_E2M1C", "ROUND_RTNE", "ROUND_STOCHASTIC", "SCALE_NV16",
           "SCALE_MX32", "SCHEDULE_AUTO", "SCHEDULE_TWO_PASS", "SCHEDULE_SINGLE_PASS", "ufp4_set_schedule",
           "ufp4_schedule_of", "ufp4_amax_tiles", "ufp4_quantize_grouped_delayed", "ufp4_quantize_rowcol_noalloc", "ufp4_quantize_delayed", "ufp4_gemm_nt", "LIB_PATH", "Ufp4Error", "config", "QTensor", "Workspace", "alloc_layout",
           "ufp4_quantize", "ufp4_quantize_rowcol", "ufp4_quantize_grouped", "ufp4_dequantize",
           "ufp4_stats", "ufp4_round_f32", "ufp4_rht_signs", "ufp4_grouped_col_offsets", "ufp4_time_rowcol", "ufp4_roof_rowcol",
           "block_len", "ufp4_recipe_config", "RECIPE_UFP4", "RECIPE_UFP4_INT4", "RECIPE_NVFP4",
           "GEMM_FWD_Y", "GEMM_BWD_DX", "GEMM_BWD_DW", "OPERAND_A", "OPERAND_B", "TENSOR_X", "TENSOR_W",
           "TENSOR_DY", "ufp4_f32_to_bf16"]


def config(grid: int = GRID_E1M2, rounding: int = ROUND_RTNE, scaling: int = SCALE_NV16,
           rht: int = 1, rht_seed: int = 0, sr_seed: int = 0) -> ufp4_config:
    return ufp4_config(int(grid), int(rounding), int(scaling), int(rht), int(rht_seed), int(sr_seed))


def block_len(scaling: int) -> int:
    return 32 if scaling == SCALE_MX32 else 16


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bf16_view(x: torch.Tensor):
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("x must hold bf16 values (bfloat16, or their 16-bit patterns)")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    return x.shape[0], x.shape[1], x.stride(0)


class QTensor:
    """Device buffers of one quantized layout: packed codes, block scales and
    per-tensor scale(s)."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor):
        self.codes, self.scales, self.tensor_scale = codes, scales, tensor_scale

    def c(self) -> ufp4_qtensor:
        return ufp4_qtensor(self.codes.data_ptr(), self.scales.data_ptr(), self.tensor_scale.data_ptr())


def alloc_layout(lines: int, length: int, scaling: int, n_tensor_scales: int = 1,
                 device="cuda") -> QTensor:
    """Output buffers for `lines` block lines of `length` elements each."""
    B = block_len(scaling)
    return QTensor(torch.empty((lines, length // 2), dtype=torch.uint8, device=device),
                   torch.empty((lines, length // B), dtype=torch.uint8, device=device),
                   torch.empty(n_tensor_scales, dtype=torch.float32, device=device))


class Workspace:
    """Caller-owned device workspace (zeroed once by ufp4_workspace_init)."""

    def __init__(self, rows: int, cols: int, num_groups: int = 1, device="cuda", stream=None):
        self.nbytes = int(lib.ufp4_workspace_size(rows, cols, num_groups))
        if self.nbytes == 0:
            raise ValueError("invalid workspace shape")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        check("ufp4_workspace_init", lib.ufp4_workspace_init(_ptr(self.buf), self.nbytes, _stream(stream)))

    @property
    def ptr(self):
        return _ptr(self.buf)

    def status(self, stream=None) -> int:
        st = ctypes.c_int(0)
        check("ufp4_workspace_status", lib.ufp4_workspace_status(self.ptr, self.nbytes, ctypes.byref(st),
                                                                   _stream(stream)))
        return st.value


def ufp4_quantize(x: torch.Tensor, cfg: ufp4_config, row_out: QTensor, ws: Workspace | None,
                  stream=None) -> None:
    rows, cols, ld = _bf16_view(x)
    check("ufp4_quantize", lib.ufp4_quantize(_ptr(x), rows, cols, ld, ctypes.byref(cfg), row_out.c(),
                                             ws.ptr if ws else None, ws.nbytes if ws else 0,
                                             _stream(stream)))


def ufp4_quantize_rowcol(x: torch.Tensor, cfg: ufp4_config, row_out: QTensor, col_out: QTensor,
                         ws: Workspace | None, stream=None) -> None:
    rows, cols, ld = _bf16_view(x)
    check("ufp4_quantize_rowcol",
          lib.ufp4_quantize_rowcol(_ptr(x), rows, cols, ld, ctypes.byref(cfg), row_out.c(), col_out.c(),
                                   ws.ptr if ws else None, ws.nbytes if ws else 0, _stream(stream)))


def ufp4_quantize_rowcol_noalloc(x: torch.Tensor, cfg: ufp4_config, row_out: QTensor, col_out: QTensor,
                                 stream=None) -> None:
    rows, cols, ld = _bf16_view(x)
    check("ufp4_quantize_rowcol_noalloc",
          lib.ufp4_quantize_rowcol_noalloc(_ptr(x), rows, cols, ld, ctypes.byref(cfg), row_out.c(), col_out.c(),
                                           _stream(stream)))


def ufp4_quantize_grouped(x: torch.Tensor, offsets_dev: torch.Tensor, padded_rows: int,
                          cfg: ufp4_config, row_out: QTensor | None, col_out: QTensor | None,
                          ws: Workspace | None, stream=None) -> None:
    rows, cols, ld = _bf16_view(x)
    if ld != cols:
        raise ValueError("grouped input must be contiguous")
    if offsets_dev.dtype != torch.int64:
        raise TypeError("offsets must be int64")
    E = offsets_dev.numel() - 1
    null = ufp4_qtensor(None, None, None)
    check("ufp4_quantize_grouped",
          lib.ufp4_quantize_grouped(_ptr(x), rows, cols, _ptr(offsets_dev), E, int(padded_rows),
                                    ctypes.byref(cfg), row_out.c() if row_out else null,
                                    col_out.c() if col_out else null, ws.ptr if ws else None,
                                    ws.nbytes if ws else 0, _stream(stream)))



def ufp4_quantize_grouped_delayed(x: torch.Tensor, offsets_dev: torch.Tensor, padded_rows: int,
                                  cfg: ufp4_config, amax_in: torch.Tensor, amax_out: torch.Tensor | None,
                                  row_out: QTensor | None, col_out: QTensor | None, ws: Workspace,
                                  stream=None) -> None:
    """amax_in / amax_out: float32 device tensors of num_groups (row, column) pairs."""
    rows, cols, ld = _bf16_view(x)
    if ld != cols:
        raise ValueError("grouped input must be contiguous")
    if offsets_dev.dtype != torch.int64 or amax_in.dtype != torch.float32:
        raise TypeError("offsets must be int64 and maxima float32")
    E = offsets_dev.numel() - 1
    if amax_in.numel() != 2 * E or (amax_out is not None and amax_out.numel() != 2 * E):
        raise ValueError("one (row, column) pair of maxima per segment")
    null = ufp4_qtensor(None, None, None)
    check("ufp4_quantize_grouped_delayed",
          lib.ufp4_quantize_grouped_delayed(_ptr(x), rows, cols, _ptr(offsets_dev), E, int(padded_rows),
                                            ctypes.byref(cfg), _ptr(amax_in), _ptr(amax_out),
                                            row_out.c() if row_out else null, col_out.c() if col_out else null,
                                            ws.ptr, ws.nbytes, _stream(stream)))

def ufp4_set_schedule(schedule: int, left_stride: int = 0) -> None:
    """Process-wide schedule of dense NV16 calls (SCHEDULE_AUTO, _TWO_PASS,
    _SINGLE_PASS); left_stride > 1 makes the single pass leave every tile whose
    index is not a multiple of it to the other workgroups (test hook)."""
    check("ufp4_set_schedule", lib.ufp4_set_schedule(int(schedule), int(left_stride)))


def ufp4_gemm_nt(cfg: ufp4_config, a: QTensor, b: QTensor, M: int, N: int, K: int, c: torch.Tensor,
                 stream=None) -> None:
    """c[m][n] = sum_k deq(a)[m][k] deq(b)[n][k] for NV16 row-wise layouts of
    an M x K and an N x K matrix; c float32 [M][ldc >= N] on the device."""
    assert c.dtype == torch.float32 and c.dim() == 2 and c.stride(1) == 1
    check("ufp4_gemm_nt", lib.ufp4_gemm_nt(ctypes.byref(cfg), int(M), int(N), int(K), a.c(), b.c(), _ptr(c),
                                           c.stride(0), _stream(stream)))


def ufp4_amax_tiles(rows: int, cols: int) -> int:
    """Pairs of tile maxima a delayed call on rows x cols writes."""
    return int(lib.ufp4_amax_tiles(int(rows), int(cols)))


def ufp4_quantize_delayed(x: torch.Tensor, cfg: ufp4_config, amax_in: torch.Tensor, amax_out,
                          row_out: QTensor, col_out: QTensor | None = None, stream=None) -> None:
    """Delayed scaling: tensor scales from amax_in (float32 [n, 2] on the
    device: row-wise, column-wise maxima); this call's tile maxima go to
    amax_out (float32 [ufp4_amax_tiles(rows, cols), 2], or None)."""
    rows, cols, ld = _bf16_view(x)
    assert amax_in.dtype == torch.float32 and amax_in.is_contiguous() and amax_in.numel() % 2 == 0
    if amax_out is not None:
        assert amax_out.dtype == torch.float32 and amax_out.is_contiguous()
        assert amax_out.numel() >= 2 * ufp4_amax_tiles(rows, cols)
    col = col_out.c() if col_out is not None else ufp4_qtensor(None, None, None)
    check("ufp4_quantize_delayed",
          lib.ufp4_quantize_delayed(_ptr(x), rows, cols, ld, ctypes.byref(cfg), _ptr(amax_in),
                                    amax_in.numel() // 2, _ptr(amax_out) if amax_out is not None else None,
                                    row_out.c(), col, _stream(stream)))


def ufp4_schedule_of(rows: int, cols: int, cfg: ufp4_config, num_groups: int = 1,
                     both_layouts: bool = True) -> int:
    """SCHEDULE_SINGLE_PASS or SCHEDULE_TWO_PASS: what a call on this shape
    and configuration (both layouts, or one) takes on the current device."""
    out = ctypes.c_int32(0)
    check("ufp4_schedule_of", lib.ufp4_schedule_of(int(rows), int(cols), int(num_groups), int(bool(both_layouts)),
                                                   ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def ufp4_time_rowcol(x: torch.Tensor, cfg: ufp4_config, row_out: QTensor, col_out: QTensor,
                     ws: Workspace, stream=None) -> tuple[float, float]:
    """One ufp4_quantize_rowcol call with hipEvents around each of its
    kernels; returns (ms of the tensor-maximum kernel, ms of the quantization
    kernel); under the single-pass schedule (0, ms of the one kernel).
    Synchronizes."""
    rows, cols, ld = _bf16_view(x)
    a, b = ctypes.c_float(0), ctypes.c_float(0)
    check("ufp4_time_rowcol", lib.ufp4_time_rowcol(_ptr(x), rows, cols, ld, ctypes.byref(cfg), row_out.c(),
                                                   col_out.c(), ws.ptr, ws.nbytes, _stream(stream),
                                                   ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def ufp4_roof_rowcol(x: torch.Tensor, row_out: QTensor, col_out: QTensor, stream=None) -> None:
    """The memory traffic of a row+col call on x with no arithmetic (a
    bandwidth reference): the quantization kernels' loads, and every byte of
    both layouts' codes and block scales written (as zeros, unless a lane's
    input words xor to one fixed constant).  rows % 128 == 0, cols % 256 == 0."""
    rows, cols, ld = _bf16_view(x)
    if ld != cols:
        raise ValueError("the roof hook takes a contiguous tensor")
    check("ufp4_roof_rowcol", lib.ufp4_roof_rowcol(_ptr(x), rows, cols, row_out.c(), col_out.c(), _stream(stream)))


def ufp4_dequantize(q: QTensor, rows: int, cols: int, cfg: ufp4_config, inverse_rht: bool,
                    out: torch.Tensor, stream=None) -> None:
    check("ufp4_dequantize",
          lib.ufp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), rows, cols,
                              ctypes.byref(cfg), int(bool(inverse_rht)), _ptr(out), _stream(stream)))


def ufp4_stats(x: torch.Tensor, layout: int, cfg: ufp4_config, q: QTensor, ws: Workspace,
               stream=None) -> dict:
    rows, cols, ld = _bf16_view(x)
    out = ufp4_stats_t()
    check("ufp4_stats", lib.ufp4_stats(_ptr(x), rows, cols, ld, int(layout), ctypes.byref(cfg),
                                       _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), ws.ptr,
                                       ws.nbytes, ctypes.byref(out), _stream(stream)))
    return out.as_dict()


def ufp4_round_f32(y: torch.Tensor, grid: int, rounding: int, sr_seed: int, codes: torch.Tensor,
                   stream=None) -> None:
    if y.dtype != torch.float32 or codes.dtype != torch.uint8 or codes.numel() != y.numel():
        raise TypeError("y must be float32 and codes uint8 of the same size")
    check("ufp4_round_f32", lib.ufp4_round_f32(_ptr(y), y.numel(), int(grid), int(rounding),
                                               int(sr_seed), _ptr(codes), _stream(stream)))


def ufp4_rht_signs(rht_seed: int) -> np.ndarray:
    s = np.zeros(16, dtype=np.int8)
    check("ufp4_rht_signs", lib.ufp4_rht_signs(int(rht_seed), s.ctypes.data_as(ctypes.c_void_p)))
    return s


def ufp4_grouped_col_offsets(offsets, block: int) -> np.ndarray:
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    out = np.zeros(off.size, dtype=np.int64)
    check("ufp4_grouped_col_offsets",
          lib.ufp4_grouped_col_offsets(off.ctypes.data_as(ctypes.c_void_p), off.size - 1, int(block),
                                       out.ctypes.data_as(ctypes.c_void_p)))
    return out


def ufp4_recipe_config(recipe: int, gemm: int, operand: int, rht_seed: int = 0, sr_seed: int = 0):
    """(config, layout, tensor) of one operand of one training GEMM under a
    recipe: layout 0 row-wise / 1 column-wise, tensor TENSOR_X/W/DY."""
    cfg = ufp4_config()
    layout, tensor = ctypes.c_int32(), ctypes.c_int32()
    check("ufp4_recipe_config", lib.ufp4_recipe_config(int(recipe), int(gemm), int(operand), int(rht_seed),
                                                       int(sr_seed), ctypes.byref(cfg), ctypes.byref(layout),
                                                       ctypes.byref(tensor)))
    return cfg, layout.value, tensor.value


def ufp4_f32_to_bf16(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 (as int16 bit patterns) of a contiguous float32 device tensor,
    rounded to nearest even by the library's kernel."""
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    check("ufp4_f32_to_bf16", lib.ufp4_f32_to_bf16(_ptr(x), x.numel(), _ptr(out), _stream(stream)))
    return out
