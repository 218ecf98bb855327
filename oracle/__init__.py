"""CPU oracle for the UFP4 quantization hot path -- TEST INFRASTRUCTURE.

A plain, slow, single-threaded C implementation (``ufp4_oracle.c``) wrapped
with ctypes and numpy.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(``fp4_quantization_amd``) never does, and shares no code with it.

Functions mirror the C-ABI semantics on host arrays.  See ``ufp4_oracle.h``
for the definitions and the sources they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libufp4_oracle.so")
SOURCES = [os.path.join(_HERE, "ufp4_oracle.c")]

GRID_E1M2, GRID_INT4, GRID_E2M1, GRID_E2M1_CLAMP = 0, 1, 2, 3
ROUND_RTNE, ROUND_SR = 0, 1
SCALE_NV16, SCALE_MX32 = 0, 1
LAYOUT_ROW, LAYOUT_COL = 0, 1


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc: binary32, round-to-nearest, no FMA contraction."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp"] + SOURCES + ["-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class Config(ctypes.Structure):
    _fields_ = [("grid", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("scaling", ctypes.c_int32), ("rht", ctypes.c_int32),
                ("rht_seed", ctypes.c_uint64), ("sr_seed", ctypes.c_uint64)]


class Stats(ctypes.Structure):
    _fields_ = [("sqnr_db", ctypes.c_double), ("mean_signed_err", ctypes.c_double),
                ("mean_signed_err_grid", ctypes.c_double), ("alpha", ctypes.c_double),
                ("amax", ctypes.c_double), ("n", ctypes.c_uint64),
                ("code_hist", ctypes.c_uint64 * 16), ("n_saturated", ctypes.c_uint64),
                ("n_nonfinite", ctypes.c_uint64), ("n_zero_scale", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_ if k != "code_hist"}
        d["code_hist"] = list(self.code_hist)
        return d


_lib = None


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_rht_signs.argtypes = [u64, P]
        L.orc_sr_word.restype = ctypes.c_uint32
        L.orc_sr_word.argtypes = [u64, u64, ctypes.c_uint32]
        L.orc_fwht16_stages.argtypes = [P]
        L.orc_rht16.argtypes = [P, P, P]
        L.orc_inverse_rht16.argtypes = [P, P, P]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_n.argtypes = [P, i64, P]
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_grid_qmax.restype = ctypes.c_float
        L.orc_grid_qmax.argtypes = [i32]
        L.orc_code_value.restype = ctypes.c_float
        L.orc_code_value.argtypes = [ctypes.c_uint8, i32]
        L.orc_round_to_code.restype = ctypes.c_uint8
        L.orc_round_to_code.argtypes = [ctypes.c_float, i32, i32, ctypes.c_uint32]
        L.orc_round_f32.restype = ctypes.c_int
        L.orc_round_f32.argtypes = [P, i64, i32, i32, u64, P]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_quantize.argtypes = [P, i64, i64, i64, ctypes.POINTER(Config), i32, P, P, P]
        L.orc_quantize_given_amax.restype = ctypes.c_int
        L.orc_quantize_given_amax.argtypes = [P, i64, i64, i64, ctypes.POINTER(Config), i32, ctypes.c_float,
                                              P, P, P, P]
        L.orc_grouped_col_offsets.restype = ctypes.c_int
        L.orc_grouped_col_offsets.argtypes = [P, i32, i32, P]
        L.orc_quantize_grouped.restype = ctypes.c_int
        L.orc_quantize_grouped.argtypes = [P, i64, i64, P, i32, ctypes.POINTER(Config),
                                           P, P, P, P, P, P]
        L.orc_quantize_grouped_given_amax.restype = ctypes.c_int
        L.orc_quantize_grouped_given_amax.argtypes = [P, i64, i64, P, i32, ctypes.POINTER(Config), P, P,
                                                      P, P, P, P, P, P]
        L.orc_dequantize.restype = ctypes.c_int
        L.orc_dequantize.argtypes = [P, P, P, i64, i64, ctypes.POINTER(Config), i32, P]
        L.orc_compute_stats.restype = ctypes.c_int
        L.orc_compute_stats.argtypes = [P, i64, i64, i64, i32, ctypes.POINTER(Config),
                                        P, P, P, ctypes.POINTER(Stats)]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def config(grid=GRID_E1M2, rounding=ROUND_RTNE, scaling=SCALE_NV16, rht=1,
           rht_seed=0, sr_seed=0) -> Config:
    return Config(int(grid), int(rounding), int(scaling), int(rht), int(rht_seed), int(sr_seed))


def block_len(scaling: int) -> int:
    return 32 if scaling == SCALE_MX32 else 16


# ---------------------------------------------------------------- primitives
def bf16_to_f32(h: int) -> float:
    return lib().orc_bf16_to_f32(h)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def rht_signs(seed: int) -> np.ndarray:
    s = np.zeros(16, dtype=np.int8)
    lib().orc_rht_signs(int(seed), _ptr(s))
    return s


def sr_word(seed: int, index: int, stream: int) -> int:
    return int(lib().orc_sr_word(int(seed), int(index), int(stream)))


def fwht16_stages(v) -> np.ndarray:
    a = np.array(v, dtype=np.float32).copy()
    lib().orc_fwht16_stages(_ptr(a))
    return a


def rht16(x, signs) -> np.ndarray:
    xa = np.ascontiguousarray(x, dtype=np.float32)
    s = np.ascontiguousarray(signs, dtype=np.int8)
    v = np.zeros(16, dtype=np.float32)
    lib().orc_rht16(_ptr(xa), _ptr(s), _ptr(v))
    return v


def inverse_rht16(v, signs) -> np.ndarray:
    va = np.ascontiguousarray(v, dtype=np.float32)
    s = np.ascontiguousarray(signs, dtype=np.int8)
    x = np.zeros(16, dtype=np.float32)
    lib().orc_inverse_rht16(_ptr(va), _ptr(s), _ptr(x))
    return x


def e4m3_encode(q: float) -> int:
    return int(lib().orc_e4m3_encode(float(q)))


def e4m3_encode_n(q: np.ndarray) -> np.ndarray:
    qa = np.ascontiguousarray(q, dtype=np.float32)
    out = np.zeros(qa.size, dtype=np.uint8)
    lib().orc_e4m3_encode_n(_ptr(qa), qa.size, _ptr(out))
    return out


def e4m3_decode(c: int) -> float:
    return float(lib().orc_e4m3_decode(int(c)))


def grid_qmax(grid: int) -> float:
    return float(lib().orc_grid_qmax(int(grid)))


def code_value(code: int, grid: int) -> float:
    return float(lib().orc_code_value(int(code), int(grid)))


def round_f32(y: np.ndarray, grid: int, rounding: int = ROUND_RTNE, sr_seed: int = 0) -> np.ndarray:
    ya = np.ascontiguousarray(y, dtype=np.float32)
    codes = np.zeros(ya.size, dtype=np.uint8)
    rc = lib().orc_round_f32(_ptr(ya), ya.size, int(grid), int(rounding), int(sr_seed), _ptr(codes))
    if rc:
        raise ValueError(f"orc_round_f32 failed ({rc})")
    return codes


# -------------------------------------------------------------- whole tensors
def out_shapes(rows: int, cols: int, layout: int, scaling: int):
    B = block_len(scaling)
    if layout == LAYOUT_ROW:
        return (rows, cols // 2), (rows, cols // B)
    return (cols, rows // 2), (cols, rows // B)


def quantize(x_bf16: np.ndarray, cfg: Config, layout: int):
    """x_bf16: uint16 array [rows][ld>=cols] (bf16 bit patterns).
    Returns (codes, scales, tensor_scale) for the layout."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    cshape, sshape = out_shapes(rows, cols, layout, cfg.scaling)
    codes = np.zeros(cshape, dtype=np.uint8)
    scales = np.zeros(sshape, dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    rc = lib().orc_quantize(_ptr(x), rows, cols, cols, ctypes.byref(cfg), int(layout),
                            _ptr(codes), _ptr(scales), _ptr(ts))
    if rc:
        raise ValueError(f"orc_quantize failed ({rc})")
    return codes, scales, ts


def grouped_col_offsets(offsets, block: int) -> np.ndarray:
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    E = off.size - 1
    col = np.zeros(E + 1, dtype=np.int64)
    rc = lib().orc_grouped_col_offsets(_ptr(off), E, int(block), _ptr(col))
    if rc:
        raise ValueError("bad offsets")
    return col


def gemm_nt_reference(a, b, cfg: Config, M: int, N: int, K: int) -> np.ndarray:
    """The product the consumer GEMM computes, in float64: each operand
    (codes, scales, tensor_scale) of an M x K / N x K row-wise layout is
    dequantized by the oracle (no inverse transform), then
    C = A_hat @ B_hat^T.  Returns (C, |A_hat| @ |B_hat|^T) for error bounds."""
    ah = dequantize(a[0], a[1], a[2], M, K, cfg).astype(np.float64)
    bh = dequantize(b[0], b[1], b[2], N, K, cfg).astype(np.float64)
    return ah @ bh.T, np.abs(ah) @ np.abs(bh).T


def quantize_given_amax(x_bf16: np.ndarray, cfg: Config, layout: int, amax_given: float):
    """Delayed scaling (NV16): quantize with the tensor scale taken from
    amax_given.  Returns (codes, scales, tensor_scale, amax_seen)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    cshape, sshape = out_shapes(rows, cols, layout, cfg.scaling)
    codes = np.zeros(cshape, dtype=np.uint8)
    scales = np.zeros(sshape, dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    seen = np.zeros(1, dtype=np.float32)
    rc = lib().orc_quantize_given_amax(_ptr(x), rows, cols, cols, ctypes.byref(cfg), int(layout),
                                       float(amax_given), _ptr(codes), _ptr(scales), _ptr(ts), _ptr(seen))
    if rc:
        raise ValueError(f"orc_quantize_given_amax failed ({rc})")
    return codes, scales, ts, float(seen[0])


def quantize_grouped(x_bf16: np.ndarray, offsets, cfg: Config, row=True, col=True):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    R, C = x.shape
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    E = off.size - 1
    B = block_len(cfg.scaling)
    coff = grouped_col_offsets(off, B)
    R_pad = int(coff[-1])
    rc_ = np.zeros((R, C // 2), np.uint8) if row else None
    rs_ = np.zeros((R, C // B), np.uint8) if row else None
    rts = np.zeros(E, np.float32)
    cc_ = np.zeros((C, R_pad // 2), np.uint8) if col else None
    cs_ = np.zeros((C, R_pad // B), np.uint8) if col else None
    cts = np.zeros(E, np.float32)
    nul = ctypes.c_void_p(0)
    rc = lib().orc_quantize_grouped(
        _ptr(x), R, C, _ptr(off), E, ctypes.byref(cfg),
        _ptr(rc_) if row else nul, _ptr(rs_) if row else nul, _ptr(rts),
        _ptr(cc_) if col else nul, _ptr(cs_) if col else nul, _ptr(cts))
    if rc:
        raise ValueError(f"orc_quantize_grouped failed ({rc})")
    return (rc_, rs_, rts), (cc_, cs_, cts), coff


def quantize_grouped_given_amax(x_bf16: np.ndarray, offsets, cfg: Config, amax_given, row=True, col=True):
    """Grouped delayed scaling (NV16): segment e's tensor scales from
    amax_given[e] = (row-wise, column-wise) maxima.  Returns the row and
    column outputs as quantize_grouped, the column offsets, and each
    segment's own maxima [E][2]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    R, C = x.shape
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    E = off.size - 1
    B = block_len(cfg.scaling)
    coff = grouped_col_offsets(off, B)
    R_pad = int(coff[-1])
    given = np.ascontiguousarray(np.asarray(amax_given, np.float32).reshape(E, 2))
    seen = np.zeros((E, 2), np.float32)
    rc_ = np.zeros((R, C // 2), np.uint8) if row else None
    rs_ = np.zeros((R, C // B), np.uint8) if row else None
    rts = np.zeros(E, np.float32)
    cc_ = np.zeros((C, R_pad // 2), np.uint8) if col else None
    cs_ = np.zeros((C, R_pad // B), np.uint8) if col else None
    cts = np.zeros(E, np.float32)
    nul = ctypes.c_void_p(0)
    rc = lib().orc_quantize_grouped_given_amax(
        _ptr(x), R, C, _ptr(off), E, ctypes.byref(cfg), _ptr(given), _ptr(seen),
        _ptr(rc_) if row else nul, _ptr(rs_) if row else nul, _ptr(rts),
        _ptr(cc_) if col else nul, _ptr(cs_) if col else nul, _ptr(cts))
    if rc:
        raise ValueError(f"orc_quantize_grouped_given_amax failed ({rc})")
    return (rc_, rs_, rts), (cc_, cs_, cts), coff, seen


def dequantize(codes, scales, tensor_scale, rows: int, cols: int, cfg: Config,
               inverse_rht: bool = False) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    t = np.ascontiguousarray(np.atleast_1d(tensor_scale), dtype=np.float32)
    out = np.zeros((rows, cols), dtype=np.float32)
    rc = lib().orc_dequantize(_ptr(c), _ptr(s), _ptr(t), rows, cols, ctypes.byref(cfg),
                              int(bool(inverse_rht)), _ptr(out))
    if rc:
        raise ValueError(f"orc_dequantize failed ({rc})")
    return out


def stats(x_bf16, layout: int, cfg: Config, codes, scales, tensor_scale) -> dict:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    t = np.ascontiguousarray(np.atleast_1d(tensor_scale), dtype=np.float32)
    st = Stats()
    rc = lib().orc_compute_stats(_ptr(x), rows, cols, cols, int(layout), ctypes.byref(cfg),
                                 _ptr(c), _ptr(s), _ptr(t), ctypes.byref(st))
    if rc:
        raise ValueError(f"orc_compute_stats failed ({rc})")
    return st.as_dict()


def _f32_to_bf16_rne(y: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(y, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def shrinkage_chain(h0_bf16: np.ndarray, weights_bf16, cfg: Config) -> dict:
    """Compounding of the quantized-GEMM gain through a chain of linear layers
    ("Shrinkage Bias: The Hidden Geometric Trap in FP4 Training" (zhichai.net),
    "Key points", compounding decay: a quantized operand is a scaled copy plus
    an orthogonal residual, A_hat = alpha_A A + R_A, a GEMM's output is scaled
    by eta ~ alpha_A alpha_B, and the gains multiply over layers).

    Layer k: y_k = A_hat B_hat^T, the float64 product of the dequantized
    row-wise layouts of its input h_{k-1} [T][D] and weight W_k [D'][D] (the
    fwd_y GEMM; both quantized with cfg and one sign vector); its gain
    eta_k = <y_k, y*_k> / <y*_k, y*_k> against the exact product
    y*_k = h_{k-1} W_k^T of the same bf16 operands; alpha of both operands as
    ufp4 statistics define it; the next input h_k = bf16(fp32(y_k)) (round to
    nearest even twice, as a GEMM with an fp32 result feeding a bf16 layer).
    The chain's gain G_k = <h_k, x*_k> / <x*_k, x*_k> is measured against the
    unquantized chain x*_k = x*_{k-1} W_k^T, x*_0 = h_0, in float64.
    Returns lists eta, alpha_a, alpha_b, gain (one entry per layer) and the
    last input."""
    h = np.ascontiguousarray(h0_bf16, dtype=np.uint16)
    f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    xs = f64(h)
    out = {"eta": [], "alpha_a": [], "alpha_b": [], "gain": []}
    for w in weights_bf16:
        w = np.ascontiguousarray(w, dtype=np.uint16)
        T, D = h.shape
        N = w.shape[0]
        qa, qb = quantize(h, cfg, LAYOUT_ROW), quantize(w, cfg, LAYOUT_ROW)
        out["alpha_a"].append(stats(h, LAYOUT_ROW, cfg, *qa)["alpha"])
        out["alpha_b"].append(stats(w, LAYOUT_ROW, cfg, *qb)["alpha"])
        y, _ = gemm_nt_reference(qa, qb, cfg, T, N, D)
        ye = f64(h) @ f64(w).T
        out["eta"].append(float(np.sum(y * ye) / np.sum(ye * ye)))
        h = _f32_to_bf16_rne(y.astype(np.float32))
        xs = xs @ f64(w).T
        out["gain"].append(float(np.sum(f64(h) * xs) / np.sum(xs * xs)))
    out["last_input"] = h
    return out
