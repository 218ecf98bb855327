"""Compounding of the quantized-GEMM gain through a chain of linear layers.

"Shrinkage Bias: The Hidden Geometric Trap in FP4 Training" (zhichai.net),
"Key points", compounding decay: a quantized operand is a scaled copy of the
original plus an orthogonal residual, A_hat = alpha_A A + R_A, so a GEMM of two
quantized operands scales its output by eta ~ alpha_A alpha_B, and over K
layers the gains multiply, prod eta_k ~ exp(-sum delta_k) with
delta_k = 1 - eta_k.  A grid whose rounding shrinks magnitudes (E2M1) makes
every eta_k < 1; a uniform grid (E1M2, INT4) keeps it at 1 on average.

Layer k quantizes its bf16 input h_{k-1} [T][D] and weight W_k [N][D]
row-wise (blocks along D) with the library, multiplies them with
ufp4_gemm_nt (the fwd_y GEMM) and rounds the fp32 result to bf16 with
ufp4_f32_to_bf16 for the next layer.  Every one of these steps runs in the
library's kernels.  The measurement around them compares with exact
products: eta_k = <y_k, y*_k> / <y*_k, y*_k> against y*_k = h_{k-1} W_k^T
of the same bf16 operands, and the chain's gain G_k = <h_k, x*_k> /
<x*_k, x*_k> against the unquantized chain x*_k = x*_{k-1} W_k^T,
x*_0 = h_0; those references are float64 matrix products (torch), and alpha
of both operands comes from ufp4_stats.
"""
from __future__ import annotations

import torch

from . import (SCALE_NV16, Workspace, alloc_layout, ufp4_f32_to_bf16, ufp4_gemm_nt, ufp4_quantize,
               ufp4_stats)


def bf16_bits_to_f64(h: torch.Tensor) -> torch.Tensor:
    """float64 values of bf16 bit patterns held in an int16 tensor."""
    return ((h.to(torch.int32) & 0xFFFF) << 16).view(torch.float32).to(torch.float64)


def shrinkage_chain(h0: torch.Tensor, weights, cfg, stream=None) -> dict:
    """Run the chain on the device.  h0: int16 bf16 patterns [T][D]; weights:
    int16 bf16 patterns [N][D] each, with the input width of one layer equal
    to the output width of the one before; D a multiple of 32 and T, N of 16
    for the quantizer.  cfg must use NV16 scales.  Returns lists eta,
    alpha_a, alpha_b, gain (one entry per layer) and the last input."""
    if cfg.scaling != SCALE_NV16:
        raise ValueError("the chain multiplies NV16 layouts")
    h = h0.contiguous()
    xs = bf16_bits_to_f64(h)
    out = {"eta": [], "alpha_a": [], "alpha_b": [], "gain": []}
    for w in weights:
        w = w.contiguous()
        T, D = h.shape
        N, Dw = w.shape
        if Dw != D:
            raise ValueError(f"layer input width {D} != weight width {Dw}")
        ws = Workspace(max(T, N), D, device=h.device)
        qa = alloc_layout(T, D, SCALE_NV16, device=h.device)
        qb = alloc_layout(N, D, SCALE_NV16, device=h.device)
        ufp4_quantize(h, cfg, qa, ws, stream)
        out["alpha_a"].append(ufp4_stats(h, 0, cfg, qa, ws, stream)["alpha"])
        ufp4_quantize(w, cfg, qb, ws, stream)
        out["alpha_b"].append(ufp4_stats(w, 0, cfg, qb, ws, stream)["alpha"])
        y = torch.empty((T, N), dtype=torch.float32, device=h.device)
        ufp4_gemm_nt(cfg, qa, qb, T, N, D, y, stream)
        wf = bf16_bits_to_f64(w).t().contiguous()
        ye = bf16_bits_to_f64(h) @ wf
        out["eta"].append(float((y.to(torch.float64) * ye).sum() / (ye * ye).sum()))
        h = ufp4_f32_to_bf16(y, stream=stream)
        xs = xs @ wf
        out["gain"].append(float((bf16_bits_to_f64(h) * xs).sum() / (xs * xs).sum()))
    out["last_input"] = h
    return out
