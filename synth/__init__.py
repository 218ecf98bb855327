"""Seeded synthetic inputs for the UFP4 quantization workloads.

This module only draws random numbers and rounds them to bf16; it holds none
of the quantization method's arithmetic.  Both the CPU oracle tests and the
GPU path (tests, smoke check, benchmark) take their inputs from here.

Every generator uses ``numpy.random.Generator(PCG64(seed))`` and a fixed
order of draws, so a (workload, seed) pair always yields the same tensor on
any machine.  fp32 -> bf16 conversion is round-to-nearest-even on the bit
pattern.  The pages measure on model tensors and training runs that are not
available; these distributions stand in for them:

* activations: N(0, 1) plus a per-channel mean bias N(0, 0.5) (variance 0.5)
  and a few channels scaled x50 -- the coherent-mean outliers the pages
  describe for activations;
* weights: N(0, 0.02^2) with Student-t(4) tails;
* output gradients: Laplace(0, 1e-3) with 0.01% of entries x100;
* MoE: activation-like rows grouped by expert, with ragged per-expert counts
  from top-8 routing over 64 experts under Zipf(1.1) popularity.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = ["f32_to_bf16", "bf16_to_f32", "activation", "weight", "output_grad",
           "moe_counts", "moe_activation", "orthogonal", "tiny", "all_bf16_patterns", "Workload",
           "workload", "sha256"]


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 22
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        nan = (v & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        # finite patterns stay below 2^32 after adding the rounding bias
        r = (np.where(nan, np.uint32(0), v) + np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        r = np.where(nan, (v >> np.uint32(16)) | np.uint32(0x40), r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def activation(rows: int, cols: int, seed: int, bias_var: float = 0.5,
               outlier_frac: float = 0.001, outlier_scale: float = 50.0,
               n_outlier_cols: int | None = None) -> np.ndarray:
    """N(0,1) + per-column bias N(0, bias_var); round(outlier_frac*cols) distinct
    seeded columns (at least one when outlier_frac > 0) scaled by outlier_scale
    after the bias is added.  Draw order: column bias, outlier columns, then the
    matrix row-block by row-block."""
    rng = _rng(seed)
    bias = (rng.standard_normal(cols) * np.sqrt(bias_var)).astype(np.float32)
    if n_outlier_cols is None:
        n_outlier_cols = max(1, int(round(outlier_frac * cols))) if outlier_frac > 0 else 0
    ocols = rng.choice(cols, size=n_outlier_cols, replace=False) if n_outlier_cols else np.zeros(0, np.int64)
    colscale = np.ones(cols, dtype=np.float32)
    colscale[ocols] = outlier_scale
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, (1 << 22) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        out[r0:r1] = f32_to_bf16((z + bias) * colscale)
    return out


def tiny(seed: int = 0, rows: int = 256, cols: int = 256) -> np.ndarray:
    """N(0,1) entries with 8 seeded distinct columns scaled x20."""
    rng = _rng(seed)
    ocols = rng.choice(cols, size=min(8, cols), replace=False)
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    z[:, ocols] *= 20.0
    return f32_to_bf16(z)


def weight(rows: int, cols: int, seed: int, sigma: float = 0.02, nu: float = 4.0) -> np.ndarray:
    """sigma * T / sqrt(nu/(nu-2)), T ~ Student-t(nu): standard deviation sigma."""
    rng = _rng(seed)
    out = np.empty((rows, cols), dtype=np.uint16)
    k = np.float32(sigma / np.sqrt(nu / (nu - 2.0)))
    step = max(1, (1 << 22) // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        t = rng.standard_t(nu, size=(r1 - r0, cols)).astype(np.float32)
        out[r0:r1] = f32_to_bf16(t * k)
    return out


def output_grad(rows: int, cols: int, seed: int, b: float = 1e-3, outlier_frac: float = 1e-4,
                outlier_scale: float = 100.0) -> np.ndarray:
    """Laplace(0, b); round(outlier_frac * N) distinct seeded entries scaled."""
    rng = _rng(seed)
    n = rows * cols
    n_out = int(round(outlier_frac * n))
    idx = rng.choice(n, size=n_out, replace=False) if n_out else np.zeros(0, np.int64)
    f = np.empty(n, dtype=np.float32)
    step = 1 << 22
    for s in range(0, n, step):
        e = min(n, s + step)
        f[s:e] = rng.laplace(0.0, b, size=e - s).astype(np.float32)
    f[idx] *= np.float32(outlier_scale)
    return f32_to_bf16(f).reshape(rows, cols)


def moe_counts(tokens: int, experts: int, top_k: int, seed: int, zipf_s: float = 1.1) -> np.ndarray:
    """Per-expert row counts of top-k routing: each token picks top_k distinct
    experts by weighted sampling without replacement, p_e ~ rank_e^-s with the
    ranks a seeded permutation (Gumbel-top-k, which draws the same distribution
    as successive weighted sampling)."""
    rng = _rng(seed)
    ranks = rng.permutation(experts) + 1
    logp = -zipf_s * np.log(ranks.astype(np.float64))
    counts = np.zeros(experts, dtype=np.int64)
    step = 4096
    for t0 in range(0, tokens, step):
        t1 = min(tokens, t0 + step)
        g = rng.gumbel(size=(t1 - t0, experts))
        choice = np.argpartition(-(logp[None, :] + g), top_k - 1, axis=1)[:, :top_k]
        counts += np.bincount(choice.reshape(-1), minlength=experts)
    return counts


def moe_activation(tokens: int, hidden: int, experts: int, top_k: int, seed: int):
    """Rows grouped by expert: returns (x [tokens*top_k][hidden] bf16, offsets[E+1])."""
    counts = moe_counts(tokens, experts, top_k, seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = activation(int(offsets[-1]), hidden, seed + 1000)
    return x, offsets


def orthogonal(n: int, seed: int) -> np.ndarray:
    """A seeded random orthogonal n x n matrix (Q of the QR factorisation of a
    standard normal matrix, column signs fixed by R's diagonal) as bf16
    patterns: weights under which a chain of layers keeps its energy."""
    g = _rng(seed).standard_normal((n, n))
    q, r = np.linalg.qr(g)
    return f32_to_bf16((q * np.sign(np.diag(r))).astype(np.float32))


def all_bf16_patterns() -> np.ndarray:
    """Every 16-bit pattern once, widened to fp32 (exact)."""
    return bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))


@dataclass
class Workload:
    name: str
    x: np.ndarray
    offsets: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def workload(name: str, scale: int = 1) -> Workload:
    """The five named workloads at full size (scale=1) or with the row count
    divided by `scale` (for quick checks).  Data seed = workload index - 1."""
    if name == "tiny":
        return Workload(name, tiny(0), meta={"seed": 0, "shape": [256, 256]})
    if name == "activation":
        r = 8192 // scale
        return Workload(name, activation(r, 2048, 1), meta={"seed": 1, "shape": [r, 2048]})
    if name == "weight":
        r = 2048 // scale
        return Workload(name, weight(r, 8192, 2), meta={"seed": 2, "shape": [r, 8192]})
    if name == "output_grad":
        r = 16384 // scale
        return Workload(name, output_grad(r, 4096, 3), meta={"seed": 3, "shape": [r, 4096]})
    if name == "moe":
        t = 8192 // scale
        x, off = moe_activation(t, 4096, 64, 8, 4)
        return Workload(name, x, offsets=off, meta={"seed": 4, "shape": list(x.shape), "experts": 64})
    raise KeyError(name)
