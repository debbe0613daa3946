"""Seeded synthetic workloads for the SLA2 forward pass.

This module only draws and rounds input data; it holds none of the method's
arithmetic (no pooling, routing, quantisation, softmax or mixing).  Both the
CPU oracle's tests and the GPU path read their inputs from here, so the two
sides always see the same bytes.

Workload recipe (see the repository's design notes for the reasoning):

* ``numpy.random.Generator(PCG64(seed))``, float32 draws, in the fixed order
  noise_q, noise_k, V, alpha, W_q, W_k (and dO when asked for).
* Structured workloads stand in for Wan2.1 video-DiT self-attention
  activations on a (T, H, W) latent grid, token n = (t*H + y)*W + x.  Q and K
  are a smooth 3D sinusoidal positional embedding plus 0.5*N(0,1) noise, so
  attention is locally peaked; V ~ N(0,1).
* Unstructured workloads use Q, K, V ~ N(0,1).
* alpha ~ U(0.3, 0.9) per (head, feature); W_q, W_k ~ N(0, 1/d) or absent
  (identity projections).
* bf16 workloads are rounded once to bf16 (round to nearest even); the
  float32 arrays returned hold exactly the bf16 values.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "make_workload", "generate", "round_to_bf16",
    "bf16_bits", "topk_from_fraction", "sinusoidal_pe_3d", "sha256",
]


def topk_from_fraction(frac: float, T: int) -> int:
    """Routed key blocks per query row for a sparse share ``frac`` of T blocks.

    The SLA2 page (section 6, SoftTop-k) fixes each row's sum at k% x N/b_k,
    which is not an integer for N = 32760; this build rounds half up and keeps
    at least one block: max(1, floor(frac*T + 0.5)).
    """
    return max(1, min(T, int(math.floor(frac * T + 0.5))))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str              # "f32" or "bf16": element type of Q, K, V, O
    qk_mode: str            # "native", "fp8" (e4m3 Q.K^T) or "fp8pv" (e4m3 Q.K^T and P.V)
    sparse_frac: float      # share of key blocks routed to the sparse branch
    projections: bool       # seeded d x d router projections (else identity)
    seed: int
    grid: Optional[Tuple[int, int, int]] = None   # (T, H, W) latent grid, None = unstructured
    block: int = 64

    @property
    def T(self) -> int:
        return (self.N + self.block - 1) // self.block

    @property
    def topk(self) -> int:
        return topk_from_fraction(self.sparse_frac, self.T)


# The five workloads of the benchmark description, 0-based.
CONFIGS = {
    "C0": Workload("C0 tiny fp32 plumbing", 1, 2, 1024, 64, "f32", "native", 0.25, False, 0, None),
    "C1": Workload("C1 Wan2.1-1.3B-shaped, bf16, 5% sparse", 1, 12, 32760, 128, "bf16", "native",
                   0.05, False, 1, (21, 30, 52)),
    "C2": Workload("C2 Wan2.1-1.3B-shaped, fp8 QK, 3% sparse", 1, 12, 32760, 128, "bf16", "fp8",
                   0.03, True, 2, (21, 30, 52)),
    "C3": Workload("C3 Wan2.1-14B-720P-shaped, fp8 QK, 3% sparse", 1, 40, 75600, 128, "bf16", "fp8",
                   0.03, True, 3, (21, 45, 80)),
    # fine-tuning step on the C1 shape: FP8 (QAT) forward, then the backward against dO ~ N(0,1)
    "C4": Workload("C4 Wan2.1-1.3B-shaped fine-tuning step, fp8 QK (QAT), 5% sparse", 1, 12, 32760, 128,
                   "bf16", "fp8", 0.05, False, 4, (21, 30, 52)),
}


def make_workload(base: str, *, grid=None, N=None, H=None, B=None, seed=None, name=None,
                  sparse_frac=None, dtype=None, qk_mode=None, projections=None, d=None) -> Workload:
    """A reduced or varied copy of one of the named workloads."""
    w = CONFIGS[base]
    kw = {}
    if grid is not None:
        kw["grid"] = tuple(grid)
        kw["N"] = int(np.prod(grid))
    if N is not None:
        kw["N"] = N
        if grid is None and w.grid is not None and N != w.N:
            kw["grid"] = None
    for key, val in (("H", H), ("B", B), ("seed", seed), ("sparse_frac", sparse_frac),
                     ("dtype", dtype), ("qk_mode", qk_mode), ("projections", projections),
                     ("d", d)):
        if val is not None:
            kw[key] = val
    kw["name"] = name or (w.name + " (varied)")
    return dataclasses.replace(w, **kw)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns (uint16) of float32 values that are already bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def sinusoidal_pe_3d(grid: Tuple[int, int, int], d: int) -> np.ndarray:
    """Smooth 3D sinusoidal positional embedding, shape [T*H*W, d], float64.

    The d features are split into contiguous groups for the t, y and x axes
    (sizes d - 2*g, g, g with g = 2*round(d/6)); within a group of m features
    on an axis of length L, pair f = 0..m/2-1 uses wavelength 4*L**(f/(m/2-1))
    (4 tokens up to 4L) and holds (sin, cos) of position*2*pi/wavelength.
    """
    Tg, Hg, Wg = grid
    g = 2 * int(round(d / 6.0))
    sizes = (d - 2 * g, g, g)
    t = np.arange(Tg).repeat(Hg * Wg)
    y = np.tile(np.arange(Hg).repeat(Wg), Tg)
    x = np.tile(np.arange(Wg), Tg * Hg)
    pe = np.empty((Tg * Hg * Wg, d), dtype=np.float64)
    col = 0
    for pos, L, m in ((t, Tg, sizes[0]), (y, Hg, sizes[1]), (x, Wg, sizes[2])):
        half = m // 2
        for f in range(half):
            expo = f / (half - 1) if half > 1 else 0.0
            lam = 4.0 * (float(L) ** expo)
            w = 2.0 * np.pi / lam
            pe[:, col + 2 * f] = np.sin(pos * w)
            pe[:, col + 2 * f + 1] = np.cos(pos * w)
        col += m
    return pe


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def generate(w: Workload, with_dout: bool = False) -> dict:
    """Draw one workload's inputs.

    Returns float32 arrays q, k, v [B,H,N,d] (bf16-exact for bf16 workloads),
    alpha [H,d], wq, wk [d,d] (or None), and dout [B,H,N,d] if asked.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.B, w.H, w.N, w.d)
    noise_q = rng.standard_normal(shape, dtype=np.float32)
    noise_k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    alpha = rng.uniform(0.3, 0.9, size=(w.H, w.d)).astype(np.float32)
    wq = wk = None
    if w.projections:
        std = np.float32(1.0 / math.sqrt(w.d))
        wq = (rng.standard_normal((w.d, w.d), dtype=np.float32) * std).astype(np.float32)
        wk = (rng.standard_normal((w.d, w.d), dtype=np.float32) * std).astype(np.float32)
    dout = rng.standard_normal(shape, dtype=np.float32) if with_dout else None

    if w.grid is not None:
        pe = sinusoidal_pe_3d(w.grid, w.d).astype(np.float32)
        q = pe + np.float32(0.5) * noise_q
        k = pe + np.float32(0.5) * noise_k
    else:
        q, k = noise_q, noise_k
    del noise_q, noise_k
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
        if dout is not None:
            dout = round_to_bf16(dout)
    out = {"q": np.ascontiguousarray(q, np.float32), "k": np.ascontiguousarray(k, np.float32),
           "v": np.ascontiguousarray(v, np.float32), "alpha": alpha, "wq": wq, "wk": wk}
    if dout is not None:
        out["dout"] = dout
    return out
