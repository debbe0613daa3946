"""Work accounting of the SLA2 forward pass: FLOPs and algorithmic bytes.

Counts what the method must compute, not what dense attention would:
* sparse branch: Q.K^T and P.V over each routed (query block, key block)
  pair, 2*n_i*n_j*d multiply-adds each, i.e. 4*d*n_i*n_j FLOPs per pair
  (n_i, n_j = valid tokens of the two blocks);
* linear branch: phi(K)^T V over every key block (2*N*d^2) plus phi(Q) H_i
  over every query (2*N*d^2), so 4*N*d^2 per (batch, head);
* dense attention: 4*N^2*d per (batch, head).
With 3% of 512 key blocks rounded to 15 and the linear branch at 4*N*d^2,
the saving at N = 32760, d = 128 is 96.68%.  That matches the roughly 96.7%
saving the SLA2 page reports at 97% sparsity once the linear branch is
counted (SLA2 page, section 1).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


def block_sizes(N: int, block: int = BLOCK) -> np.ndarray:
    T = (N + block - 1) // block
    n = np.full(T, block, dtype=np.int64)
    n[-1] = N - block * (T - 1)
    return n


def sparse_flops_from_lut(lut: np.ndarray, N: int, d: int, block: int = BLOCK) -> int:
    """Exact routed-block FLOPs for a LUT of shape [..., T, topk]."""
    n = block_sizes(N, block)
    lut = np.asarray(lut).reshape(-1, lut.shape[-2], lut.shape[-1])
    tot = 0
    for row in lut:
        tot += int((n[:, None] * n[row]).sum())
    return 4 * d * tot


def sparse_flops_nominal(B: int, H: int, N: int, d: int, topk: int, block: int = BLOCK) -> int:
    """Routed-block FLOPs counting every block as full (block x block)."""
    T = (N + block - 1) // block
    return 4 * d * block * block * B * H * T * topk


def linear_flops(B: int, H: int, N: int, d: int) -> int:
    return 4 * B * H * N * d * d


def dense_flops(B: int, H: int, N: int, d: int) -> int:
    return 4 * B * H * N * N * d


def effective_flops(B: int, H: int, N: int, d: int, topk: int, lut=None) -> int:
    sp = sparse_flops_from_lut(lut, N, d) if lut is not None else sparse_flops_nominal(B, H, N, d, topk)
    return sp + linear_flops(B, H, N, d)


def computation_saving(B: int, H: int, N: int, d: int, topk: int) -> float:
    return 1.0 - effective_flops(B, H, N, d, topk) / dense_flops(B, H, N, d)
