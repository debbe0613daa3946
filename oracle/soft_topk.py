"""Plain fp64 CPU oracle of the SLA2 SoftTop-k router mask.

TEST INFRASTRUCTURE ONLY.  It defines the expected results: only tests/, the
package entry point's smoke check and the benchmark's CPU-baseline leg may
import or run it.  It shares no code with the HIP path and imports nothing
from it.

Sources (titles of the pages and the section of each):
* "SLA2: Sparse-Linear Attention with Learnable Routing and QAT" (AI summary
  page): section 4 (for training, the router's hard Top-k is replaced by
  SoftTop-k, which keeps the row-sum constraint of Top-k and lets gradients
  flow), section 6 (SoftTop-k is a sigmoid with a temperature tau and a
  per-row offset lambda_i found by binary search so that every row sums to
  k% x N / b_k), section 7 (inference uses the hard Top-k).
* "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable
  Sparse-Linear Attention" (detailed summary page): section 2 Q2 step 1 and
  the section 3 figure (the compressed attention P_c is the row softmax of
  the pooled scores / sqrt(d)).

Readings where the pages are silent (each is listed in the design notes):
* The SoftTop-k input is P_c = softmax over each row of the router scores
  s_ij = (q_bar_i W_q).(k_bar_j W_k)/sqrt(d), the same scores the hard Top-k
  ranks (the softmax is monotone, so the hard mask is unchanged by it).
* M_ij = sigmoid((P_ij - lambda_i) / tau); the target row sum is the integer
  k_sel of the hard router.
* Binary search: the bracket is [min_j P_ij - tau (ln T + 2),
  max_j P_ij + tau (ln T + 2)].  At its lower end every term exceeds
  sigmoid(ln T + 2), so the row sum is above T - 1 >= k_sel; at its upper end
  every term is below sigmoid(-(ln T + 2)), so the sum is below 1 <= k_sel.
  Each of 60 halvings evaluates the row sum at the midpoint and keeps the
  half in which it crosses k_sel (the sum falls as lambda grows); lambda_i is
  the final midpoint.
* k_sel = T: every M_ij is 1 and lambda_i = -inf (no finite offset reaches
  the sum T).
"""
from __future__ import annotations

import numpy as np

BISECTION_STEPS = 60


def router_probs(scores: np.ndarray) -> np.ndarray:
    """P_c: softmax over each row of the block scores (fp64)."""
    s = np.asarray(scores, np.float64)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)) without overflow warnings for large |x|."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def soft_topk(P: np.ndarray, k_sel: int, tau: float, steps: int = BISECTION_STEPS):
    """SoftTop-k of each row of P [rows, T]: returns (M [rows, T], lambda [rows]).

    M_ij = sigmoid((P_ij - lambda_i) / tau) with lambda_i from the binary search
    described in the module notes.
    """
    P = np.asarray(P, np.float64)
    rows, T = P.shape
    if not 1 <= k_sel <= T:
        raise ValueError("k_sel out of range")
    if not tau > 0:
        raise ValueError("tau must be positive")
    if k_sel == T:
        return np.ones_like(P), np.full(rows, -np.inf)
    pad = tau * (np.log(T) + 2.0)
    lo = P.min(axis=1) - pad
    hi = P.max(axis=1) + pad
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        total = sigmoid((P - mid[:, None]) / tau).sum(axis=1)
        above = total > k_sel          # sum too large: the offset must grow
        lo = np.where(above, mid, lo)
        hi = np.where(above, hi, mid)
    lam = 0.5 * (lo + hi)
    return sigmoid((P - lam[:, None]) / tau), lam


def soft_route_head(scores: np.ndarray, k_sel: int, tau: float):
    """SoftTop-k mask of one head from its block scores: (P_c, M, lambda)."""
    P = router_probs(scores)
    M, lam = soft_topk(P, k_sel, tau)
    return P, M, lam
