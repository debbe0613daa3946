"""Pins of the SoftTop-k oracle against what the pages and the mathematics fix.

SLA2 page, section 6: SoftTop-k is sigmoid((P - lambda_i) / tau) with lambda_i
found by binary search so that each row sums to the Top-k count.  SLA2 page,
sections 4 and 7: it stands in for the hard Top-k during training, so it must
approach the hard mask as tau -> 0.  The checks below use closed forms, an
independent root finder and limits, never the oracle's own arithmetic.
"""
import math

import numpy as np
import pytest
from scipy.optimize import brentq

from oracle import soft_topk as S
from oracle import sla2_oracle as O


def _rows(rows, T, seed):
    rng = np.random.default_rng(seed)
    return S.router_probs(rng.standard_normal((rows, T)) * 3.0)


@pytest.mark.parametrize("tau", [0.3, 0.05, 0.002])
@pytest.mark.parametrize("k_sel", [1, 4, 15])
def test_rows_sum_to_k(tau, k_sel):
    P = _rows(8, 32, seed=11)
    M, lam = S.soft_topk(P, k_sel, tau)
    assert np.all(np.abs(M.sum(axis=1) - k_sel) < 1e-9)
    assert np.all((M >= 0) & (M <= 1))


def test_uniform_row_closed_form():
    # all P equal: every M_ij = k/T, and sigmoid((p - lambda)/tau) = k/T gives
    # lambda = p - tau * ln(k / (T - k))
    T, k, tau = 40, 7, 0.01
    P = np.full((1, T), 1.0 / T)
    M, lam = S.soft_topk(P, k, tau)
    assert np.max(np.abs(M - k / T)) < 1e-12
    assert abs(lam[0] - (1.0 / T - tau * math.log(k / (T - k)))) < 1e-12


def test_two_level_row_closed_form():
    # a entries at value u, T - a at value w: the row sum a s(u) + (T - a) s(w) = k is
    # solved exactly for the sigmoid argument when tau is large enough for both terms;
    # check the oracle's lambda satisfies the defining equation to rounding
    T, a, k, tau = 24, 6, 9, 0.05
    P = np.array([[0.2] * a + [0.8 / (T - a)] * (T - a)])
    M, lam = S.soft_topk(P, k, tau)
    u, w = P[0, 0], P[0, -1]
    f = a / (1 + math.exp(-(u - lam[0]) / tau)) + (T - a) / (1 + math.exp(-(w - lam[0]) / tau))
    assert abs(f - k) < 1e-9


def test_lambda_matches_an_independent_root_finder():
    P = _rows(6, 64, seed=5)
    tau, k = 0.02, 5
    _, lam = S.soft_topk(P, k, tau)
    for r in range(P.shape[0]):
        f = lambda x: sum(1.0 / (1.0 + math.exp(-(p - x) / tau)) if (p - x) / tau > -700 else 0.0
                          for p in P[r]) - k
        pad = tau * (math.log(64) + 2.0)
        ref = brentq(f, P[r].min() - pad, P[r].max() + pad, xtol=1e-15, rtol=1e-15, maxiter=500)
        assert abs(lam[r] - ref) < 1e-12 * max(1.0, abs(ref))


def test_small_tau_gives_the_hard_topk_mask():
    rng = np.random.default_rng(3)
    scores = rng.standard_normal((10, 48))
    k = 6
    _, hard = O.topk_blocks(scores, k)
    P = S.router_probs(scores)
    srt = np.sort(P, axis=1)[:, ::-1]
    gap = np.min(srt[:, k - 1] - srt[:, k])
    M, _ = S.soft_topk(P, k, tau=gap * 1e-3)
    assert np.max(np.abs(M - hard)) < 1e-6


def test_shift_invariance_and_order():
    P = _rows(4, 30, seed=9)
    tau, k = 0.05, 4
    M, lam = S.soft_topk(P, k, tau)
    M2, lam2 = S.soft_topk(P + 0.37, k, tau)
    assert np.max(np.abs(M - M2)) < 1e-12
    assert np.max(np.abs(lam2 - lam - 0.37)) < 1e-12
    for r in range(P.shape[0]):
        order = np.argsort(P[r], kind="stable")
        assert np.all(np.diff(M[r][order]) >= -1e-15)


def test_all_blocks_routed():
    P = _rows(3, 16, seed=1)
    M, lam = S.soft_topk(P, 16, 0.1)
    assert np.all(M == 1.0) and np.all(np.isneginf(lam))


def test_router_probs_is_a_row_softmax():
    s = np.array([[0.0, math.log(3.0)], [5.0, 5.0]])
    P = S.router_probs(s)
    assert np.allclose(P, [[0.25, 0.75], [0.5, 0.5]], atol=1e-15)
