"""Pins of the backward oracle: central finite differences of the forward oracle.

The loss is L = sum(dO * O) with the routing held fixed (the mask is constant,
SLA2 page, appendix A; the router gets no gradient).  Each check perturbs single
input elements of a tiny head (three blocks, the last one partial) by +-h and
compares (L+ - L-)/2h with the oracle's gradient.  FP8 mode: V and alpha enter
the forward smoothly, so their gradients are still exact; for Q and K the
straight-through quantiser is pinned on inputs the quantiser reproduces
exactly (then FP8 and native gradients must coincide).
"""
import numpy as np
import pytest

from oracle import sla2_backward as BW
from oracle import sla2_oracle as O
from oracle import fp8_e4m3 as F8


def _head(N=150, d=8, seed=0):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((N, d)).astype(np.float32) for _ in range(4))
    alpha = rng.uniform(0.3, 0.9, d)
    return q, k, v, do, alpha


def _loss(q, k, v, alpha, do, lut, smooth_k, qk_fp8=False):
    fw = O.forward_head(q, k, v, alpha, topk=lut.shape[1], smooth_k=smooth_k, qk_fp8=qk_fp8, lut=lut)
    return float((np.asarray(do, np.float64) * fw["o"]).sum())


def _fd(which, idx, q, k, v, alpha, do, lut, smooth_k, h=1e-4, qk_fp8=False):
    args = {"q": q.astype(np.float64), "k": k.astype(np.float64), "v": v.astype(np.float64),
            "alpha": np.array(alpha, np.float64)}
    plus = {kk: vv.copy() for kk, vv in args.items()}
    minus = {kk: vv.copy() for kk, vv in args.items()}
    plus[which][idx] += h
    minus[which][idx] -= h
    lp = _loss(plus["q"], plus["k"], plus["v"], plus["alpha"], do, lut, smooth_k, qk_fp8)
    lm = _loss(minus["q"], minus["k"], minus["v"], minus["alpha"], do, lut, smooth_k, qk_fp8)
    return (lp - lm) / (2 * h)


LUTS = [np.array([[0], [2], [1]]), np.array([[0, 2], [1, 2], [0, 1]]), np.array([[0, 1, 2]] * 3)]


@pytest.mark.parametrize("smooth_k", [True, False])
@pytest.mark.parametrize("lut_id", [0, 1, 2])
def test_gradients_match_finite_differences(smooth_k, lut_id):
    # float64 inputs through the float32-typed oracle: keep values exactly representable
    q, k, v, do, alpha = _head(seed=lut_id + 3 * smooth_k)
    lut = LUTS[lut_id]
    g = BW.backward_head(q, k, v, alpha, do, lut, smooth_k=smooth_k)
    rng = np.random.default_rng(7)
    for which, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        for _ in range(12):
            idx = (int(rng.integers(q.shape[0])), int(rng.integers(q.shape[1])))
            # perturb in float32 steps: the forward oracle reads float32 inputs
            num = _fd32(which, idx, q, k, v, alpha, do, lut, smooth_k)
            assert abs(num - grad[idx]) < 2e-3 * (1 + abs(grad[idx])), (which, idx, num, grad[idx])
    for c in range(q.shape[1]):
        num = _fd("alpha", c, q, k, v, alpha, do, lut, smooth_k, h=1e-6)
        assert abs(num - g["dalpha"][c]) < 1e-6 * (1 + abs(num)), (c, num, g["dalpha"][c])


def _fd32(which, idx, q, k, v, alpha, do, lut, smooth_k, qk_fp8=False):
    """Central difference with a float32-representable step (the forward reads float32)."""
    base = {"q": q, "k": k, "v": v}
    x = base[which]
    h = np.float32(2.0 ** -9) * max(np.float32(1.0), abs(x[idx]))
    plus = {kk: vv.copy() for kk, vv in base.items()}
    minus = {kk: vv.copy() for kk, vv in base.items()}
    plus[which][idx] = np.float32(x[idx] + h)
    minus[which][idx] = np.float32(x[idx] - h)
    step = float(plus[which][idx]) - float(minus[which][idx])
    lp = _loss(plus["q"], plus["k"], plus["v"], alpha, do, lut, smooth_k, qk_fp8)
    lm = _loss(minus["q"], minus["k"], minus["v"], alpha, do, lut, smooth_k, qk_fp8)
    return (lp - lm) / step


def test_fp8_value_and_alpha_gradients_are_exact():
    q, k, v, do, alpha = _head(seed=21)
    lut = LUTS[1]
    g = BW.backward_head(q, k, v, alpha, do, lut, smooth_k=True, qk_fp8=True)
    rng = np.random.default_rng(8)
    for _ in range(12):
        idx = (int(rng.integers(q.shape[0])), int(rng.integers(q.shape[1])))
        num = _fd32("v", idx, q, k, v, alpha, do, lut, True, qk_fp8=True)
        assert abs(num - g["dv"][idx]) < 2e-3 * (1 + abs(g["dv"][idx]))
    for c in range(q.shape[1]):
        num = _fd("alpha", c, q, k, v, alpha, do, lut, True, h=1e-6, qk_fp8=True)
        assert abs(num - g["dalpha"][c]) < 1e-6 * (1 + abs(num))


def test_fp8_straight_through_on_exactly_quantised_inputs():
    # inputs on the e4m3 grid times 2^-6, each block holding +-448 * 2^-6: the quantiser
    # returns them unchanged, so the FP8 forward equals the native one and the
    # straight-through gradients must equal the native (finite-difference-pinned) ones
    rng = np.random.default_rng(5)
    grid = F8.decode(np.arange(256, dtype=np.uint8))
    grid = grid[np.isfinite(grid) & (np.abs(grid) <= 16)]
    N, d = 150, 8
    def on_grid():
        x = rng.choice(grid, size=(N, d)).astype(np.float32) * np.float32(2.0 ** -6)
        for j in range(3):
            x[64 * j, 0] = np.float32(448.0 * 2.0 ** -6)
        return x
    q, k = on_grid(), on_grid()
    v = rng.standard_normal((N, d)).astype(np.float32)
    do = rng.standard_normal((N, d)).astype(np.float32)
    alpha = rng.uniform(0.3, 0.9, d)
    lut = LUTS[1]
    g8 = BW.backward_head(q, k, v, alpha, do, lut, smooth_k=False, qk_fp8=True)
    gn = BW.backward_head(q, k, v, alpha, do, lut, smooth_k=False, qk_fp8=False)
    assert np.allclose(g8["fw"]["o"], gn["fw"]["o"], rtol=0, atol=1e-12)
    for key in ("dq", "dk", "dv", "dalpha"):
        assert np.allclose(g8[key], gn[key], rtol=1e-12, atol=1e-12), key


def test_all_routed_alpha_one_is_softmax_attention_backward():
    # every block routed and alpha = 1: the gradients are those of exact softmax attention,
    # written out here with per-query loops
    q, k, v, do, _ = _head(N=130, d=4, seed=9)
    lut = np.array([[0, 1, 2]] * 3)
    g = BW.backward_head(q, k, v, np.ones(4), do, lut, smooth_k=False)
    N, d = q.shape
    Q, K, V, dO = (x.astype(np.float64) for x in (q, k, v, do))
    dq = np.zeros((N, d)); dk = np.zeros((N, d)); dv = np.zeros((N, d))
    for t in range(N):
        s = np.array([Q[t] @ K[u] for u in range(N)]) / np.sqrt(d)
        p = np.exp(s - s.max()); p /= p.sum()
        o = sum(p[u] * V[u] for u in range(N))
        dp = np.array([dO[t] @ V[u] for u in range(N)])
        ds = p * (dp - dO[t] @ o)
        for u in range(N):
            dq[t] += ds[u] * K[u] / np.sqrt(d)
            dk[u] += ds[u] * Q[t] / np.sqrt(d)
            dv[u] += p[u] * dO[t]
    assert np.allclose(g["dq"], dq, atol=1e-12)
    assert np.allclose(g["dk"], dk, atol=1e-12)
    assert np.allclose(g["dv"], dv, atol=1e-12)
