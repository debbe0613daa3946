"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check uses an independent brute-force routine written here with plain
Python loops on tiny inputs (never the oracle's own code), or an exact
identity the pages state:
* SLA page, section 4 (boundary cases): routing every block to the sparse
  branch gives FlashAttention, i.e. exact softmax attention.
* SLA page, section 4 (linear re-association) and SLA2 page, section 3 (the
  linear branch computes K^T V over the M = 0 positions, then multiplies by
  phi(Q)): the blockwise linear branch equals the token-level direct sum.
* SLA page, section 2 Q2 (P = P*M + P*(1-M)) and SLA2 page, section 1 (the
  learnable ratio matches the direct decomposition): with the ideal per-row
  ratio the mixed output equals full attention.
* SLA2 page, section 4: Top-k keeps the k highest scores of each row; the
  compressed mask and the LUT describe the same sets.
"""
import math

import numpy as np
import pytest

from oracle import sla2_oracle as O
from oracle import fp8_e4m3 as F8


def _rand(N, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal((N, d)) * scale).astype(np.float32) for _ in range(3)]


# ---------------------------------------------------------------- brute force
def bf_softmax_attention(q, k, v, keys_of_row, scale):
    """Loop softmax attention: row t attends to the key indices keys_of_row(t)."""
    N, d = q.shape
    out = np.zeros((N, v.shape[1]))
    for t in range(N):
        keys = keys_of_row(t)
        logits = []
        for s in keys:
            acc = 0.0
            for c in range(d):
                acc += float(q[t, c]) * float(k[s, c])
            logits.append(acc * scale)
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        tot = sum(w)
        for s, ws in zip(keys, w):
            out[t] += (ws / tot) * v[s].astype(np.float64)
    return out


def bf_feature_softmax(row):
    m = max(float(x) for x in row)
    e = [math.exp(float(x) - m) for x in row]
    s = sum(e)
    return [x / s for x in e]


def bf_mean_rows(x, lo, hi):
    d = x.shape[1]
    return [sum(float(x[t, c]) for t in range(lo, hi)) / (hi - lo) for c in range(d)]


def bf_decode_e4m3(code):
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 10)


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("smooth_k", [True, False])
@pytest.mark.parametrize("N,d", [(150, 8), (64, 4), (200, 16)])
def test_all_sparse_alpha_one_is_exact_softmax_attention(N, d, smooth_k):
    q, k, v = _rand(N, d, 11 + N + d)
    T = O.num_blocks(N)
    alpha = np.ones(d, np.float32)
    res = O.forward_head(q, k, v, alpha, topk=T, smooth_k=smooth_k)
    ref = bf_softmax_attention(q, k, v, lambda t: range(N), 1.0 / math.sqrt(d))
    assert np.max(np.abs(res["o"] - ref)) < 1e-12


def test_all_sparse_fp8_is_softmax_attention_on_dequantised_operands():
    N, d = 130, 8
    q, k, v = _rand(N, d, 5, scale=3.0)
    T = O.num_blocks(N)
    res = O.forward_head(q, k, v, np.ones(d, np.float32), topk=T, smooth_k=True, qk_fp8=True)
    # dequantise with the test's own bit-field decoder
    dq = np.array([[bf_decode_e4m3(int(c)) for c in row] for row in res["q8"]])
    dk = np.array([[bf_decode_e4m3(int(c)) for c in row] for row in res["k8"]])
    for j in range(T):
        r = slice(64 * j, min(64 * j + 64, N))
        dq[r] *= float(res["q_scale"][j])
        dk[r] *= float(res["k_scale"][j])
    ref = bf_softmax_attention(dq, dk, v, lambda t: range(N), 1.0 / math.sqrt(d))
    assert np.max(np.abs(res["o"] - ref)) < 1e-12
    # and the quantisation error is within half a code step (relative 2^-4 in
    # the normal range, absolute 2^-10 * scale below it)
    kt = (k.astype(np.float32) - res["mu32"]).astype(np.float32)
    for x, deq, sc in ((q.astype(np.float64), dq, res["q_scale"]), (kt.astype(np.float64), dk, res["k_scale"])):
        for j in range(T):
            r = slice(64 * j, min(64 * j + 64, N))
            s = float(sc[j])
            err = np.abs(x[r] - deq[r])
            bound = np.maximum(np.abs(x[r]) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)
            assert np.all(err <= bound)


# ---------------------------------------------------------------- P2 / P8
@pytest.mark.parametrize("topk", [1, 2])
def test_linear_branch_equals_token_level_direct_sum(topk):
    N, d = 170, 8
    q, k, v = _rand(N, d, 21 + topk)
    alpha0 = np.zeros(d, np.float32)
    res = O.forward_head(q, k, v, alpha0, topk=topk, smooth_k=True)
    lut = res["lut"]
    mu = [sum(float(k[t, c]) for t in range(N)) / N for c in range(d)]
    phik = [bf_feature_softmax([float(k[s, c]) - mu[c] for c in range(d)]) for s in range(N)]
    eps = 1e-5
    ref = np.zeros((N, d))
    for t in range(N):
        pq = bf_feature_softmax(q[t])
        routed = set()
        for j in lut[t // 64]:
            routed.update(range(64 * j, min(64 * j + 64, N)))
        num = np.zeros(d)
        den = 0.0
        for s in range(N):
            if s in routed:
                continue
            w = sum(pq[c] * phik[s][c] for c in range(d))
            num += w * v[s].astype(np.float64)
            den += w
        ref[t] = num / (den + eps)
    assert np.max(np.abs(res["o"] - ref)) < 1e-12
    # complement form: H_tot - sum over routed h_j equals the unrouted sum
    for i in range(O.num_blocks(N)):
        routed = res["h"][lut[i]].sum(axis=0)
        unrouted = sum(res["h"][j] for j in range(O.num_blocks(N)) if j not in set(lut[i]))
        assert np.max(np.abs(res["h_sum"] - routed - unrouted)) < 1e-12


def test_h_and_z_match_loops():
    N, d = 100, 4
    q, k, v = _rand(N, d, 3)
    res = O.forward_head(q, k, v, np.zeros(d, np.float32), topk=1, smooth_k=False)
    for j in range(2):
        lo, hi = 64 * j, min(64 * j + 64, N)
        h = np.zeros((d, d))
        z = np.zeros(d)
        for t in range(lo, hi):
            pk = bf_feature_softmax(k[t])
            for a in range(d):
                z[a] += pk[a]
                for b in range(d):
                    h[a, b] += pk[a] * float(v[t, b])
        assert np.max(np.abs(res["h"][j] - h)) < 1e-13
        assert np.max(np.abs(res["z"][j] - z)) < 1e-13


# ---------------------------------------------------------------- P9
def test_ideal_ratio_recovers_full_attention():
    N, d, topk = 192, 8, 1
    q, k, v = _rand(N, d, 9)
    res = O.forward_head(q, k, v, np.ones(d, np.float32), topk=topk, smooth_k=False)
    lut = res["lut"]
    scale = 1.0 / math.sqrt(d)
    full = bf_softmax_attention(q, k, v, lambda t: range(N), scale)

    def routed(t):
        out = []
        for j in lut[t // 64]:
            out.extend(range(64 * j, min(64 * j + 64, N)))
        return out

    def rest(t):
        r = set(routed(t))
        return [s for s in range(N) if s not in r]

    o_rest = bf_softmax_attention(q, k, v, rest, scale)
    for t in range(N):
        logits = np.array([sum(float(q[t, c]) * float(k[s, c]) for c in range(d)) * scale for s in range(N)])
        p = np.exp(logits - logits.max())
        p /= p.sum()
        a_t = p[routed(t)].sum()
        mixed = a_t * res["o_s"][t] + (1 - a_t) * o_rest[t]
        assert np.max(np.abs(mixed - full[t])) < 1e-12


# ---------------------------------------------------------------- P3 / P4
def test_router_scores_match_loops_and_mask_is_consistent():
    N, d, topk = 300, 6, 2
    q, k, _ = _rand(N, d, 31)
    rng = np.random.default_rng(4)
    wq = (rng.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    wk = (rng.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    r = O.route_head(q, k, wq, wk, topk, smooth_k=True)
    T = O.num_blocks(N)
    mu = [sum(float(k[t, c]) for t in range(N)) / N for c in range(d)]
    qb = [bf_mean_rows(q, 64 * i, min(64 * i + 64, N)) for i in range(T)]
    kb = [[x - m for x, m in zip(bf_mean_rows(k, 64 * j, min(64 * j + 64, N)), mu)] for j in range(T)]
    qh = [[sum(qb[i][a] * float(wq[a, b]) for a in range(d)) for b in range(d)] for i in range(T)]
    kh = [[sum(kb[j][a] * float(wk[a, b]) for a in range(d)) for b in range(d)] for j in range(T)]
    for i in range(T):
        for j in range(T):
            s = sum(qh[i][c] * kh[j][c] for c in range(d)) / math.sqrt(d)
            assert abs(s - r["scores"][i, j]) < 1e-12
        # textbook Top-k: sort by (-score, index), keep k, list ascending
        order = sorted(range(T), key=lambda j: (-r["scores"][i, j], j))
        assert list(r["lut"][i]) == sorted(order[:topk])
        assert r["mask"][i].sum() == topk
        assert sorted(np.nonzero(r["mask"][i])[0].tolist()) == list(r["lut"][i])
        assert all(np.diff(r["lut"][i]) > 0)


def test_topk_ties_go_to_lower_index():
    scores = np.array([[1.0, 2.0, 2.0, 0.5, 2.0]])
    lut, mask = O.topk_blocks(scores, 2)
    assert lut.tolist() == [[1, 2]]
    lut, mask = O.topk_blocks(scores, 4)
    assert lut.tolist() == [[0, 1, 2, 4]]
    assert mask.tolist() == [[1, 1, 1, 0, 1]]


def _min_gap(scores, topk):
    srt = -np.sort(-scores, axis=1)
    if topk >= scores.shape[1]:
        return np.inf
    return np.min(srt[:, topk - 1] - srt[:, topk])


def test_mask_invariant_under_smoothing_and_positive_rescale():
    N, d, topk = 640, 8, 3
    q, k, _ = _rand(N, d, 41)
    rng = np.random.default_rng(5)
    wq = (rng.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    wk = (rng.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    a = O.route_head(q, k, wq, wk, topk, smooth_k=True)
    b = O.route_head(q, k, wq, wk, topk, smooth_k=False)
    c = O.route_head(q, k, (wq * 3).astype(np.float32), (wk * 0.5).astype(np.float32), topk, smooth_k=True)
    assert _min_gap(a["scores"], topk) > 1e-9
    # smoothing subtracts q_hat . (mu W_k) from a whole row; rescaling W scales it
    assert np.array_equal(a["mask"], b["mask"])
    assert np.array_equal(a["mask"], c["mask"])
    # softmax of a row is monotone: same Top-k
    e = np.exp(a["scores"] - a["scores"].max(axis=1, keepdims=True))
    sm = e / e.sum(axis=1, keepdims=True)
    lut2, _ = O.topk_blocks(sm, topk)
    assert np.array_equal(lut2, a["lut"])


def test_complementary_branches_partition_the_keys():
    N, d = 1000, 4
    q, k, _ = _rand(N, d, 7)
    T = O.num_blocks(N)
    for topk in (1, 5, T):
        r = O.route_head(q, k, None, None, topk)
        sparse = r["mask"].astype(bool)
        linear = ~sparse
        assert np.all(sparse ^ linear)
        assert np.all(sparse.sum(axis=1) == topk)
        assert np.all(linear.sum(axis=1) == T - topk)


# ---------------------------------------------------------------- P5 / P6
def test_mixing_endpoints_and_affinity():
    N, d = 200, 8
    q, k, v = _rand(N, d, 17)
    rng = np.random.default_rng(2)
    a1 = rng.uniform(0, 1, d).astype(np.float64)
    a2 = rng.uniform(0, 1, d).astype(np.float64)
    base = O.forward_head(q, k, v, np.ones(d), topk=2)
    assert np.array_equal(base["o"], base["o_s"])
    z = O.forward_head(q, k, v, np.zeros(d), topk=2)
    assert np.array_equal(z["o"], z["o_l"])
    r1 = O.forward_head(q, k, v, a1, topk=2)["o"]
    r2 = O.forward_head(q, k, v, a2, topk=2)["o"]
    rm = O.forward_head(q, k, v, 0.5 * (a1 + a2), topk=2)["o"]
    assert np.max(np.abs(rm - 0.5 * (r1 + r2))) < 1e-12


def test_branch_outputs_are_convex_combinations_of_values():
    N, d = 260, 8
    q, k, v = _rand(N, d, 19)
    res = O.forward_head(q, k, v, np.ones(d), topk=2, eps=0.0)
    lo, hi = v.min(axis=0), v.max(axis=0)
    assert np.all(res["o_s"] >= lo - 1e-12) and np.all(res["o_s"] <= hi + 1e-12)
    assert np.all(res["o_l"] >= lo - 1e-12) and np.all(res["o_l"] <= hi + 1e-12)


# ---------------------------------------------------------------- P7
def test_fp8_decode_matches_bit_fields_for_all_codes():
    got = F8.decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        ref = bf_decode_e4m3(c)
        if math.isnan(ref):
            assert math.isnan(got[c])
        else:
            assert got[c] == ref and math.copysign(1, got[c]) == math.copysign(1, ref)
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0


def test_fp8_encode_round_trip_midpoints_and_saturation():
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array([bf_decode_e4m3(c) for c in finite])
    assert F8.encode(vals).tolist() == finite
    mags = sorted(set(abs(bf_decode_e4m3(c)) for c in range(127)))
    codes = {abs(bf_decode_e4m3(c)): c for c in range(127)}
    for a, b in zip(mags[:-1], mags[1:]):
        mid = 0.5 * (a + b)
        even = codes[a] if codes[a] % 2 == 0 else codes[b]
        assert F8.encode(np.array([mid]))[0] == even
        assert F8.encode(np.array([-mid]))[0] == even | 0x80
        assert F8.encode(np.array([np.nextafter(mid, 0)]))[0] == codes[a]
        assert F8.encode(np.array([np.nextafter(mid, 1e9)]))[0] == codes[b]
    assert F8.encode(np.array([448.0, 449.0, 464.0, 1e30, -1e30])).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert F8.encode(np.array([-0.0, -1e-30, 1e-30]))[:].tolist() == [0x80, 0x80, 0x00]


def test_fp8_encode_agrees_with_torch_cast_inside_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        rng.standard_normal(20000) * 2.0 ** -8]).astype(np.float32)
    ours = F8.encode(y.astype(np.float64))
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_quantiser_scale_and_codes():
    x = np.zeros((70, 4), np.float32)
    x[3, 1] = -2.5
    x[10, 2] = 1.0
    x[66, 0] = 0.0           # second block all zero -> scale 1
    codes, scales, deq = O.quantize_fp8_blocks(x)
    assert scales[0] == np.float32(np.float32(2.5) / np.float32(448))
    assert scales[1] == np.float32(1.0)
    assert codes[3, 1] == 0xFE                      # -448 after scaling
    assert deq[3, 1] == -448.0 * float(scales[0])
    assert np.all(codes[64:] == 0)
