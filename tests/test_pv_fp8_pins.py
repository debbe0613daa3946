"""Pins of the oracle's low-bit P.V (SLA2 page, section 5: the sparse branch
quantises P and V and dequantises their product).

What fixes the oracle here, independently of its own code:
* the power-of-two V scale is the smallest one that avoids saturation, checked
  against its defining inequalities; the P scale puts each row's largest code
  in the top binade;
* on inputs that both quantisers reproduce exactly (scores whose log2 values
  are integers, V with at most four significant bits per channel), the low-bit
  sparse output equals the plain softmax attention output: any wrong scale
  exponent, dropped factor or transposed operand breaks the equality;
* on random inputs the low-bit output stays within the e4m3 rounding bound of
  the exact one (each of P and V off by at most 2**-4 relative in the normal
  range) and the quantisation is visibly active.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import fp8_e4m3 as F8
from oracle import sla2_oracle as O


def test_v_exponent_is_the_smallest_non_saturating_power_of_two():
    rng = np.random.default_rng(3)
    blk = rng.standard_normal((64, 9)) * np.exp2(rng.integers(-20, 20, size=9))
    blk[:, 4] = 0.0                      # all-zero channel
    blk[:, 5] = 0.0
    blk[7, 5] = 448.0                    # exactly at the boundary of e = 0
    blk[:, 6] = 0.0
    blk[0, 6] = -1.75 * 2.0 ** 3         # 448 * 2**-5 exactly
    e = O.v_channel_exponents(blk)
    amax = np.abs(blk).max(axis=0)
    for c in range(blk.shape[1]):
        if amax[c] == 0.0:
            assert e[c] == -127
            continue
        assert amax[c] <= 448.0 * 2.0 ** e[c]
        assert amax[c] > 448.0 * 2.0 ** (e[c] - 1)
    assert e[5] == 0 and e[6] == -5


def test_v_codes_round_within_half_an_e4m3_step():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((200, 16)) * 3.0).astype(np.float32)
    codes, exps, deq = O.quantize_v_blocks(v)
    assert exps.shape == (4, 16)
    for j in range(4):
        r = O.block_rows(j, 200)
        scaled = np.ldexp(v[r].astype(np.float64), -exps[j])
        assert np.abs(scaled).max() <= F8.FP8_E4M3_MAX
        # half a step: 2**-4 relative for normals, 2**-10 absolute below 2**-6
        err = np.abs(np.ldexp(deq[r], -exps[j]) - scaled)
        assert np.all(err <= np.maximum(np.abs(scaled) * 2.0 ** -4, 2.0 ** -10) + 1e-300)
        np.testing.assert_array_equal(deq[r], np.ldexp(F8.decode(codes[r]), exps[j]))


def test_p_codes_put_each_row_max_in_the_top_binade():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 64)) * 6.0 + 3.0
    codes, c, deq = O.quantize_p_block(x)
    top = F8.decode(codes).max(axis=1)
    # the row max maps into (128, 256] before rounding; rounding can land on 128 itself
    assert np.all(top >= 128.0) and np.all(top <= 256.0)
    np.testing.assert_array_equal(c, np.ceil(x.max(axis=1)).astype(np.int64))
    p = np.exp2(x)
    assert np.all(np.abs(deq - p) <= np.maximum(p * 2.0 ** -4, np.exp2(c - 8.0)[:, None] * 2.0 ** -10))


@pytest.mark.parametrize("N", [192, 170])
def test_low_bit_pv_is_exact_on_representable_inputs(N):
    # d = 4, scores s = q.k / 2 = n ln 2 with integer n, so the log2 scores are integers (up to
    # input rounding); V has at most four significant bits per value, one power of two per column
    d = 4
    rng = np.random.default_rng(6)
    T = O.num_blocks(N)
    q = np.zeros((N, d), np.float64)
    q[:, 0] = 2.0 * math.log(2.0)
    k = np.zeros((N, d), np.float64)
    n = rng.integers(-8, 8, size=N)     # spread within 16 keeps every P code normal or subnormal
    k[:, 0] = n
    v = rng.integers(-15, 16, size=(N, d)).astype(np.float64) * np.exp2(rng.integers(-6, 6, size=d))
    lut = np.array([sorted(rng.choice(T, size=2, replace=False)) for _ in range(T)], np.int32)
    alpha = np.ones(d)
    exact = O.forward_head(q, k, v, alpha, topk=2, smooth_k=False, lut=lut)
    low = O.forward_head(q, k, v, alpha, topk=2, smooth_k=False, lut=lut, pv_fp8=True)
    # q passes through float32, which moves the log2 scores off the integers by ~1e-8 relative:
    # e4m3 rounding takes that back out of P, the exact path keeps it.  A wrong exponent would
    # be off by a factor of two or more.
    np.testing.assert_allclose(low["o_s"], exact["o_s"], rtol=1e-6, atol=1e-9 * np.abs(v).max())
    np.testing.assert_array_equal(low["lse"], exact["lse"])


def test_low_bit_pv_error_is_within_the_e4m3_bound():
    rng = np.random.default_rng(7)
    N, d, topk = 250, 32, 2
    T = O.num_blocks(N)
    q = rng.standard_normal((N, d)).astype(np.float32)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    lut = np.array([sorted(rng.choice(T, size=topk, replace=False)) for _ in range(T)], np.int32)
    alpha = np.ones(d, np.float32)
    exact = O.forward_head(q, k, v, alpha, topk=topk, qk_fp8=True, lut=lut)
    low = O.forward_head(q, k, v, alpha, topk=topk, qk_fp8=True, lut=lut, pv_fp8=True)
    v64 = v.astype(np.float64)
    worst = 0.0
    for i in range(T):
        rows = O.block_rows(i, N)
        keys = np.concatenate([np.arange(N)[O.block_rows(j, N)] for j in lut[i]])
        # the exact softmax weights of the same (dequantised) scores
        qd = F8.decode(exact["q8"][rows]) * exact["q_scale"][i]
        kd = np.concatenate([F8.decode(exact["k8"][O.block_rows(j, N)]) * exact["k_scale"][j] for j in lut[i]])
        s = qd @ kd.T / math.sqrt(d)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        bound = (2 * 2.0 ** -4 + 2.0 ** -8) * (w @ np.abs(v64[keys])) + 2.0 ** -12 * np.abs(v64[keys]).max(axis=0)
        diff = np.abs(low["o_s"][rows] - exact["o_s"][rows])
        assert np.all(diff <= bound)
        worst = max(worst, float(diff.max()))
    assert worst > 1e-4   # the quantisation is active
