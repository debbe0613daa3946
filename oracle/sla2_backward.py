"""Plain fp64 CPU oracle of the SLA2 backward pass (gradients of one head).

TEST INFRASTRUCTURE ONLY.  It defines the expected results: only tests/, the
package entry point's smoke check and the benchmark's CPU-baseline leg may
import or run it.  It shares no code with the HIP path and imports nothing
from it.  It is autograd-free: every gradient is written out from the chain
rule of the forward pass that sla2_oracle.forward_head defines, in fp64 numpy.

Sources (titles of the pages and the section of each):
* "SLA2: Sparse-Linear Attention with Learnable Routing and QAT" (AI summary
  page): section 3 (O = alpha*O_s + (1-alpha)*O_l), section 5 (QAT: the
  low-bit forward, with the backward kept in 16-bit floating point),
  appendix A (the backward derives the gradients of Q, K, V, phi(Q) and
  phi(K) by hand; dH_i and dZ_i are formed per query block and accumulated,
  for each key block, over the query blocks that do not route to it).
* "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable
  Sparse-Linear Attention" (detailed summary page): section 4 (the sparse
  branch follows the FlashAttention backward; the linear branch's gradients
  go through the precomputed dH_i, dZ_i, symmetric to the forward).

Readings where the pages are silent (each is listed in the design notes):
* The router's mask is constant: no gradient reaches W_q, W_k or the pooling.
* Straight-through quantiser: in FP8 mode the forward scores use the
  dequantised Q', K' and the backward passes dQ' to Q and dK' to K~
  unchanged.
* Key smoothing K~ = K - mean_t(K) is differentiated: dK = dK~ - mean_t(dK~).
  (The sparse branch contributes nothing to that mean: each row of dS sums
  to zero.)
* alpha is per head and per feature; dalpha sums over the tokens.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import sla2_oracle as O


def backward_head(q, k, v, alpha_h, dout, lut, smooth_k=True, qk_fp8=False, eps=O.EPS, block=O.BLOCK):
    """Gradients of sum(dout * O) for one (batch, head) with the routing `lut` held fixed.

    q, k, v, dout: [N, d] (float32 holding the exact inputs); alpha_h: [d]; lut: [T, k_sel].
    Returns dict(dq, dk, dv [N, d], dalpha [d]) in fp64, plus the forward's dict under "fw".
    """
    lut = np.asarray(lut, dtype=np.int32)
    fw = O.forward_head(q, k, v, alpha_h, topk=lut.shape[1], smooth_k=smooth_k, qk_fp8=qk_fp8,
                        eps=eps, block=block, lut=lut)
    q32 = np.asarray(q, np.float32)
    k32 = np.asarray(k, np.float32)
    q64 = q32.astype(np.float64)
    k64 = k32.astype(np.float64)
    v64 = np.asarray(v, np.float64)
    dO = np.asarray(dout, np.float64)
    a = np.asarray(alpha_h, np.float64)
    N, d = q64.shape
    T = O.num_blocks(N, block)
    mu = fw["mu"]
    kt64 = k64 - mu
    # the sparse branch's operands, exactly as the forward used them
    if qk_fp8:
        _, _, q_s = O.quantize_fp8_blocks(q32, block)
        _, _, k_s = O.quantize_fp8_blocks((k32 - fw["mu32"]).astype(np.float32), block)
    else:
        q_s, k_s = q64, kt64
    o_s, o_l, lse = fw["o_s"], fw["o_l"], fw["lse"]
    mask = fw["mask"]
    unrouted = (1 - mask).astype(np.float64)
    inv_sqrt_d = 1.0 / math.sqrt(d)

    # O = alpha*O_s + (1-alpha)*O_l
    dalpha = (dO * (o_s - o_l)).sum(axis=0)
    dOs = a * dO
    dOl = (1.0 - a) * dO

    # ---- sparse branch: FlashAttention backward over each row's routed keys
    dq_s = np.zeros((N, d))
    dk_s = np.zeros((N, d))
    dv = np.zeros((N, d))
    for i in range(T):
        rows = O.block_rows(i, N, block)
        keys = np.concatenate([np.arange(N)[O.block_rows(j, N, block)] for j in lut[i]])
        s = (q_s[rows] @ k_s[keys].T) * inv_sqrt_d
        p = np.exp(s - lse[rows][:, None])             # the forward's probabilities
        dp = dOs[rows] @ v64[keys].T
        dsum = (p * dp).sum(axis=1)                    # = dO_s . O_s per query
        ds = p * (dp - dsum[:, None])
        dq_s[rows] += (ds @ k_s[keys]) * inv_sqrt_d
        dk_s[keys] += (ds.T @ q_s[rows]) * inv_sqrt_d
        dv[keys] += p.T @ dOs[rows]

    # ---- linear branch: O_l = phi(q) H_i / (phi(q).Z_i + eps) over the unrouted blocks
    phi_q = O.phi(q64)
    phi_k = O.phi(kt64)
    h, z = fw["h"], fw["z"]
    dphi_q = np.zeros((N, d))
    dH = np.zeros((T, d, d))
    dZ = np.zeros((T, d))
    for i in range(T):
        rows = O.block_rows(i, N, block)
        H_i = np.tensordot(unrouted[i], h, axes=(0, 0))
        Z_i = unrouted[i] @ z
        pq = phi_q[rows]
        den = pq @ Z_i + eps
        ol = (pq @ H_i) / den[:, None]
        dnum = dOl[rows] / den[:, None]
        dden = -(dOl[rows] * ol).sum(axis=1) / den
        dphi_q[rows] = dnum @ H_i.T + dden[:, None] * Z_i[None, :]
        dH[i] = pq.T @ dnum
        dZ[i] = dden @ pq
    # each key block collects dH_i, dZ_i of the query blocks that do not route to it
    dh = np.tensordot(unrouted, dH, axes=(0, 0))       # dh[j] = sum_i unrouted[i, j] dH[i]
    dz = unrouted.T @ dZ
    dphi_k = np.zeros((N, d))
    for j in range(T):
        r = O.block_rows(j, N, block)
        dphi_k[r] = v64[r] @ dh[j].T + dz[j][None, :]
        dv[r] += phi_k[r] @ dh[j]

    # phi = softmax over the features: d x = phi * (d phi - <phi, d phi>)
    dq_lin = phi_q * (dphi_q - (phi_q * dphi_q).sum(axis=1, keepdims=True))
    dkt_lin = phi_k * (dphi_k - (phi_k * dphi_k).sum(axis=1, keepdims=True))

    dq = dq_s + dq_lin                                 # straight through Q' in FP8 mode
    dkt = dk_s + dkt_lin                               # straight through K' in FP8 mode
    dk = dkt - dkt.mean(axis=0, keepdims=True) if smooth_k else dkt
    return {"dq": dq, "dk": dk, "dv": dv, "dalpha": dalpha, "fw": fw, "dH": dH, "dZ": dZ}


def backward(inputs: dict, dout: np.ndarray, luts: dict, smooth_k=True, qk_fp8=False, heads=None):
    """Gradients over [B, H, N, d] inputs; dalpha [H, d] sums over the batch.

    luts: {(b, h): lut}.  heads: optional list of (b, h) (dalpha then covers only those).
    """
    q, k, v, alpha = inputs["q"], inputs["k"], inputs["v"], inputs["alpha"]
    B, H = q.shape[:2]
    heads = [(b, hh) for b in range(B) for hh in range(H)] if heads is None else heads
    res = {}
    dalpha = np.zeros(alpha.shape)
    for (b, hh) in heads:
        r = backward_head(q[b, hh], k[b, hh], v[b, hh], alpha[hh], dout[b, hh], luts[(b, hh)],
                          smooth_k=smooth_k, qk_fp8=qk_fp8)
        res[(b, hh)] = r
        dalpha[hh] += r["dalpha"]
    return res, dalpha
