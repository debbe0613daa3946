"""Plain fp64 CPU oracle of the SLA2 sparse-linear attention forward pass.

TEST INFRASTRUCTURE ONLY.  It defines the expected results: only tests/, the
package entry point's smoke check and the benchmark's CPU-baseline leg may
import or run it.  It shares no code with the HIP path and imports nothing
from it.  Every step is the plain definition, in fp64 numpy, one (batch, head)
at a time, with a library matmul as the only building block.

Sources (titles of the pages and the section of each):
* "SLA2: Sparse-Linear Attention with Learnable Routing and QAT" (AI summary
  page): section 3 (SLA2 design: O = alpha*O_s + (1-alpha)*O_l, sparse branch
  only where M = 1, linear branch from K^T V over M = 0), section 4 (learnable
  router: mean pooling of consecutive Q and K blocks, d x d projections
  proj_q / proj_k, row-wise Top-k into a compressed block mask), section 5
  (QAT: Q and K quantised to low bit with scales before the scores), section 6
  (key smoothing before block processing).
* "SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable
  Sparse-Linear Attention" (detailed summary page): section 2 Q2 (compressed
  scores from pooled Q, K over 64-token blocks; h_j = phi(K_j)^T V_j and
  z_j = rowsum phi(K_j)^T), section 3 figure (O_s = diag(l)^-1 O_acc,
  O_l = phi(Q_i) H_i / (phi(Q_i) Z_i)), section 4 (phi = softmax feature map,
  1e-5 added to the linear denominator, linear re-association), section 7
  (the mean over tokens subtracted from K).

Readings where the pages are silent (each is listed in the design notes):
alpha is a per-head d-vector used as given; the sparse softmax is
renormalised over the routed keys only; the linear branch covers exactly the
unrouted blocks; phi is a plain softmax over the d features of Q and of the
smoothed K; key smoothing subtracts the per-(batch, head) token mean of K and
applies to routing, the sparse branch and phi(K); scores are
(q_bar W_q).(k_bar W_k)/sqrt(d) with W shared by all heads and no bias; ties
in Top-k go to the lower block index; the last block may be partial (means
over its valid tokens, only valid keys attend); no causal mask; FP8 is OCP
e4m3 with one absmax scale per 64-token block of each (batch, head), round to
nearest even, saturating at 448.

Precision of decisions: the FP8 codes are integers decided by floating point,
so this oracle takes those decisions in the kernel's precision (float32):
K_tilde32 = fl32(K - fl32(mu)), scale = fl32(absmax / 448),
y = fl32(x / scale).  Everything else is fp64.

Low-bit P.V (SLA2 page, section 5: the sparse branch also quantises P and V
and dequantises their product).  The pages fix neither granularity nor scale
form; the reading here: V gets one power-of-two scale per (64-token block,
channel), the smallest 2**e with max|V| <= 448 * 2**e; P gets one
power-of-two scale per (query, routed block), 2**(ceil(M) - 8) with M the
largest log2-scaled score of that query in that block, so the block's
largest P code lies in (128, 256].  The softmax normaliser sums the
unquantised P.  Powers of two make the scaling exact, so only the e4m3
rounding of P and V differs from the plain product.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from . import fp8_e4m3

BLOCK = 64
EPS = 1e-5


# --------------------------------------------------------------------------
# blocks and pooling (SLA2 page, section 4; SLA page, section 2 Q2 step 1)
# --------------------------------------------------------------------------
def num_blocks(N: int, block: int = BLOCK) -> int:
    return (N + block - 1) // block


def block_rows(j: int, N: int, block: int = BLOCK) -> slice:
    """Token rows of block j: [block*j, min(block*(j+1), N))."""
    return slice(block * j, min(block * (j + 1), N))


def mean_pool(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Mean of each block of consecutive tokens over its valid rows: [T, d]."""
    N = x.shape[0]
    T = num_blocks(N, block)
    return np.stack([x[block_rows(j, N, block)].mean(axis=0) for j in range(T)])


# --------------------------------------------------------------------------
# router (SLA2 page, section 4; hard Top-k at inference, section 7)
# --------------------------------------------------------------------------
def router_scores(q_pool: np.ndarray, k_pool: np.ndarray, wq: Optional[np.ndarray],
                  wk: Optional[np.ndarray]) -> np.ndarray:
    """Block scores s_ij = (q_bar_i W_q) . (k_bar_j W_k) / sqrt(d); W None = identity.

    The softmax the SLA page applies to the compressed scores is monotone in
    each row, so it does not change the Top-k and is left out.
    """
    d = q_pool.shape[1]
    qh = q_pool if wq is None else q_pool @ np.asarray(wq, np.float64)
    kh = k_pool if wk is None else k_pool @ np.asarray(wk, np.float64)
    return (qh @ kh.T) / math.sqrt(d)


def topk_blocks(scores: np.ndarray, topk: int):
    """Row-wise hard Top-k: the topk largest scores, ties to the lower index.

    Returns (lut [T_q, topk] int32 ascending, mask [T_q, T_kv] uint8).
    """
    Tq, Tk = scores.shape
    if not 1 <= topk <= Tk:
        raise ValueError("topk out of range")
    lut = np.empty((Tq, topk), dtype=np.int32)
    mask = np.zeros((Tq, Tk), dtype=np.uint8)
    idx = np.arange(Tk)
    for i in range(Tq):
        order = np.lexsort((idx, -scores[i]))   # primary: score desc, then index asc
        chosen = np.sort(order[:topk])
        lut[i] = chosen
        mask[i, chosen] = 1
    return lut, mask


# --------------------------------------------------------------------------
# low-bit Q.K^T (SLA2 page, section 5): per-block absmax FP8 e4m3 fake quant
# --------------------------------------------------------------------------
def quantize_fp8_blocks(x32: np.ndarray, block: int = BLOCK):
    """Quantise float32 rows block by block.

    Per block: scale = fl32(absmax/448) (1 if that is 0), y = fl32(x/scale),
    code = e4m3(clamp(y, +-448)).  Returns (codes [N, d] uint8, scales [T]
    float32, dequantised values [N, d] fp64 = decode(code)*scale).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    N = x32.shape[0]
    T = num_blocks(N, block)
    codes = np.empty(x32.shape, dtype=np.uint8)
    scales = np.empty(T, dtype=np.float32)
    deq = np.empty(x32.shape, dtype=np.float64)
    for j in range(T):
        r = block_rows(j, N, block)
        blk = x32[r]
        amax = np.float32(np.max(np.abs(blk)))
        s = np.float32(amax / np.float32(fp8_e4m3.FP8_E4M3_MAX))
        if s == np.float32(0.0):
            s = np.float32(1.0)
        y = (blk / s).astype(np.float32)
        y = np.clip(y, -fp8_e4m3.FP8_E4M3_MAX, fp8_e4m3.FP8_E4M3_MAX)
        c = fp8_e4m3.encode(y)
        codes[r] = c
        scales[j] = s
        deq[r] = fp8_e4m3.decode(c) * np.float64(s)
    return codes, scales, deq


# --------------------------------------------------------------------------
# low-bit P.V (SLA2 page, section 5): power-of-two scales, e4m3 codes
# --------------------------------------------------------------------------
E8M0_MIN = -127   # smallest power-of-two exponent a scale takes


def v_channel_exponents(v_blk: np.ndarray) -> np.ndarray:
    """Per channel c of one key block: the smallest integer e >= -127 with
    max_t |V[t, c]| <= 448 * 2**e (-127 for an all-zero channel)."""
    amax = np.max(np.abs(np.asarray(v_blk, np.float64)), axis=0)
    e = np.full(amax.shape, E8M0_MIN, dtype=np.int64)
    for c, a in enumerate(amax):
        if a == 0.0:
            continue
        _, x = math.frexp(a)            # a = f * 2**x with 0.5 <= f < 1
        ec = x - 10                     # 448 * 2**(x-10) < 0.5 * 2**x <= a
        while math.ldexp(fp8_e4m3.FP8_E4M3_MAX, ec) < a:
            ec += 1
        e[c] = max(ec, E8M0_MIN)
    return e


def quantize_v_blocks(v: np.ndarray, block: int = BLOCK):
    """V codes with per-(block, channel) power-of-two scales.

    Returns (codes [N, d] uint8, exponents [T, d] int, dequantised [N, d] fp64
    = decode(code) * 2**e)."""
    v64 = np.asarray(v, np.float64)
    N = v64.shape[0]
    T = num_blocks(N, block)
    codes = np.empty(v64.shape, dtype=np.uint8)
    exps = np.empty((T, v64.shape[1]), dtype=np.int64)
    deq = np.empty(v64.shape, dtype=np.float64)
    for j in range(T):
        r = block_rows(j, N, block)
        e = v_channel_exponents(v64[r])
        c = fp8_e4m3.encode(np.ldexp(v64[r], -e))   # exact scaling, then round to e4m3
        codes[r], exps[j] = c, e
        deq[r] = np.ldexp(fp8_e4m3.decode(c), e)
    return codes, exps, deq


def quantize_p_block(x: np.ndarray):
    """P of one (query rows x routed block) tile from log2-scaled scores x.

    Per row: c = ceil(max x) (an integer), codes = e4m3(2**(x - c + 8)), and
    the dequantised P = decode(codes) * 2**(c - 8).  Returns (codes, c, deq)."""
    x = np.asarray(x, np.float64)
    c = np.ceil(x.max(axis=1, keepdims=True))
    codes = fp8_e4m3.encode(np.exp2(x - c + 8.0))
    deq = np.ldexp(fp8_e4m3.decode(codes), (c - 8.0).astype(np.int64))
    return codes, c[:, 0].astype(np.int64), deq


# --------------------------------------------------------------------------
# linear branch (SLA page, sections 2-4; SLA2 page, section 3)
# --------------------------------------------------------------------------
def phi(x: np.ndarray) -> np.ndarray:
    """Softmax feature map over the last (feature) axis."""
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def linear_stats(phi_k: np.ndarray, v: np.ndarray, block: int = BLOCK):
    """h_j = phi(K_j)^T V_j [T, d, d] and z_j = column sums of phi(K_j) [T, d]."""
    N = phi_k.shape[0]
    T = num_blocks(N, block)
    h = np.stack([phi_k[block_rows(j, N, block)].T @ v[block_rows(j, N, block)] for j in range(T)])
    z = np.stack([phi_k[block_rows(j, N, block)].sum(axis=0) for j in range(T)])
    return h, z


# --------------------------------------------------------------------------
# one (batch, head)
# --------------------------------------------------------------------------
def route_head(q, k, wq, wk, topk, smooth_k=True, block=BLOCK):
    """Router of one head: pooled means, key mean, scores, LUT and mask."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    mu = k.mean(axis=0) if smooth_k else np.zeros(k.shape[1])
    q_pool = mean_pool(q, block)
    k_pool = mean_pool(k, block) - mu          # pool(K - mu) = pool(K) - mu
    scores = router_scores(q_pool, k_pool, wq, wk)
    lut, mask = topk_blocks(scores, topk)
    return {"mu": mu, "q_pool": q_pool, "k_pool": k_pool, "scores": scores,
            "lut": lut, "mask": mask}


def forward_head(q, k, v, alpha_h, wq=None, wk=None, topk=1, smooth_k=True, qk_fp8=False,
                 eps=EPS, block=BLOCK, lut=None, query_blocks: Optional[Sequence[int]] = None,
                 pv_fp8=False):
    """SLA2 forward of one (batch, head).

    q, k, v: [N, d] values (float32 holding the exact inputs); alpha_h: [d].
    pv_fp8: the sparse branch's P.V with e4m3 P and V (quantize_p_block,
    quantize_v_blocks); the softmax normaliser and the linear branch are exact.
    lut: use this routing instead of the router's (rows ascending).
    query_blocks: compute the outputs of these query blocks only (the router
    and the per-key-block statistics always cover every block).
    Returns a dict with every intermediate and the outputs o_s, o_l, o
    (rows of query blocks that were not computed are NaN).
    """
    q32 = np.asarray(q, np.float32)
    k32 = np.asarray(k, np.float32)
    q64 = q32.astype(np.float64)
    k64 = k32.astype(np.float64)
    v64 = np.asarray(v, np.float64)
    N, d = q64.shape
    T = num_blocks(N, block)
    out = route_head(q64, k64, wq, wk, topk, smooth_k, block)
    if lut is not None:
        lut = np.asarray(lut, dtype=np.int32)
        mask = np.zeros((T, T), dtype=np.uint8)
        for i in range(T):
            mask[i, lut[i]] = 1
        out["lut"], out["mask"] = lut, mask
    lut, mask = out["lut"], out["mask"]
    mu = out["mu"]
    mu32 = mu.astype(np.float32)
    out["mu32"] = mu32

    # key smoothing (SLA2 page section 6; SLA page section 7)
    kt64 = k64 - mu

    # sparse-branch operands: FP8 fake quant or the inputs themselves
    if qk_fp8:
        q8, sq, q_s = quantize_fp8_blocks(q32, block)
        kt32 = (k32 - mu32).astype(np.float32)
        k8, sk, k_s = quantize_fp8_blocks(kt32, block)
        out.update(q8=q8, q_scale=sq, k8=k8, k_scale=sk)
    else:
        q_s, k_s = q64, kt64
    if pv_fp8:
        v8, v_exp, v_pv = quantize_v_blocks(v64, block)
        out.update(v8=v8, v_exp=v_exp)

    # linear-branch statistics over every key block
    phi_k = phi(kt64)
    h, z = linear_stats(phi_k, v64, block)
    out.update(h=h, z=z, h_sum=h.sum(axis=0), z_sum=z.sum(axis=0))

    blocks = range(T) if query_blocks is None else query_blocks
    o_s = np.full((N, d), np.nan)
    o_l = np.full((N, d), np.nan)
    lse = np.full(N, np.nan)
    unrouted = (1 - mask).astype(np.float64)
    phi_q = None
    inv_sqrt_d = 1.0 / math.sqrt(d)
    for i in blocks:
        rows = block_rows(i, N, block)
        keys = np.concatenate([np.arange(N)[block_rows(j, N, block)] for j in lut[i]])
        # sparse branch: softmax over the routed keys only, then P V
        s = (q_s[rows] @ k_s[keys].T) * inv_sqrt_d
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        if pv_fp8:
            # per routed block: e4m3 P (in units of 2**x, x = s / ln 2) times e4m3 V; the
            # normaliser sum_t 2**x_t is exact.  An integer reference keeps the scaling exact.
            x = s / math.log(2.0)
            ref = np.ceil(x.max(axis=1, keepdims=True))
            num = np.zeros((s.shape[0], d))
            col = 0
            for j in lut[i]:
                n_j = block_rows(j, N, block).stop - block_rows(j, N, block).start
                _, _, p_deq = quantize_p_block(x[:, col:col + n_j] - ref)
                num += p_deq @ v_pv[keys[col:col + n_j]]
                col += n_j
            o_s[rows] = num / np.exp2(x - ref).sum(axis=1, keepdims=True)
        else:
            o_s[rows] = (p / l) @ v64[keys]
        lse[rows] = (m + np.log(l))[:, 0]
        # linear branch over the unrouted blocks
        H_i = np.tensordot(unrouted[i], h, axes=(0, 0))
        Z_i = unrouted[i] @ z
        pq = phi(q64[rows])
        o_l[rows] = (pq @ H_i) / (pq @ Z_i + eps)[:, None]
    a = np.asarray(alpha_h, np.float64)
    o = a * o_s + (1.0 - a) * o_l
    out.update(o_s=o_s, o_l=o_l, o=o, lse=lse)
    return out


def forward(inputs: dict, topk: int, smooth_k: bool = True, qk_fp8: bool = False,
            eps: float = EPS, block: int = BLOCK, luts=None, heads=None, query_blocks=None,
            pv_fp8: bool = False):
    """SLA2 forward over [B, H, N, d] inputs (dict from the input generator).

    heads: optional list of (b, h) to compute; luts: optional {(b, h): lut}.
    Returns {(b, h): forward_head(...) result}.
    """
    q, k, v, alpha = inputs["q"], inputs["k"], inputs["v"], inputs["alpha"]
    B, H = q.shape[:2]
    heads = [(b, hh) for b in range(B) for hh in range(H)] if heads is None else heads
    res = {}
    for (b, hh) in heads:
        res[(b, hh)] = forward_head(
            q[b, hh], k[b, hh], v[b, hh], alpha[hh], inputs.get("wq"), inputs.get("wk"),
            topk=topk, smooth_k=smooth_k, qk_fp8=qk_fp8, eps=eps, block=block,
            lut=None if luts is None else luts.get((b, hh)), query_blocks=query_blocks,
            pv_fp8=pv_fp8)
    return res
