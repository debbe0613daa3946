"""Shared helpers of the GPU parity tests: upload seeded inputs, run the three
C-ABI calls, fetch results, and compare them with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import sla2_inputs as I
from oracle import sla2_oracle as O

TIE_GAP = 1e-5          # rows whose k-th / (k+1)-th score gap is at most this may route either way
TOL_LOWP = dict(max_abs=2e-2, mean_rel=1e-2)   # bf16 / fp8 paths
TOL_F32 = dict(max_abs=1e-4)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(w: I.Workload, inp: dict):
    import torch
    el = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = {}
    for key in ("q", "k", "v"):
        dev[key] = torch.from_numpy(inp[key]).to(el).cuda()
    dev["alpha"] = torch.from_numpy(inp["alpha"]).cuda()
    for key in ("wq", "wk"):
        dev[key] = None if inp[key] is None else torch.from_numpy(inp[key]).cuda()
    return dev


def params_for(w: I.Workload, topk=None, smooth_k=True):
    from sparse_linear_attention_pool_amd import binding as Bn
    return Bn.make_params(w.B, w.H, w.N, w.d, w.topk if topk is None else topk, w.dtype, w.qk_mode,
                          smooth_k=smooth_k)


class GpuResult:
    """Device buffers of one run; out[key][b, h] fetches one head as numpy (bf16 -> fp64)."""

    def __init__(self, bufs):
        self.bufs = bufs

    def __getitem__(self, key):
        return _HeadView(self.bufs[key])

    def __contains__(self, key):
        return key in self.bufs


class _HeadView:
    def __init__(self, t):
        self.t = t

    def __getitem__(self, idx):
        import torch
        x = self.t[idx]
        if x.dtype == torch.bfloat16:
            return x.float().cpu().numpy().astype(np.float64)
        return x.cpu().numpy()

    def all(self):
        return self[...]

    def any(self):
        return bool(self.t.any().item())


def run_gpu(w: I.Workload, inp: dict, topk=None, smooth_k=True, with_lse=True, per_block_stats=True) -> GpuResult:
    """Upload, run route -> precompute -> forward on the current stream, keep results on device.
    per_block_stats=False leaves out h and z (bf16 modes), so the precompute skips storing them."""
    import torch
    from sparse_linear_attention_pool_amd import binding as Bn
    say(f"[gpu] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} topk={topk or w.topk} {w.dtype}/{w.qk_mode} seed={w.seed}")
    p = params_for(w, topk, smooth_k)
    dev = to_device(w, inp)
    bufs = Bn.allocate(p, "cuda", with_lse=with_lse, per_block_stats=per_block_stats)
    Bn.forward(p, dev, bufs)
    torch.cuda.synchronize()
    say("[gpu] done")
    return GpuResult(bufs)


def tie_rows(scores: np.ndarray, topk: int) -> np.ndarray:
    T = scores.shape[1]
    if topk >= T:
        return np.zeros(scores.shape[0], dtype=bool)
    srt = -np.sort(-scores, axis=1)
    return (srt[:, topk - 1] - srt[:, topk]) <= TIE_GAP


def check_lut(gpu_lut: np.ndarray, ref: dict, topk: int) -> np.ndarray:
    """LUT bit-exact outside tie rows; inside them a valid top-k within the tie band.
    Returns the tie-row flags."""
    scores, lut = ref["scores"], ref["lut"]
    ties = tie_rows(scores, topk)
    T = scores.shape[1]
    for i in range(scores.shape[0]):
        g = gpu_lut[i]
        assert np.all(np.diff(g) > 0) and g.min() >= 0 and g.max() < T, f"row {i}: LUT not ascending/in range"
        if not ties[i]:
            assert np.array_equal(g, lut[i]), f"row {i}: LUT {g.tolist()} != oracle {lut[i].tolist()}"
        else:
            kth = np.sort(scores[i])[::-1][topk - 1]
            assert np.all(scores[i][g] >= kth - TIE_GAP), f"tie row {i}: a chosen block is below the band"
    return ties


def compare(got: np.ndarray, ref: np.ndarray, max_abs: float, mean_rel: float = None, what: str = "",
            allow: np.ndarray = None):
    """max |got - ref| <= max_abs (+ allow, per element, where several roundings are correct)
    and mean |got - ref| <= mean_rel * mean |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    ma = float(err.max()) if err.size else 0.0
    mr = float(err.mean() / max(np.abs(ref).mean(), 1e-30)) if err.size else 0.0
    extra = 0.0 if allow is None else allow
    n_over = int(np.sum(err > max_abs)) if err.size else 0
    say(f"    {what}: max_abs={ma:.3e} mean_rel={mr:.3e}" +
        ("" if allow is None else f" (elements above {max_abs} inside their rounding allowance: {n_over})"))
    assert np.all(err <= max_abs + extra), f"{what}: max abs error {ma} > {max_abs}" + \
        ("" if allow is None else " plus the element's rounding allowance")
    if mean_rel is not None:
        assert mr <= mean_rel, f"{what}: mean rel error {mr} > {mean_rel}"
    return ma, mr


PV8_DELTA = 3e-5   # relative gap between the kernel's fp32 scores / hardware exp2 and the oracle's fp64


def pv8_flip_allowance(ref: dict, v: np.ndarray, lut: np.ndarray, d: int, alpha: np.ndarray) -> np.ndarray:
    """Per output element, what the low-bit P.V may differ by where a P code or a block's P scale
    sits at a rounding boundary: the kernel forms the scores in fp32 and exp2 in hardware, the
    oracle in fp64, so a P value within PV8_DELTA (relative) of an e4m3 rounding midpoint, or a
    block max within PV8_DELTA of an integer (the block's P scale), may be coded either way.
    Such a key k may contribute its other dequantised value: the allowance of element (q, f) is
    alpha_f * sum over those keys of |p_alt - p| |V8_kf| / l_q, with p_alt the farthest of the
    alternatives (the neighbouring code; at the other block scale, that scale's codes, saturation
    at 448 included) and V8 the dequantised e4m3 V.  Zero for rows with no such key.  Computed
    for the query blocks the oracle did."""
    from oracle import fp8_e4m3 as F8
    N = v.shape[0]
    T = O.num_blocks(N)
    allow = np.zeros((N, d))
    _, _, v8 = O.quantize_v_blocks(v)
    va = np.abs(v8)
    al = np.abs(np.asarray(alpha, np.float64))
    done = np.isfinite(ref["o"][:, 0])

    def deq(xr, c):   # the oracle's dequantised P of log2 scores xr (relative) at block scale c
        return F8.decode(F8.encode(np.exp2(xr - c + 8.0))) * np.exp2(c - 8.0)

    for i in range(T):
        rows = O.block_rows(i, N)
        if not done[rows].all():
            continue
        blocks = lut[i]
        keys = np.concatenate([np.arange(N)[O.block_rows(j, N)] for j in blocks])
        qd = F8.decode(ref["q8"][rows]) * np.float64(ref["q_scale"][i])
        kd = np.concatenate([F8.decode(ref["k8"][O.block_rows(j, N)]) * np.float64(ref["k_scale"][j]) for j in blocks])
        x = (qd @ kd.T) / np.sqrt(d) / np.log(2.0)
        x = x - np.ceil(x.max(axis=1, keepdims=True))      # relative to the row's reference
        dev = np.zeros(x.shape)                             # |p_alt - p| of each key
        col = 0
        for j in blocks:
            n_j = O.block_rows(j, N).stop - O.block_rows(j, N).start
            xb = x[:, col:col + n_j]
            M = xb.max(axis=1, keepdims=True)
            c = np.ceil(M)
            p0 = deq(xb, c)
            tol = PV8_DELTA * np.maximum(np.abs(M), 1)
            c_lo, c_hi = np.ceil(M - tol), np.ceil(M + tol)
            worst = np.zeros(xb.shape)
            for cc in (c_lo, c_hi):                         # the oracle's scale and, near an integer, the other
                for f in (1.0 - PV8_DELTA, 1.0 + PV8_DELTA):  # either side of a code midpoint
                    worst = np.maximum(worst, np.abs(deq(xb + np.log2(f), cc) - p0))
            dev[:, col:col + n_j] = worst
            col += n_j
        l = np.exp2(x).sum(axis=1, keepdims=True)
        allow[rows] = al[None, :] * ((dev @ va[keys]) / l)
    return allow


def oracle_head(w: I.Workload, inp: dict, b: int, h: int, topk=None, smooth_k=True, lut=None,
                query_blocks=None):
    return O.forward_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], inp["alpha"][h], inp["wq"],
                          inp["wk"], topk=w.topk if topk is None else topk, smooth_k=smooth_k,
                          qk_fp8=(w.qk_mode in ("fp8", "fp8pv")), lut=lut, query_blocks=query_blocks,
                          pv_fp8=(w.qk_mode == "fp8pv"))


def check_head(w: I.Workload, inp: dict, out: dict, b: int, h: int, topk=None, smooth_k=True,
               query_blocks=None, check_stats=True):
    """Full parity of one (batch, head): router, quantiser, statistics, output."""
    topk = w.topk if topk is None else topk
    route = O.route_head(inp["q"][b, h], inp["k"][b, h], inp["wq"], inp["wk"], topk, smooth_k)
    ties = check_lut(out["lut"][b, h], route, topk)
    mask = out["mask"][b, h]
    T = route["scores"].shape[0]
    for i in range(T):
        assert mask[i].sum() == topk and np.array_equal(np.nonzero(mask[i])[0], out["lut"][b, h][i])
    ref = oracle_head(w, inp, b, h, topk, smooth_k, lut=out["lut"][b, h], query_blocks=query_blocks)
    # router intermediates
    compare(out["q_pool"][b, h], ref["q_pool"], 1e-5 * max(1, np.abs(ref["q_pool"]).max()), what="q_pool")
    compare(out["k_pool"][b, h], ref["k_pool"], 1e-5 * max(1, np.abs(ref["k_pool"]).max()), what="k_pool")
    assert np.array_equal(out["k_mean"][b, h], ref["mu32"]), "k_mean differs from fp32(mean)"
    if w.qk_mode in ("fp8", "fp8pv"):
        N = w.N
        assert np.array_equal(out["q_scale"][b, h], ref["q_scale"]), "q_scale"
        assert np.array_equal(out["k_scale"][b, h], ref["k_scale"]), "k_scale"
        assert np.array_equal(out["q8"][b, h][:N], ref["q8"]), "q8 codes"
        assert np.array_equal(out["k8"][b, h][:N], ref["k8"]), "k8 codes"
        assert not out["q8"][b, h][N:].any() and not out["k8"][b, h][N:].any(), "pad rows not zero"
    if check_stats:
        # h is stored transposed: h[j][c][a] = sum_t phi(K~_t)[a] V_t[c].  bf16 path: phi enters
        # the product as bf16 hi + lo parts (relative 2^-16) in fp32 arithmetic, and h is
        # rounded to bf16 (relative 2^-9), so per element |err| <= 2^-14 * S + 2^-8 * |h| with
        # S = sum_t phi[t][a] |V_t[c]|; fp32 path: 1e-5 * (S + |h|).  h_sum stays fp32:
        # |err| <= 1e-5 * sum_j S_j.
        h_ref = np.transpose(ref["h"], (0, 2, 1))
        kt = inp["k"][b, h].astype(np.float64) - ref["mu"]
        h_abs, _ = O.linear_stats(O.phi(kt), np.abs(inp["v"][b, h].astype(np.float64)))
        h_abs = np.transpose(h_abs, (0, 2, 1))
        if "h" in out:   # per-block h, z are optional outputs in bf16 modes
            got_h = out["h"][b, h]
            err = np.abs(got_h - h_ref)
            if w.dtype == "bf16":
                bound = 2.0 ** -14 * h_abs + 2.0 ** -8 * np.abs(h_ref) + 1e-12
            else:
                bound = 1e-5 * (h_abs + np.abs(h_ref)) + 1e-12
            say(f"    h: max_abs={err.max():.3e}  max err/bound={np.max(err / bound):.3f}")
            assert np.all(err <= bound), "h outside its rounding bound"
            compare(out["z"][b, h], ref["z"], 1e-4 * max(np.abs(ref["z"]).max(), 1), what="z")
        hs_err = np.abs(out["h_sum"][b, h] - ref["h_sum"].T)
        hs_bound = 1e-5 * h_abs.sum(axis=0) + 1e-12
        say(f"    h_sum: max_abs={hs_err.max():.3e}  max err/bound={np.max(hs_err / hs_bound):.3f}")
        assert np.all(hs_err <= hs_bound), "h_sum outside its bound"
        compare(out["z_sum"][b, h], ref["z_sum"], 1e-4 * max(np.abs(ref["z_sum"]).max(), 1), what="z_sum")
    rows = np.isfinite(ref["o"][:, 0])
    tol = TOL_LOWP if w.dtype == "bf16" else TOL_F32
    if w.qk_mode == "fp8pv":
        allow = pv8_flip_allowance(ref, inp["v"][b, h], out["lut"][b, h], w.d, inp["alpha"][h])
        compare(out["o"][b, h][rows], ref["o"][rows], what="o", allow=allow[rows], **tol)
    else:
        compare(out["o"][b, h][rows], ref["o"][rows], what="o", **tol)
    lse_rows = rows & np.isfinite(ref["lse"])
    compare(out["lse"][b, h][lse_rows], ref["lse"][lse_rows], 1e-2 if w.dtype == "bf16" else 1e-4, what="lse")
    return ties
