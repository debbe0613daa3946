"""Benchmark of the SLA2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C2]
    python bench.py --copy-calibration MiB    # plain device copy, for HBM counter scaling

One step is the whole forward over one batch whose inputs are already in HBM:
sla2_route (pooling, FP8 quantisation of Q, projections, Top-k) ->
sla2_linear_precompute (phi(K~), h_j, z_j, sums, FP8 codes of K~) ->
sla2_attention_fwd (routed-block attention + linear complement + mix).
The default workload is the Wan2.1-1.3B-shaped layer at 97% sparsity
(B=1, H=12, N=32760 on a 21x30x52 latent grid, d=128, 15 of 512 key blocks
routed per query block, FP8 e4m3 Q.K^T, bf16 P.V, seeded d x d router
projections), with synthetic seeded inputs.

Prints one JSON line: effective TFLOPS of the step (routed-block FLOPs plus
linear-branch FLOPs over the step time), the step latency, the dominant
kernel's roofline figures measured with HIP events on its stream, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import sla2_inputs as I  # noqa: E402
from sparse_linear_attention_pool_amd import accounting as A  # noqa: E402

METRIC = "attn fwd latency (ms) + effective TFLOPS, N=32760 H=12 d=128, 97% sparse"

# MI355X published peaks (dense)
PEAK_BF16 = 2500.0     # TFLOP/s
PEAK_FP8 = 5000.0      # TFLOP/s
PEAK_HBM = 8000.0      # GB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_bytes(w: I.Workload):
    """Algorithmic HBM bytes of each call (what the method must move), per step."""
    BH, N, d, T = w.B * w.H, w.N, w.d, w.T
    el = 2 if w.dtype == "bf16" else 4
    fp8 = w.qk_mode == "fp8"
    tok = BH * N * d * el
    route = 2 * tok + (BH * T * 64 * d if fp8 else 0) + 2 * BH * T * d * 4
    pre = 2 * tok + BH * T * d * d * el + BH * T * d * 4 + (BH * T * 64 * d if fp8 else 0)
    return {"route": route, "precompute": pre}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "fwd_mfma_kernel_c2_hbm_traffic.md")
KERNEL_SOURCES = ("sparse_linear_attention_pool_amd/csrc/sla2_fwd.hip",
                  "sparse_linear_attention_pool_amd/csrc/sla2_device.hpp")


def kernel_source_hash() -> str:
    """sha256 of the fused kernel's sources with comments and blank space removed, so that a
    documentation edit keeps a counter record valid and any code change invalidates it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the fused kernel from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by the same counter's reading for a plain copy of known size), or
    None if there is none for this workload or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    for line in open(TRAFFIC_RECORD):
        if line.startswith("traffic-record: "):
            rec = json.loads(line[len("traffic-record: "):])
            if rec.get("workload") == workload and rec.get("source_sha256") == kernel_source_hash():
                return rec["bytes_per_launch"]
    return None


def copy_calibration(mib: int):
    """A plain device-to-device copy of `mib` MiB, three times: the known-size reference that
    FETCH_SIZE / WRITE_SIZE readings are scaled by."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def cpu_baseline(w: I.Workload, inp: dict, heads: int):
    """The oracle as it stands, timed on the host on `heads` heads of the workload."""
    from oracle import sla2_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    lut_flops = 0
    refs = []
    for h in range(heads):
        r = O.forward_head(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h], inp["alpha"][h], inp["wq"],
                           inp["wk"], topk=w.topk, qk_fp8=(w.qk_mode == "fp8"))
        lut_flops += A.sparse_flops_from_lut(r["lut"][None], w.N, w.d)
        refs.append({"o": r["o"], "lut": r["lut"], "scores": r["scores"]})
    dt = time.perf_counter() - t0
    flops = lut_flops + A.linear_flops(1, heads, w.N, w.d)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPS (effective)", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{heads} of {w.H} heads of the same workload (batch 0), full sequence, fp64 numpy",
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}, refs


def pass_times(evs):
    """Mean, median and min (ms) of each call's event interval over the recorded steps."""
    names = ("route", "precompute", "fwd")
    outp = {}
    for c, name in enumerate(names):
        x = np.array([e[c].elapsed_time(e[c + 1]) for e in evs])
        outp[name] = {"mean": float(x.mean()), "median": float(np.median(x)), "min": float(x.min())}
    return outp


TIE_GAP = 1e-5   # rows whose k-th and (k+1)-th block scores are this close may route either way


def parity_check(w: I.Workload, refs, lut_gpu, o_gpu):
    """The timed run's LUT and O against the oracle, on every query block of the sampled heads:
    LUT rows bit-exact outside tie rows; O within max-abs 2e-2 and mean-rel 1e-2 (bf16/FP8) or
    max-abs 1e-4 (fp32) on the query blocks whose LUT row equals the oracle's."""
    tol_abs = 2e-2 if w.dtype == "bf16" else 1e-4
    tol_rel = 1e-2 if w.dtype == "bf16" else None
    lut_diff = ties = 0
    err_max = err_sum = ref_sum = 0.0
    n_el = 0
    for h, r in enumerate(refs):
        g = lut_gpu[0, h]
        srt = -np.sort(-r["scores"], axis=1)
        tie = (srt[:, w.topk - 1] - srt[:, w.topk]) <= TIE_GAP if w.topk < w.T else np.zeros(w.T, bool)
        same = np.all(g == r["lut"], axis=1)
        ties += int(tie.sum())
        lut_diff += int(np.sum(~same & ~tie))
        rows = np.repeat(same, 64)[:w.N]
        d = np.abs(o_gpu[0, h][rows].astype(np.float64) - r["o"][rows])
        err_max = max(err_max, float(d.max()) if d.size else 0.0)
        err_sum += float(d.sum())
        ref_sum += float(np.abs(r["o"][rows]).sum())
        n_el += d.size
    mean_rel = err_sum / max(ref_sum, 1e-30)
    ok = lut_diff == 0 and err_max <= tol_abs and (tol_rel is None or mean_rel <= tol_rel)
    return {"heads": len(refs), "query_blocks": len(refs) * w.T, "lut_rows_diff": lut_diff,
            "tie_rows": ties, "o_elements": n_el, "max_abs": float(f"{err_max:.4g}"),
            "mean_rel": float(f"{mean_rel:.4g}"), "tol_max_abs": tol_abs, "tol_mean_rel": tol_rel,
            "ok": bool(ok)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C2", choices=sorted(I.CONFIGS))
    ap.add_argument("--cpu-heads", type=int, default=12,
                    help="heads in the CPU oracle sample, also checked against the timed run (0 = skip)")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="steps timed after a 1 GiB cache-evicting read each (0 = skip)")
    ap.add_argument("--backward", action="store_true",
                    help="also time sla2_attention_bwd (default for the C4 fine-tuning workload)")
    ap.add_argument("--pv-fp8", type=int, default=1,
                    help="also time the low-bit P.V forward (e4m3 P and V) on FP8 workloads (0 = skip)")
    ap.add_argument("--soft-tau", type=float, default=0.001,
                    help="temperature of the separately timed SoftTop-k router leg (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (HBM counter scaling) and exit")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path (heads would shard across GPUs with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_linear_attention_pool_amd import binding as Bn

    w = I.CONFIGS[args.config]
    log(f"[bench] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} T={w.T} topk={w.topk}")
    inp = I.generate(w)
    dev = torch.device("cuda:0")
    el = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d_in = {k: torch.from_numpy(inp[k]).to(el).to(dev) for k in ("q", "k", "v")}
    d_in["alpha"] = torch.from_numpy(inp["alpha"]).to(dev)
    d_in["wq"] = None if inp["wq"] is None else torch.from_numpy(inp["wq"]).to(dev)
    d_in["wk"] = None if inp["wk"] is None else torch.from_numpy(inp["wk"]).to(dev)
    p = Bn.make_params(w.B, w.H, w.N, w.d, w.topk, w.dtype, w.qk_mode)
    want_bwd = args.backward or args.config == "C4"
    bufs = Bn.allocate(p, dev, per_block_stats=(w.dtype != "bf16"), with_lse=want_bwd,
                       with_bwd=want_bwd)
    t = dict(bufs)
    t.update(d_in)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        Bn.sla2_route(p, t, stream)
        if ev is not None:
            ev[1].record(stream)
        Bn.sla2_linear_precompute(p, t, stream)
        if ev is not None:
            ev[2].record(stream)
        Bn.sla2_attention_fwd(p, t, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup {args.warmup} done")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    warm = pass_times(evs)
    t_route, t_pre, t_fwd = warm["route"]["mean"], warm["precompute"]["mean"], warm["fwd"]["mean"]
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (wall {wall / args.steps * 1e3:.4f} ms); "
        f"route {t_route:.4f} precompute {t_pre:.4f} fwd {t_fwd:.4f} ms")
    # the timed run's outputs, before any other leg touches the buffers
    lut = bufs["lut"].cpu().numpy()
    o_gpu = bufs["o"].float().cpu().numpy() if args.cpu_heads > 0 else None

    # cold passes: a read of 1 GiB (four times the 256 MB MALL) before each step, so every pass
    # starts from memory that is not in any cache.  The sweep only reads: a fill would leave up
    # to the whole MALL dirty, and the first pass after it would pay for writing that back.  The
    # buffer is filled once, and one untimed sweep takes that fill's dirty lines out first.
    # Per-pass events as above.
    cold = None
    if args.cold_reps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        flush.fill_(1.0)
        sink = flush.sum()
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.cold_reps)]
        for k in range(args.cold_reps):
            sink += flush.sum()
            step(evc[k])
        torch.cuda.synchronize(dev)
        cold = pass_times(evc)
        del flush, sink
        log(f"[bench] cold (MALL flushed), median: route {cold['route']['median']:.4f} precompute "
            f"{cold['precompute']['median']:.4f} fwd {cold['fwd']['median']:.4f} ms")
    f_sparse = A.sparse_flops_from_lut(lut, w.N, w.d)
    f_lin = A.linear_flops(w.B, w.H, w.N, w.d)
    f_eff = f_sparse + f_lin
    tflops = f_eff / (ms_step * 1e-3) / 1e12

    # dominant kernel: the fused forward.  Its routed-block work is half FP8 (Q.K^T) and half
    # bf16 (P.V); the peak for that mix is F / (F/2 / P_fp8 + F/2 / P_bf16).
    fp8 = w.qk_mode == "fp8"
    peak = (1.0 / (0.5 / PEAK_FP8 + 0.5 / PEAK_BF16)) if fp8 else PEAK_BF16
    achieved = f_sparse / (t_fwd * 1e-3) / 1e12
    kb = kernel_bytes(w)
    passes = {
        "route_ms": round(float(t_route), 5),
        "route_GBps": round(kb["route"] / (t_route * 1e-3) / 1e9, 1),
        "precompute_ms": round(float(t_pre), 5),
        "precompute_GBps": round(kb["precompute"] / (t_pre * 1e-3) / 1e9, 1),
        "fwd_ms": round(float(t_fwd), 5),
        "fwd_routed_TFLOPS": round(achieved, 2),
        "warm": {k: {s: round(float(v), 5) for s, v in st.items()} for k, st in warm.items()},
    }
    if cold is not None:
        passes["cold"] = {k: {s: round(float(v), 5) for s, v in st.items()} for k, st in cold.items()}
        passes["cold_GBps_median"] = {
            "route": round(kb["route"] / (cold["route"]["median"] * 1e-3) / 1e9, 1),
            "precompute": round(kb["precompute"] / (cold["precompute"]["median"] * 1e-3) / 1e9, 1)}
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOPS (effective: routed-block + linear-branch FLOPs per step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 QK^T + bf16" if fp8 else w.dtype,
        "data": "synthetic (seeded 3D sinusoidal PE + 0.5 N(0,1) for Q,K; N(0,1) V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "block": 64,
                   "topk": w.topk, "T": w.T, "sparsity": round(1 - w.topk / w.T, 4),
                   "grid": list(w.grid) if w.grid else None, "seed": w.seed,
                   "effective_GFLOP": round(f_eff / 1e9, 3), "routed_GFLOP": round(f_sparse / 1e9, 3),
                   "linear_GFLOP": round(f_lin / 1e9, 3)},
        "roofline": {"kernel": "fwd_mfma_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name)},
        "passes": passes,
    }
    if want_bwd:
        # the fine-tuning step's backward on the forward's buffers, timed alone
        dout = torch.from_numpy(I.generate(w, with_dout=True)["dout"]).to(el).to(dev)
        grads = {k: torch.empty_like(d_in["q"]) for k in ("dq", "dk", "dv")}
        dal = torch.empty((w.H, w.d), dtype=torch.float32, device=dev)
        def bwd():
            Bn.sla2_attention_bwd(p, t, dout, grads["dq"], grads["dk"], grads["dv"], dal, stream)
        for _ in range(2):
            bwd()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for _ in range(args.steps):
            bwd()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        t_bwd = e0.elapsed_time(e1) / args.steps
        # the four gradient products of the routed blocks (dP, dV, dQ, dK): 2 x the forward's two
        f_bwd = 2 * f_sparse
        passes["bwd_ms"] = round(float(t_bwd), 5)
        passes["bwd_routed_TFLOPS"] = round(f_bwd / (t_bwd * 1e-3) / 1e12, 2)
        passes["train_step_ms"] = round(float(ms_step + t_bwd), 5)
        log(f"[bench] sla2_attention_bwd: {t_bwd:.4f} ms ({passes['bwd_routed_TFLOPS']} TFLOP/s over the 4 routed "
            f"gradient products)")
    if args.pv_fp8 and w.qk_mode == "fp8":
        # the low-bit P.V forward (SLA2 page, section 5: P and V in e4m3 too) on the same inputs,
        # in its own buffers, timed like the main step
        p8 = Bn.make_params(w.B, w.H, w.N, w.d, w.topk, w.dtype, "fp8pv")
        t8 = dict(Bn.allocate(p8, dev, per_block_stats=False))
        t8.update(d_in)
        ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

        def step8(ev=None):
            if ev is not None:
                ev[0].record(stream)
            Bn.sla2_route(p8, t8, stream)
            Bn.sla2_linear_precompute(p8, t8, stream)
            if ev is not None:
                ev[1].record(stream)
            Bn.sla2_attention_fwd(p8, t8, stream)
            if ev is not None:
                ev[2].record(stream)
        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize(dev)
        for k in range(args.steps):
            step8(ev8[k])
        torch.cuda.synchronize(dev)
        t8_step = np.mean([e[0].elapsed_time(e[2]) for e in ev8])
        t8_pre = np.mean([e[0].elapsed_time(e[1]) for e in ev8])
        t8_fwd = np.mean([e[1].elapsed_time(e[2]) for e in ev8])
        passes["pv_fp8_step_ms"] = round(float(t8_step), 5)
        passes["pv_fp8_route_precompute_ms"] = round(float(t8_pre), 5)
        passes["pv_fp8_fwd_ms"] = round(float(t8_fwd), 5)
        passes["pv_fp8_fwd_routed_TFLOPS"] = round(f_sparse / (t8_fwd * 1e-3) / 1e12, 2)
        log(f"[bench] low-bit P.V step: {t8_step:.4f} ms (route + precompute {t8_pre:.4f}, fwd {t8_fwd:.4f} ms, "
            f"{passes['pv_fp8_fwd_routed_TFLOPS']} TFLOP/s routed-block)")
    if args.soft_tau > 0:
        # the training router (not part of the inference step): sla2_route_soft on the same
        # inputs, timed alone; its SoftTop-k kernel runs kSoftSteps fp64 sigmoid sums per row
        T = w.T
        soft = torch.empty((w.B, w.H, T, T), dtype=torch.float32, device=dev)
        lam = torch.empty((w.B, w.H, T), dtype=torch.float32, device=dev)
        for _ in range(2):
            Bn.sla2_route_soft(p, t, args.soft_tau, soft, lam, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for _ in range(args.steps):
            Bn.sla2_route_soft(p, t, args.soft_tau, soft, lam, stream)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        t_soft = e0.elapsed_time(e1) / args.steps
        passes["soft_route_ms"] = round(float(t_soft), 5)
        passes["soft_route_tau"] = args.soft_tau
        log(f"[bench] sla2_route_soft (tau {args.soft_tau}): {t_soft:.4f} ms")
    ok = True
    if args.cpu_heads > 0:
        log(f"[bench] timing the CPU oracle on {args.cpu_heads} heads")
        out["cpu_baseline"], refs = cpu_baseline(w, inp, min(args.cpu_heads, w.H))
        out["parity"] = parity_check(w, refs, lut, o_gpu)
        ok = out["parity"]["ok"]
        log(f"[bench] parity of the timed run against the oracle: {out['parity']}")
    print(json.dumps(out), flush=True)
    if not ok:
        log("[bench] the timed run's output does not match the oracle")
        sys.exit(1)


if __name__ == "__main__":
    main()
