"""GPU parity of the HIP path against the CPU oracle, called through the C ABI.

Every case runs route -> linear precompute -> fused forward on seeded inputs
and compares, element by element, with the fp64 oracle:
* integer / byte results bit-exact: LUT and mask (outside rows whose k-th and
  (k+1)-th block scores are within 1e-5), FP8 codes and scales, k_mean;
* the output within max-abs 2e-2 and mean-rel 1e-2 (bf16 and FP8 paths) or
  max-abs 1e-4 (fp32 path).
Tie rows are judged with the oracle re-run on the GPU's LUT.
"""
import numpy as np
import pytest

import sla2_inputs as I
from oracle import sla2_oracle as O
from tests.gpu_util import (TOL_F32, TOL_LOWP, check_head, compare, oracle_head, run_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_linear_attention_pool_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    yield


# ----------------------------------------------------------------------------- matrix cores
def _bf16_bits(x):
    return I.bf16_bits(I.round_to_bf16(x.astype(np.float32)))


def test_mfma_bf16_operand_layout():
    import torch
    from sparse_linear_attention_pool_amd import binding as Bn
    rng = np.random.default_rng(0)
    A = I.round_to_bf16(rng.standard_normal((16, 32)).astype(np.float32))
    Bm = I.round_to_bf16(rng.standard_normal((32, 16)).astype(np.float32))
    a = np.zeros((64, 8), np.uint16)
    b = np.zeros((64, 8), np.uint16)
    for l in range(64):
        for e in range(8):
            a[l, e] = I.bf16_bits(A[l % 16, 8 * (l // 16) + e:8 * (l // 16) + e + 1])[0]
            b[l, e] = I.bf16_bits(Bm[8 * (l // 16) + e, l % 16:l % 16 + 1])[0]
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    dd = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    Bn.sla2_selftest_mfma(0, da, db, dd)
    d = dd.cpu().numpy()
    ref = A.astype(np.float64) @ Bm.astype(np.float64)
    got = np.zeros((16, 16))
    for l in range(64):
        for r in range(4):
            got[4 * (l // 16) + r, l % 16] = d[l, r]
    assert np.max(np.abs(got - ref)) < 1e-4


def test_mfma_fp8_operand_layout_and_scale():
    import torch
    from oracle import fp8_e4m3 as F8
    from sparse_linear_attention_pool_amd import binding as Bn
    rng = np.random.default_rng(1)
    ca = rng.integers(0, 256, (16, 128)).astype(np.uint8)
    cb = rng.integers(0, 256, (128, 16)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x38   # avoid NaN codes
    cb[(cb & 0x7F) == 0x7F] = 0x38
    a = np.zeros((64, 32), np.uint8)
    b = np.zeros((64, 32), np.uint8)
    for l in range(64):
        a[l] = ca[l % 16, 32 * (l // 16):32 * (l // 16) + 32]
        b[l] = cb[32 * (l // 16):32 * (l // 16) + 32, l % 16]
    dd = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    Bn.sla2_selftest_mfma(1, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), dd)
    d = dd.cpu().numpy()
    ref = F8.decode(ca) @ F8.decode(cb)
    got = np.zeros((16, 16))
    for l in range(64):
        for r in range(4):
            got[4 * (l // 16) + r, l % 16] = d[l, r]
    # a wrong lane layout pairs unrelated codes and gives O(1) relative errors; the
    # instruction's own accumulation is measured here at below 2^-12 of sum |a||b|
    absum = np.abs(F8.decode(ca)) @ np.abs(F8.decode(cb))
    rel = np.max(np.abs(got - ref) / (absum + 1e-30))
    say(f"    fp8 mfma: max |err| / sum|a||b| = {rel:.3e}")
    assert rel <= 2.0 ** -12


def test_mfma_fp8_scaled_operand_layout():
    """The scaled e4m3 product of the low-bit P.V path: lane l's E8M0 scale applies to row
    l % 16 of A and column l % 16 of B (every lane of a row carries the same exponent, as in the
    kernel), and the selected byte of the scale word is the one used."""
    import torch
    from oracle import fp8_e4m3 as F8
    from sparse_linear_attention_pool_amd import binding as Bn
    rng = np.random.default_rng(2)
    ca = rng.integers(0, 256, (16, 128)).astype(np.uint8)
    cb = rng.integers(0, 256, (128, 16)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x38
    cb[(cb & 0x7F) == 0x7F] = 0x38
    ea = rng.integers(-12, 13, 16)
    eb = rng.integers(-12, 13, 16)
    a = np.zeros((64, 36), np.uint8)
    b = np.zeros((64, 36), np.uint8)
    for l in range(64):
        a[l, :32] = ca[l % 16, 32 * (l // 16):32 * (l // 16) + 32]
        b[l, :32] = cb[32 * (l // 16):32 * (l // 16) + 32, l % 16]
    wa = rng.integers(0, 256, (64, 4)).astype(np.uint8)   # unused bytes hold noise
    wb = rng.integers(0, 256, (64, 4)).astype(np.uint8)
    for l in range(64):
        wa[l, 2] = 127 + ea[l % 16]
        wb[l, 0] = 127 + eb[l % 16]
    ab = np.concatenate([a[:, :32].reshape(-1), wa.reshape(-1)])
    bb = np.concatenate([b[:, :32].reshape(-1), wb.reshape(-1)])
    dd = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    Bn.sla2_selftest_mfma(3, torch.from_numpy(ab).cuda(), torch.from_numpy(bb).cuda(), dd)
    d = dd.cpu().numpy()
    ref = np.ldexp(F8.decode(ca), ea[:, None]) @ np.ldexp(F8.decode(cb), eb[None, :])
    absum = np.abs(np.ldexp(F8.decode(ca), ea[:, None])) @ np.abs(np.ldexp(F8.decode(cb), eb[None, :]))
    got = np.zeros((16, 16))
    for l in range(64):
        for r in range(4):
            got[4 * (l // 16) + r, l % 16] = d[l, r]
    rel = np.max(np.abs(got - ref) / (absum + 1e-30))
    say(f"    scaled fp8 mfma: max |err| / sum|a||b| = {rel:.3e}")
    assert rel <= 2.0 ** -12


def test_mfma_f64_operand_layout():
    import torch
    from sparse_linear_attention_pool_amd import binding as Bn
    rng = np.random.default_rng(2)
    # small integers: every product and sum is exact in fp64, so the result is bit-exact
    A = rng.integers(-64, 64, (16, 4)).astype(np.float64)
    Bm = rng.integers(-64, 64, (4, 16)).astype(np.float64)
    a = np.array([A[l % 16, l // 16] for l in range(64)])
    b = np.array([Bm[l // 16, l % 16] for l in range(64)])
    dd = torch.zeros((64, 4), dtype=torch.float64, device="cuda")
    Bn.sla2_selftest_mfma(2, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), dd)
    d = dd.cpu().numpy()
    got = np.zeros((16, 16))
    for l in range(64):
        for r in range(4):
            got[4 * r + l // 16, l % 16] = d[l, r]   # fp64 output rows are interleaved
    assert np.array_equal(got, A @ Bm)


# ----------------------------------------------------------------------------- whole path
SMALL = [
    # (base, overrides)
    ("C0", dict()),                                          # fp32, d=64, 16x16 blocks, topk 4
    ("C0", dict(N=1000, seed=10, name="C0 ragged N=1000")),  # partial last block (40 tokens)
    ("C0", dict(N=50, seed=11, name="C0 single partial block")),
    ("C0", dict(d=128, N=700, H=3, seed=12, name="fp32 d=128 ragged")),
    ("C1", dict(grid=(4, 16, 64), seed=21, name="C1-shaped bf16 N=4096")),
    ("C1", dict(grid=(3, 10, 37), seed=22, name="C1-shaped bf16 ragged N=1110")),
    ("C2", dict(grid=(4, 16, 64), seed=31, name="C2-shaped fp8 N=4096")),
    ("C2", dict(grid=(5, 9, 41), H=3, seed=32, name="C2-shaped fp8 ragged N=1845")),
    ("C2", dict(N=2000, seed=33, name="C2 fp8 unstructured ragged", B=2, H=2)),
    # low-bit P.V (e4m3 P and V with power-of-two scales) against the oracle's same mode
    ("C2", dict(grid=(4, 16, 64), seed=34, qk_mode="fp8pv", name="C2-shaped fp8 P.V N=4096")),
    ("C2", dict(grid=(5, 9, 41), H=3, seed=35, qk_mode="fp8pv", name="C2-shaped fp8 P.V ragged N=1845")),
    ("C2", dict(N=2000, seed=36, qk_mode="fp8pv", name="fp8 P.V unstructured ragged", B=2, H=2)),
]


@pytest.mark.parametrize("base,kw", SMALL, ids=[k.get("name", b) for b, k in SMALL])
def test_small_workloads_match_oracle(base, kw):
    w = I.make_workload(base, **kw)
    inp = I.generate(w)
    out = run_gpu(w, inp)
    for b in range(w.B):
        for h in range(w.H):
            say(f"  head ({b},{h})")
            check_head(w, inp, out, b, h)


@pytest.mark.parametrize("mode", ["f32", "bf16", "fp8", "fp8pv"])
def test_every_block_routed_is_softmax_attention(mode):
    base = {"f32": "C0", "bf16": "C1", "fp8": "C2", "fp8pv": "C2"}[mode]
    w = I.make_workload(base, grid=None, N=900, H=2, seed=40, d=(64 if mode == "f32" else 128),
                        qk_mode=("fp8pv" if mode == "fp8pv" else None), name=f"all routed {mode}")
    inp = I.generate(w)
    inp["alpha"][:] = 1.0
    T = w.T
    out = run_gpu(w, inp, topk=T)
    for h in range(w.H):
        check_head(w, inp, out, 0, h, topk=T)


@pytest.mark.parametrize("mode", ["bf16", "fp8", "fp8pv"])
def test_lut_rows_longer_than_a_wave(mode):
    # k_sel > 64: the forward reads the LUT row from memory instead of one register.  27% of
    # the blocks routed (the complement form of the linear branch in every mode), a ragged
    # last block
    base = "C1" if mode == "bf16" else "C2"
    w = I.make_workload(base, grid=None, N=16350, H=2, seed=42, qk_mode=("fp8pv" if mode == "fp8pv" else None),
                        name=f"k_sel 70 of 256 blocks, {mode}")
    inp = I.generate(w)
    out = run_gpu(w, inp, topk=70)
    T = w.T
    for h in range(w.H):
        check_head(w, inp, out, 0, h, topk=70, check_stats=(h == 0), query_blocks=[0, 1, 100, 177, T - 2, T - 1])


@pytest.mark.parametrize("N", [57000, 90000, 128000, 150000, 262144])
def test_router_tiers_up_to_the_largest_sequence(N):
    # T = 891, 1407, 2000, 2344 and 4096 blocks: the row selection's 16-, 24-, 32- and 64-slot
    # instances (keys per lane; 2344 fills 37 of 64 slots) after the scores kernel's partial key
    # ranges; 3% routed, so k_sel reaches 123: above 64 the selection skips its narrowing step,
    # and the forward reads its LUT rows from memory.  Router, quantiser and sampled query blocks.
    w = I.make_workload("C2", grid=None, N=N, H=1, seed=47, name=f"router tiers N={N}")
    inp = I.generate(w)
    out = run_gpu(w, inp)
    T = w.T
    check_head(w, inp, out, 0, 0, check_stats=False, query_blocks=[0, T // 2, T - 1])


@pytest.mark.parametrize("mode", ["native", "fp8", "fp8pv"])
def test_without_per_block_stats_matches_oracle(mode):
    # bf16 modes without h, z buffers: the precompute skips storing them and accumulates h_sum
    # in its matrix-core accumulators directly (the variant the benchmark runs)
    w = I.make_workload("C1" if mode == "native" else "C2", grid=(5, 9, 41), H=2, seed=49,
                        qk_mode=(None if mode == "native" else mode), name=f"no h/z buffers, {mode}")
    inp = I.generate(w)
    out = run_gpu(w, inp, per_block_stats=False)
    assert "h" not in out
    for h in range(w.H):
        check_head(w, inp, out, 0, h)   # h_sum and z_sum too; per-block h, z absent


@pytest.mark.parametrize("mode,k_sel", [(m, k) for m in ("native", "fp8") for k in (47, 48, 70)] +
                         [("fp8pv", k) for k in (31, 32, 47, 70)])
def test_large_routed_shares(mode, k_sel):
    # 94 blocks.  bf16 P.V: k_sel 47 keeps the complement form of the linear branch, 48 and 70
    # (more than half routed) sum the unrouted blocks directly.  Low-bit P.V switches at a
    # third (31: complement, 32 and up: direct, with bf16 V rows).  70: LUT row from memory.
    w = I.make_workload("C1" if mode == "native" else "C2", grid=None, N=6000, H=2, seed=51,
                        qk_mode=(None if mode == "native" else mode), name=f"k_sel {k_sel} of 94, {mode}")
    inp = I.generate(w)
    out = run_gpu(w, inp, topk=k_sel, per_block_stats=False)
    for h in range(w.H):
        check_head(w, inp, out, 0, h, topk=k_sel)


def test_smoothing_off_and_topk_one():
    w = I.make_workload("C2", grid=(2, 16, 64), seed=41, name="fp8 smooth_k=0 topk=1")
    inp = I.generate(w)
    out = run_gpu(w, inp, topk=1, smooth_k=False)
    assert not out["k_mean"].any()
    check_head(w, inp, out, 0, 0, topk=1, smooth_k=False)
    out = run_gpu(w, inp, topk=1, smooth_k=True)
    check_head(w, inp, out, 0, 5, topk=1, smooth_k=True)


def test_topk_exact_and_near_ties():
    """Router Top-k where the k-th and (k+1)-th scores tie exactly (repeated key blocks) or
    differ only far below the top 32 bits of their fp64 keys (one element 1 ulp apart)."""
    T = 24
    w = I.make_workload("C0", N=64 * T, H=2, seed=44, name="router ties")
    inp = I.generate(w)
    k = inp["k"]
    for j in range(6):
        k[:, :, (12 + j) * 64:(13 + j) * 64] = k[:, :, j * 64:(j + 1) * 64]
        blk = k[:, :, (6 + j) * 64:(7 + j) * 64].copy()
        blk[:, :, 5, 3] = np.nextafter(blk[:, :, 5, 3], np.float32(np.inf))
        k[:, :, (18 + j) * 64:(19 + j) * 64] = blk
    exact_hits = near_hits = 0
    for topk in range(1, T):
        out = run_gpu(w, inp, topk=topk, with_lse=False)
        for h in range(w.H):
            route = O.route_head(inp["q"][0, h], inp["k"][0, h], inp["wq"], inp["wk"], topk, True)
            sc, lut = route["scores"], out["lut"][0, h]
            for i in range(T):
                srt = np.sort(sc[i])[::-1]
                gap = srt[topk - 1] - srt[topk]
                exact_hits += gap == 0
                near_hits += 0 < gap < 1e-6 * abs(srt[topk - 1])
                # exact ties go to the lower index; every other gap here is far above fp64
                # rounding, so the choice must be the oracle's
                assert np.array_equal(lut[i], route["lut"][i]), (topk, h, i, lut[i], route["lut"][i])
    say(f"    boundary at an exact tie in {exact_hits} rows, at a near tie in {near_hits} rows")
    assert exact_hits > 0 and near_hits > 0


def test_runs_are_deterministic():
    w = I.make_workload("C2", grid=(4, 16, 64), seed=42, name="determinism")
    inp = I.generate(w)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for key in ("lut", "mask", "q8", "k8", "o", "h", "h_sum", "lse"):
        assert np.array_equal(a[key].all(), b[key].all()), key


def test_fp8_encoder_on_every_bf16_value():
    """Every finite bf16 value in [-448, 448] through the Q quantiser with scale exactly 1."""
    from oracle import fp8_e4m3 as F8
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    per_block = 64 * 128 - 1
    nblk = -(-len(vals) // per_block)
    q = np.zeros((nblk, 64 * 128), np.float32)
    for bi in range(nblk):
        chunk = vals[bi * per_block:(bi + 1) * per_block]
        q[bi, 0] = 448.0
        q[bi, 1:1 + len(chunk)] = chunk
    N = nblk * 64
    q = q.reshape(1, 1, N, 128)
    w = I.make_workload("C2", N=N, H=1, seed=43, name="fp8 encoder sweep", sparse_frac=1.0 / nblk)
    inp = I.generate(w)
    inp["q"] = q
    out = run_gpu(w, inp, topk=1)
    assert np.all(out["q_scale"].all() == 1.0)
    want = F8.encode(q.astype(np.float64)).reshape(1, 1, N, 128)
    got = out["q8"].all()
    bad = np.nonzero(got != want)
    assert len(bad[0]) == 0, f"{len(bad[0])} codes differ, e.g. value {q[bad][:5]} gpu {got[bad][:5]} want {want[bad][:5]}"


def test_fp8_decoder_on_every_code():
    """The kernels' e4m3 decode (the hardware conversion) against the e4m3 definition on all 256
    codes; the two NaN codes, which the quantiser never produces, decode to NaN."""
    import torch
    from oracle import fp8_e4m3 as F8
    from sparse_linear_attention_pool_amd import binding as Bn
    codes = np.arange(256, dtype=np.uint8)
    a = torch.from_numpy(codes.copy()).cuda()
    d = torch.zeros(256, dtype=torch.float32, device="cuda")
    Bn.sla2_selftest_mfma(4, a, a, d)
    torch.cuda.synchronize()
    got = d.cpu().numpy().astype(np.float64)
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(got[nan]))
    want = F8.decode(codes[~nan])
    assert np.array_equal(got[~nan], want), np.nonzero(got[~nan] != want)


# ----------------------------------------------------------------------------- full sizes
def _sampled_full(base, heads, blocks_per_head=6, **overrides):
    """Full-size run; parity of the listed heads on `blocks_per_head` sampled query blocks
    (always the first and the last), or on every query block when blocks_per_head is None."""
    w = I.make_workload(base, **overrides) if overrides else I.CONFIGS[base]
    say(f"[full] generating {w.name}")
    inp = I.generate(w)
    out = run_gpu(w, inp, with_lse=True)
    T = w.T
    rng = np.random.default_rng(123)
    for (b, h) in heads:
        if blocks_per_head is None:
            qb = None
            say(f"  head ({b},{h}) every query block")
        else:
            qb = sorted(set([0, T - 1] + rng.integers(0, T, blocks_per_head - 2).tolist()))
            say(f"  head ({b},{h}) query blocks {qb}")
        check_head(w, inp, out, b, h, query_blocks=qb, check_stats=(h == heads[0][1]))


def test_full_size_c1_sampled():
    _sampled_full("C1", [(0, 0), (0, 7)])


def test_full_size_c2_every_block():
    """The benchmark workload at its launch configuration: LUT, mask, quantiser codes and O of
    all 12 heads x 512 query blocks against the oracle."""
    _sampled_full("C2", [(0, h) for h in range(12)], blocks_per_head=None)


def test_full_size_c2_low_bit_pv_sampled():
    _sampled_full("C2", [(0, 0), (0, 11)], qk_mode="fp8pv", name="C2 fp8 P.V")


def test_full_size_c3_two_heads_every_block():
    _sampled_full("C3", [(0, 0), (0, 39)], blocks_per_head=None)
