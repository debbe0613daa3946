"""GPU parity of the SoftTop-k router (sla2_route_soft) against the fp64 oracle.

The soft mask M_ij = sigmoid((P_ij - lambda_i)/tau) and lambda_i come from the
same fp64 scores on both sides; they may differ only by the summation order of
the scores, the softmax and the row sums (about 1e-15 relative), which moves
lambda by far less than the float32 rounding of the outputs.  Bar: lambda and
every mask entry within 1e-6 absolute (float32 output rounding is 6e-8 on
[0, 1]), each row of the returned mask summing to k_sel within 1e-3 (float32
accumulation over T entries), and the hard LUT of the same call bit-exact
outside tie rows, as for sla2_route.
"""
import numpy as np
import pytest

import sla2_inputs as I
from oracle import sla2_oracle as O
from oracle import soft_topk as S
from tests.gpu_util import TIE_GAP, params_for, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_linear_attention_pool_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    yield


def _run_soft(w, inp, tau, topk=None, rows=None):
    import torch
    from sparse_linear_attention_pool_amd import binding as Bn
    k_sel = w.topk if topk is None else topk
    say(f"[gpu] soft route {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} topk={k_sel} tau={tau} {w.dtype}/{w.qk_mode}")
    p = params_for(w, topk)
    dev = to_device(w, inp)
    bufs = Bn.allocate(p, "cuda")
    t = dict(bufs)
    t.update(dev)
    T = (w.N + 63) // 64
    soft = torch.full((w.B, w.H, T, T), float("nan"), dtype=torch.float32, device="cuda")
    lam = torch.full((w.B, w.H, T), float("nan"), dtype=torch.float32, device="cuda")
    Bn.sla2_route_soft(p, t, tau, soft, lam)
    torch.cuda.synchronize()
    return soft.cpu().numpy(), lam.cpu().numpy(), bufs["lut"].cpu().numpy()


def _check(w, inp, tau, soft, lam, lut, topk=None, rows=None):
    k_sel = w.topk if topk is None else topk
    for b in range(w.B):
        for h in range(w.H):
            r = O.route_head(inp["q"][b, h], inp["k"][b, h], inp["wq"], inp["wk"], k_sel, True)
            sc = r["scores"] if rows is None else r["scores"][rows]
            _, M, L = S.soft_route_head(sc, k_sel, tau)
            gm = soft[b, h] if rows is None else soft[b, h][rows]
            gl = lam[b, h] if rows is None else lam[b, h][rows]
            assert np.all(np.isfinite(gm)), "mask entries left unwritten"
            err_m = np.max(np.abs(gm - M))
            if k_sel == sc.shape[1]:
                assert np.all(np.isneginf(gl))
                err_l = 0.0
            else:
                err_l = np.max(np.abs(gl - L))
            say(f"  head ({b},{h}): max |dM| {err_m:.2e}  max |dlambda| {err_l:.2e}")
            assert err_m < 1e-6 and err_l < 1e-6
            assert np.max(np.abs(gm.astype(np.float64).sum(axis=1) - k_sel)) < 1e-3
            # the hard LUT of the same call: bit-exact outside tie rows
            srt = np.sort(sc, axis=1)[:, ::-1]
            clear = (srt[:, k_sel - 1] - srt[:, k_sel] > TIE_GAP) if k_sel < sc.shape[1] else np.ones(len(sc), bool)
            gl_lut = lut[b, h] if rows is None else lut[b, h][rows]
            ol_lut = r["lut"] if rows is None else r["lut"][rows]
            assert np.array_equal(gl_lut[clear], ol_lut[clear])


@pytest.mark.parametrize("base,kw,tau", [
    ("C0", dict(), 0.05),
    ("C0", dict(N=1000, seed=10, name="C0 ragged N=1000"), 0.01),
    ("C0", dict(N=50, seed=11, name="C0 single partial block"), 0.1),
    ("C2", dict(grid=(5, 9, 41), H=3, seed=32, name="C2-shaped fp8 ragged N=1845"), 0.002),
    ("C1", dict(grid=(3, 10, 37), seed=22, name="C1-shaped bf16 ragged N=1110"), 0.02),
])
def test_soft_topk_small(base, kw, tau):
    w = I.make_workload(base, **kw)
    inp = I.generate(w)
    soft, lam, lut = _run_soft(w, inp, tau)
    _check(w, inp, tau, soft, lam, lut)


def test_soft_topk_every_block_and_one_block():
    w = I.make_workload("C0", N=700, H=2, seed=13, name="C0 k_sel = T and 1")
    inp = I.generate(w)
    T = (w.N + 63) // 64
    for k_sel in (T, 1):
        soft, lam, lut = _run_soft(w, inp, 0.03, topk=k_sel)
        _check(w, inp, 0.03, soft, lam, lut, topk=k_sel)


@pytest.mark.parametrize("N", [57000, 75600, 128000, 262144])
def test_soft_topk_large_sequences(N):
    """T = 891, 1182, 2000, 4096: the soft selection's 16-, 24-, 32- and 64-slot instances (the
    64-slot one at one wave per SIMD; T = 1182 is the C3 sequence length); 96 sampled rows
    checked."""
    w = I.make_workload("C2", grid=None, N=N, H=1, seed=48, name=f"soft tiers N={N}")
    inp = I.generate(w)
    T = (N + 63) // 64
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(5).integers(0, T, 94)]))
    soft, lam, lut = _run_soft(w, inp, 0.001)
    _check(w, inp, 0.001, soft, lam, lut, rows=rows)


def test_soft_topk_full_size_c2():
    """All 6,144 rows of the C2 router (12 heads x 512 query blocks, 512 key blocks each)."""
    w = I.CONFIGS["C2"]
    inp = I.generate(w)
    soft, lam, lut = _run_soft(w, inp, 0.001)
    _check(w, inp, 0.001, soft, lam, lut)


def test_tau_must_be_positive():
    import torch
    from sparse_linear_attention_pool_amd import binding as Bn
    w = I.CONFIGS["C0"]
    p = params_for(w)
    bufs = Bn.allocate(p, "cuda")
    t = dict(bufs)
    t.update(to_device(w, I.generate(w)))
    soft = torch.empty((1, 2, 16, 16), dtype=torch.float32, device="cuda")
    lam = torch.empty((1, 2, 16), dtype=torch.float32, device="cuda")
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(Bn.SLA2Error) as e:
            Bn.sla2_route_soft(p, t, bad, soft, lam)
        assert e.value.status == Bn.SLA2_ERR_INVALID_ARG
