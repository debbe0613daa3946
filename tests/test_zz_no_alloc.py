"""sla2_route_noalloc, the router entry point that allocates nothing, against sla2_route.

Both calls run the same kernels, so every router output must agree bit for bit: the pooled
rows, the key mean, the LUT and mask, and in FP8 mode the Q codes and scales.  Two calls in a
row share the library's device scratch: the full 12-head layer first, then a smaller shape, so
a second call that read anything stale from the first would show.  Sizes beyond the scratch are
rejected before any launch."""
import numpy as np
import pytest

import sla2_inputs as I
from tests.gpu_util import params_for, say, to_device

pytestmark = pytest.mark.gpu

ROUTE_OUT = ("q_pool", "k_pool", "k_mean", "lut", "mask", "q8", "q_scale")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_linear_attention_pool_amd import binding  # noqa: F401  (fails loudly if unbuilt)
    yield


def _route_both(w):
    import torch
    from sparse_linear_attention_pool_amd import binding as Bn
    say(f"[noalloc] {w.name}: B={w.B} H={w.H} N={w.N} topk={w.topk} {w.qk_mode}")
    inp = I.generate(w)
    p = params_for(w)
    dev = to_device(w, inp)
    ref = Bn.allocate(p, "cuda")
    got = Bn.allocate(p, "cuda")
    for key in ROUTE_OUT:   # outputs the call must overwrite, filled with a pattern first
        got[key].view(torch.uint8).fill_(0xA5)
    ta = dict(ref)
    ta.update(dev)
    tb = {k: v for k, v in got.items() if k != "workspace"}
    tb.update(dev)
    Bn.sla2_route(p, ta)
    Bn.sla2_route_noalloc(p, tb)
    torch.cuda.synchronize()
    for key in ROUTE_OUT:
        a, b = ref[key], got[key]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{w.name}: {key} differs"
    say(f"[noalloc] {w.name}: every router output equal to sla2_route's")


def test_route_noalloc_matches_route_on_two_calls():
    _route_both(I.CONFIGS["C2"])                                   # 12 x 512 query blocks
    _route_both(I.make_workload("C2", grid=(5, 9, 41), H=3, seed=61, name="C2-shaped ragged N=1845"))


def test_route_noalloc_rejects_sizes_beyond_its_scratch():
    from sparse_linear_attention_pool_amd import binding as Bn
    w = I.CONFIGS["C3"]   # 40 x 1182 query blocks: far beyond the 64 MiB scratch
    p = params_for(w)
    with pytest.raises(Bn.SLA2Error) as e:
        Bn.sla2_route_noalloc(p, {})
    assert e.value.status == Bn.SLA2_ERR_UNSUPPORTED
    assert "scratch" in Bn.lib.sla2_last_error().decode()
