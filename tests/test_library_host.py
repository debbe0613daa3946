"""Host-side checks of libsla2.so that need no GPU: symbols, sizes, argument errors."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla2.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def B():
    from sparse_linear_attention_pool_amd import binding
    return binding


def test_library_exports_every_declared_function(B):
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(B.lib, n), n
    assert set(B.ENTRY_POINTS) == set(names)


def test_buffer_sizes_c2(B):
    p = B.make_params(1, 12, 32760, 128, 15, "bf16", "fp8")
    s = B.sla2_buffer_sizes(p)
    T = 512
    assert s["lut"] == 12 * T * 15 * 4
    assert s["mask"] == 12 * T * T
    assert s["q8"] == 12 * T * 64 * 128 == s["k8"]
    assert s["h"] == 12 * T * 128 * 128 * 2
    assert s["o"] == 12 * 32760 * 128 * 2
    assert s["workspace"] % 256 == 0 and s["workspace"] > 0
    p32 = B.make_params(1, 2, 1024, 64, 4, "f32", "native")
    s32 = B.sla2_buffer_sizes(p32)
    assert s32["q8"] == 0 and s32["h"] == 2 * 16 * 64 * 64 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), -1), (dict(topk=0), -1), (dict(topk=17), -1), (dict(N=0), -1),
    (dict(block=32), -1), (dict(dtype=7), -1), (dict(qk_mode=5), -1), (dict(smooth_k=2), -1),
    (dict(eps=-1.0), -1), (dict(dtype=0, qk_mode=1), -2), (dict(dtype=0, qk_mode=2), -2),
    (dict(d=64, dtype=1, qk_mode=0), -2), (dict(d=64, dtype=1, qk_mode=2), -2),
    (dict(N=64 * 4097, topk=4), -2),
])
def test_invalid_params_are_rejected_before_any_launch(B, kw, status):
    base = dict(B=1, H=2, N=1024, d=64, block=64, topk=4, smooth_k=1, dtype=0, qk_mode=0, eps=1e-5)
    base.update(kw)
    p = B.Params(**base)
    s = B.Sizes()
    rc = B.lib.sla2_buffer_sizes(ctypes.byref(p), ctypes.byref(s))
    assert rc == status
    assert len(B.lib.sla2_last_error()) > 0
    t = B.Tensors()
    for fn in (B.lib.sla2_route, B.lib.sla2_linear_precompute, B.lib.sla2_attention_fwd):
        assert fn(ctypes.byref(p), ctypes.byref(t), None) == status


def test_missing_tensors_are_rejected(B):
    p = B.make_params(1, 2, 1024, 64, 4, "f32", "native")
    t = B.Tensors()
    assert B.lib.sla2_route(ctypes.byref(p), ctypes.byref(t), None) == B.SLA2_ERR_INVALID_ARG
    assert b"workspace" in B.lib.sla2_last_error()
    t.workspace = 256 * 7 + 3          # misaligned pointer, never dereferenced
    assert B.lib.sla2_route(ctypes.byref(p), ctypes.byref(t), None) == B.SLA2_ERR_INVALID_ARG
    assert b"aligned" in B.lib.sla2_last_error()
    t.workspace = 256 * 7
    assert B.lib.sla2_route(ctypes.byref(p), ctypes.byref(t), None) == B.SLA2_ERR_INVALID_ARG
    assert b"'q'" in B.lib.sla2_last_error()


def test_bf16_precompute_does_not_read_the_lut(B):
    """The precompute needs only the router's key mean: with every tensor it reads given and no
    LUT, argument checking passes and the call reaches its first launch, which fails on a
    machine without a GPU.  (Skipped where a GPU is present: the call would run.)"""
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    p = B.make_params(1, 2, 1024, 128, 4, "bf16", "fp8")
    t = B.Tensors()
    fake = 256 * 1024          # aligned, never dereferenced: no device runs the launch
    for name in ("workspace", "k", "v", "k_mean", "h_sum", "z_sum", "k8", "k_scale"):
        setattr(t, name, fake)
    assert B.lib.sla2_linear_precompute(ctypes.byref(p), ctypes.byref(t), None) == B.SLA2_ERR_HIP
    # and without k8 in FP8 mode it stops at the check, before any launch
    t.k8 = 0
    assert B.lib.sla2_linear_precompute(ctypes.byref(p), ctypes.byref(t), None) == B.SLA2_ERR_INVALID_ARG
    assert b"'k8'" in B.lib.sla2_last_error()


def test_soft_route_rejects_bad_tau_before_any_launch(B):
    p = B.make_params(1, 2, 1024, 64, 4, "f32", "native")
    t = B.Tensors()
    fake = 256 * 1024          # aligned, never dereferenced
    for name in ("workspace", "q", "k", "q_pool", "k_pool", "k_mean", "lut", "mask"):
        setattr(t, name, fake)
    for tau in (0.0, -0.5, float("nan"), float("inf")):
        assert B.lib.sla2_route_soft(ctypes.byref(p), ctypes.byref(t), tau, fake, fake, None) == \
            B.SLA2_ERR_INVALID_ARG
        assert b"tau" in B.lib.sla2_last_error()
    assert B.lib.sla2_route_soft(ctypes.byref(p), ctypes.byref(t), 0.1, None, fake, None) == B.SLA2_ERR_INVALID_ARG
    assert b"'soft_mask'" in B.lib.sla2_last_error()


def test_backward_reports_unsupported(B):
    # implemented for bf16 inputs with FP8 Q.K^T and d = 128 only
    p = B.make_params(1, 2, 1024, 64, 4, "f32", "native")
    with pytest.raises(B.SLA2Error) as e:
        B.sla2_attention_bwd(p, {"workspace": 256 * 1024}, None, None, None, None, None, stream=0)
    assert e.value.status == B.SLA2_ERR_UNSUPPORTED
    assert B.lib.sla2_status_string(-2) == b"unsupported"
    assert B.sla2_buffer_sizes(p)["workspace_bwd"] == 0
    # the backward is 16-bit: a low-bit P.V forward has none
    p8 = B.make_params(1, 2, 1024, 128, 4, "bf16", "fp8pv")
    with pytest.raises(B.SLA2Error) as e:
        B.sla2_attention_bwd(p8, {"workspace": 256 * 1024}, None, None, None, None, None, stream=0)
    assert e.value.status == B.SLA2_ERR_UNSUPPORTED
    assert B.sla2_buffer_sizes(p8)["workspace_bwd"] == 0


def test_low_bit_pv_workspace_holds_e4m3_v_tiles_and_exponents(B):
    # C2 shape: bf16 V^T tiles (100.7 MB) become e4m3 tiles (50.3 MB) plus one exponent byte per
    # (block, channel) (786 KB); everything else is the same
    s8 = B.sla2_buffer_sizes(B.make_params(1, 12, 32760, 128, 15, "bf16", "fp8"))
    s8pv = B.sla2_buffer_sizes(B.make_params(1, 12, 32760, 128, 15, "bf16", "fp8pv"))
    tiles = 12 * 512 * 128 * 64
    assert s8["workspace"] - s8pv["workspace"] == tiles - 12 * 512 * 128
    for key in ("q8", "k8", "q_scale", "k_scale", "o", "lse", "h", "z"):
        assert s8[key] == s8pv[key]


def test_backward_needs_the_forward_buffers(B):
    p = B.make_params(1, 12, 32760, 128, 15, "bf16", "fp8")
    sz = B.sla2_buffer_sizes(p)
    assert sz["workspace_bwd"] > 0
    fake = 256 * 1024          # aligned, never dereferenced: every call fails before a launch
    have = {"workspace": fake}
    # h and z (the per-block statistics) are not needed: the backward never forms H_i per block
    for name in ("q", "k", "v", "alpha", "k_mean", "lut", "mask", "q8", "q_scale", "k8", "k_scale",
                 "h_sum", "z_sum", "lse", "workspace_bwd"):
        with pytest.raises(B.SLA2Error) as e:
            B.sla2_attention_bwd(p, have, fake, fake, fake, fake, fake, stream=0)
        assert e.value.status == B.SLA2_ERR_INVALID_ARG and f"'{name}'" in str(e.value), (name, str(e.value))
        have[name] = fake
    with pytest.raises(B.SLA2Error) as e:
        B.sla2_attention_bwd(p, have, None, fake, fake, fake, fake, stream=0)
    assert "'dout'" in str(e.value)


def test_training_forward_rejects_a_misaligned_backward_workspace(B):
    # given the backward workspace, the forward also stores O_s, O_l and 1/den there
    p = B.make_params(1, 12, 32760, 128, 15, "bf16", "fp8")
    fake = 256 * 1024
    have = {name: fake for name in ("workspace", "q", "k", "v", "alpha", "lut", "h_sum", "z_sum", "o",
                                    "k_mean", "q8", "k8", "q_scale", "k_scale")}
    have["workspace_bwd"] = fake + 16
    with pytest.raises(B.SLA2Error) as e:
        B.sla2_attention_fwd(p, have, stream=0)
    assert e.value.status == B.SLA2_ERR_INVALID_ARG and "workspace_bwd" in str(e.value)


class _DeviceTensorStandIn:
    """What the binding reads of a torch device tensor, for checking its argument validation on a
    machine without a GPU (nothing here is ever dereferenced)."""

    def __init__(self, dtype, numel, address=1 << 20):
        self.dtype, self._numel, self._address = dtype, numel, address
        self.is_cuda, self.device = True, "cuda:0"

    def is_contiguous(self):
        return True

    def numel(self):
        return self._numel

    def element_size(self):
        import torch
        return torch.empty(0, dtype=self.dtype).element_size()

    def data_ptr(self):
        return self._address


def _fwd_tensors(B, p, **override):
    import torch
    el = torch.bfloat16
    tok = p.B * p.H * p.N * p.d
    sz = B.sla2_buffer_sizes(p)
    t = {"q": _DeviceTensorStandIn(el, tok), "k": _DeviceTensorStandIn(el, tok), "v": _DeviceTensorStandIn(el, tok),
         "alpha": _DeviceTensorStandIn(torch.float32, p.H * p.d),
         "lut": _DeviceTensorStandIn(torch.int32, sz["lut"] // 4),
         "workspace": _DeviceTensorStandIn(torch.uint8, sz["workspace"])}
    t.update(override)
    return t


@pytest.mark.parametrize("field,bad,msg", [
    ("q", "float32", "must be bfloat16"),
    ("lut", "int64", "must be int32"),
    ("q", "short", "holds"),
    ("workspace", "short", "holds"),
    ("v", "misaligned", "16-byte boundary"),
    ("k", "host", "device tensor"),
    ("alpha", "strided", "contiguous"),
])
def test_binding_rejects_bad_tensors_before_any_call(B, field, bad, msg, monkeypatch):
    """Each tensor is checked (device, element type, size for these params, 16-byte alignment,
    contiguity) in the binding, before the library is called."""
    import torch
    p = B.make_params(1, 2, 1000, 128, 3, "bf16", "fp8")
    good = _fwd_tensors(B, p)
    x = good[field]
    if bad == "float32":
        bad_t = _DeviceTensorStandIn(torch.float32, x.numel())
    elif bad == "int64":
        bad_t = _DeviceTensorStandIn(torch.int64, x.numel())
    elif bad == "short":
        bad_t = _DeviceTensorStandIn(x.dtype, x.numel() - 1)
    elif bad == "misaligned":
        bad_t = _DeviceTensorStandIn(x.dtype, x.numel(), address=(1 << 20) + 8)
    elif bad == "host":
        bad_t = torch.zeros(x.numel(), dtype=x.dtype)
    else:
        bad_t = torch.zeros(2, p.H * p.d, dtype=torch.float32).t()
    called = []
    monkeypatch.setattr(B, "lib", _RecordingLib(B.lib, called))
    with pytest.raises(ValueError, match=msg):
        B.sla2_linear_precompute(p, dict(good, **{field: bad_t}), stream=0)
    assert called == []


class _RecordingLib:
    """The library with its compute entry points recorded instead of called."""

    def __init__(self, lib, called):
        self._lib, self._called = lib, called

    def __getattr__(self, name):
        if name in ("sla2_buffer_sizes", "sla2_last_error", "sla2_status_string"):
            return getattr(self._lib, name)

        def rec(*args):
            self._called.append(name)
            return 0
        return rec


def test_a_failing_hip_call_maps_to_err_hip(B):
    """On a machine without a GPU the no-alloc router's first HIP call (the device query, before
    anything is launched) fails; the library returns SLA2_ERR_HIP with HIP's message, and the
    binding raises it with that status.  (Skipped where a GPU is present: the call would run.)"""
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    p = B.make_params(1, 2, 1000, 128, 3, "bf16", "fp8")
    fake = {f: 1 << 20 for f in ("q", "k", "q_pool", "k_pool", "k_mean", "lut", "mask", "q8", "q_scale")}
    with pytest.raises(B.SLA2Error) as e:
        B.sla2_route_noalloc(p, fake, stream=0)
    assert e.value.status == B.SLA2_ERR_HIP == -3
    assert "sla2_route_noalloc" in str(e.value) and "device" in str(e.value)
    assert B.lib.sla2_status_string(B.SLA2_ERR_HIP) == b"HIP runtime error"


def test_selftest_rejects_unknown_modes_before_any_launch(B):
    for which in (-1, 5):
        assert B.lib.sla2_selftest_mfma(which, None, None, None, None) == B.SLA2_ERR_INVALID_ARG
        assert b"which must be 0 to 4" in B.lib.sla2_last_error()
