"""ctypes binding of libsla2.so: argument marshalling only.

Every step of the SLA2 forward runs in the library's HIP kernels; the
functions here turn torch device tensors into the pointers of the C ABI
declared in include/sla2.h, pass the current HIP stream, and raise on a
non-zero status.  torch provides device memory and streams only.

If the library has not been built this module raises at import: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsla2.so")

SLA2_OK, SLA2_ERR_INVALID_ARG, SLA2_ERR_UNSUPPORTED, SLA2_ERR_HIP = 0, -1, -2, -3
SLA2_F32, SLA2_BF16 = 0, 1
SLA2_QK_NATIVE, SLA2_QK_FP8_E4M3, SLA2_QK_PV_FP8_E4M3 = 0, 1, 2

ENTRY_POINTS = ("sla2_buffer_sizes", "sla2_route", "sla2_linear_precompute", "sla2_attention_fwd",
                "sla2_attention_bwd", "sla2_selftest_mfma", "sla2_route_soft", "sla2_route_noalloc",
                "sla2_status_string", "sla2_last_error")


class SLA2Error(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("smooth_k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("qk_mode", ctypes.c_int32), ("eps", ctypes.c_float)]


SIZE_FIELDS = ("q_pool", "k_pool", "k_mean", "lut", "mask", "q8", "k8", "q_scale", "k_scale",
               "h", "z", "h_sum", "z_sum", "o", "lse", "workspace", "workspace_bwd")


class Sizes(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in SIZE_FIELDS]


TENSOR_FIELDS = ("q", "k", "v", "wq", "wk", "alpha", "q_pool", "k_pool", "k_mean", "lut", "mask",
                 "q8", "q_scale", "k8", "k_scale", "h", "z", "h_sum", "z_sum", "o", "lse", "workspace",
                 "workspace_bwd")


class Tensors(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in TENSOR_FIELDS]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m sparse_linear_attention_pool_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, T = ctypes.POINTER(Params), ctypes.POINTER(Tensors)
    lib.sla2_buffer_sizes.argtypes = [P, ctypes.POINTER(Sizes)]
    for name in ("sla2_route", "sla2_route_noalloc", "sla2_linear_precompute", "sla2_attention_fwd"):
        getattr(lib, name).argtypes = [P, T, ctypes.c_void_p]
    lib.sla2_attention_bwd.argtypes = [P, T, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.sla2_selftest_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.sla2_status_string.restype = ctypes.c_char_p
    lib.sla2_status_string.argtypes = [ctypes.c_int]
    lib.sla2_last_error.restype = ctypes.c_char_p
    lib.sla2_last_error.argtypes = []
    lib.sla2_route_soft.argtypes = [P, T, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for name in ENTRY_POINTS[:8]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()
LIB_PATH = _LIB_PATH


def _check(fn: str, status: int) -> None:
    if status != SLA2_OK:
        raise SLA2Error(fn, status, lib.sla2_last_error().decode())


def make_params(B: int, H: int, N: int, d: int, topk: int, dtype: str = "bf16", qk_mode: str = "native",
                smooth_k: bool = True, eps: float = 1e-5) -> Params:
    return Params(B=B, H=H, N=N, d=d, block=64, topk=topk, smooth_k=int(bool(smooth_k)),
                  dtype={"f32": SLA2_F32, "bf16": SLA2_BF16}[dtype],
                  qk_mode={"native": SLA2_QK_NATIVE, "fp8": SLA2_QK_FP8_E4M3,
                           "fp8pv": SLA2_QK_PV_FP8_E4M3}[qk_mode], eps=eps)


def sla2_buffer_sizes(params: Params) -> Dict[str, int]:
    s = Sizes()
    _check("sla2_buffer_sizes", lib.sla2_buffer_sizes(ctypes.byref(params), ctypes.byref(s)))
    return {f: int(getattr(s, f)) for f in SIZE_FIELDS}


# element type each tensor field must have: "el" is the input dtype (bf16 or fp32); None takes
# any (byte buffers)
_F32, _I32, _U8, _EL = "float32", "int32", "uint8", "el"
_FIELD_DTYPE = {"q": _EL, "k": _EL, "v": _EL, "o": _EL, "h": _EL, "wq": _F32, "wk": _F32, "alpha": _F32,
                "q_pool": _F32, "k_pool": _F32, "k_mean": _F32, "h_sum": _F32, "z_sum": _F32, "z": _F32,
                "q_scale": _F32, "k_scale": _F32, "lse": _F32, "lut": _I32, "mask": _U8, "q8": _U8, "k8": _U8,
                "workspace": None, "workspace_bwd": None}


def _bytes_needed(params: Params, name: str, sizes: Optional[Dict[str, int]] = None) -> int:
    """Bytes the library reads or writes through tensor field `name` for these params."""
    el = 2 if params.dtype == SLA2_BF16 else 4
    tok = params.B * params.H * params.N * params.d * el
    if name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        return tok
    if name in ("alpha", "dalpha"):
        return params.H * params.d * 4
    if name in ("wq", "wk"):
        return params.d * params.d * 4
    T = (params.N + 63) // 64
    if name == "soft_mask":
        return params.B * params.H * T * T * 4
    if name == "lambda":
        return params.B * params.H * T * 4
    return (sizes if sizes is not None else sla2_buffer_sizes(params))[name]


def _ptr(x, params: Optional[Params] = None, name: str = "", dtype: Optional[str] = None,
         sizes: Optional[Dict[str, int]] = None) -> Optional[int]:
    """Device address of tensor x after checking, before anything is launched, that it is a
    contiguous device tensor of the expected element type, holds at least the bytes the library
    touches for `params`, and starts on a 16-byte boundary (the kernels use 16-byte loads and
    LDS copies).  None passes as NULL; a plain int passes through as a raw device address, for
    callers that manage the memory themselves."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    what = f"tensor '{name}'" if name else "tensor"
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if not x.is_cuda:
        raise ValueError(f"{what} must be a device tensor (got {x.device})")
    if dtype is not None and params is not None:
        want = ("bfloat16" if params.dtype == SLA2_BF16 else "float32") if dtype == _EL else dtype
        got = str(x.dtype).replace("torch.", "")
        if got != want:
            raise ValueError(f"{what} must be {want} (got {got})")
    if params is not None and name:
        need = _bytes_needed(params, name, sizes)
        have = x.numel() * x.element_size()
        if have < need:
            raise ValueError(f"{what} holds {have} bytes; these params need {need}")
    if x.data_ptr() % 16 != 0:
        raise ValueError(f"{what} must start on a 16-byte boundary (address {x.data_ptr():#x})")
    return x.data_ptr()


def _tensors(t: dict, params: Optional[Params] = None) -> Tensors:
    unknown = set(t) - set(TENSOR_FIELDS)
    if unknown:
        raise KeyError(f"unknown tensor names {sorted(unknown)}")
    sizes = sla2_buffer_sizes(params) if params is not None else None
    return Tensors(**{f: _ptr(t.get(f), params, f, _FIELD_DTYPE.get(f), sizes) for f in TENSOR_FIELDS})


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def sla2_route(params: Params, tensors: dict, stream=None) -> None:
    tt = _tensors(tensors, params)
    _check("sla2_route", lib.sla2_route(ctypes.byref(params), ctypes.byref(tt), _stream(stream)))


def sla2_route_noalloc(params: Params, tensors: dict, stream=None) -> None:
    """sla2_route with the router's scratch in the library's device array (no workspace)."""
    tt = _tensors(tensors, params)
    _check("sla2_route_noalloc", lib.sla2_route_noalloc(ctypes.byref(params), ctypes.byref(tt), _stream(stream)))


def sla2_route_soft(params: Params, tensors: dict, tau: float, soft_mask, lam, stream=None) -> None:
    """sla2_route plus the SoftTop-k mask: soft_mask float32 [B,H,T,T], lam float32 [B,H,T]."""
    tt = _tensors(tensors, params)
    _check("sla2_route_soft", lib.sla2_route_soft(ctypes.byref(params), ctypes.byref(tt), float(tau),
                                                  _ptr(soft_mask, params, "soft_mask", _F32),
                                                  _ptr(lam, params, "lambda", _F32), _stream(stream)))


def sla2_linear_precompute(params: Params, tensors: dict, stream=None) -> None:
    tt = _tensors(tensors, params)
    _check("sla2_linear_precompute",
           lib.sla2_linear_precompute(ctypes.byref(params), ctypes.byref(tt), _stream(stream)))


def sla2_attention_fwd(params: Params, tensors: dict, stream=None) -> None:
    tt = _tensors(tensors, params)
    _check("sla2_attention_fwd", lib.sla2_attention_fwd(ctypes.byref(params), ctypes.byref(tt), _stream(stream)))


def sla2_attention_bwd(params: Params, tensors: dict, dout, dq, dk, dv, dalpha, stream=None) -> None:
    tt = _tensors(tensors, params)
    _check("sla2_attention_bwd",
           lib.sla2_attention_bwd(ctypes.byref(params), ctypes.byref(tt), _ptr(dout, params, "dout", _EL),
                                  _ptr(dq, params, "dq", _EL), _ptr(dk, params, "dk", _EL),
                                  _ptr(dv, params, "dv", _EL), _ptr(dalpha, params, "dalpha", _F32),
                                  _stream(stream)))


def backward(params: Params, inputs: dict, buffers: dict, dout, stream=None) -> dict:
    """sla2_attention_bwd after `forward` ran on the same inputs and buffers (allocated with
    with_lse=True and with_bwd=True, which makes that forward store what the backward reads).
    Returns dq, dk, dv, dalpha."""
    import torch
    t = dict(buffers)
    for key in ("q", "k", "v", "alpha", "wq", "wk"):
        t[key] = inputs.get(key)
    q = inputs["q"]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dalpha = torch.empty((params.H, params.d), dtype=torch.float32, device=q.device)
    sla2_attention_bwd(params, t, dout, dq, dk, dv, dalpha, stream)
    return {"dq": dq, "dk": dk, "dv": dv, "dalpha": dalpha}


def sla2_selftest_mfma(which: int, a, b, d, stream=None) -> None:
    _check("sla2_selftest_mfma", lib.sla2_selftest_mfma(which, _ptr(a), _ptr(b), _ptr(d), _stream(stream)))


# --------------------------------------------------------------------------------------
# device buffers (torch allocations sized by sla2_buffer_sizes)
# --------------------------------------------------------------------------------------
def allocate(params: Params, device="cuda", with_lse: bool = False, per_block_stats: bool = True,
             with_bwd: bool = False) -> dict:
    """Allocate every output and scratch buffer the three calls need, on `device`.

    per_block_stats=False leaves out h and z (bf16 modes only): the forward pass reads
    only their sums, and the precompute then skips storing them.  with_bwd adds the
    backward pass's workspace (the backward also needs with_lse; it does not read h or z).
    """
    import torch
    sz = sla2_buffer_sizes(params)
    B, H, N, d = params.B, params.H, params.N, params.d
    T = (N + 63) // 64
    el = torch.bfloat16 if params.dtype == SLA2_BF16 else torch.float32
    out = {
        "q_pool": torch.empty((B, H, T, d), dtype=torch.float32, device=device),
        "k_pool": torch.empty((B, H, T, d), dtype=torch.float32, device=device),
        "k_mean": torch.empty((B, H, d), dtype=torch.float32, device=device),
        "lut": torch.empty((B, H, T, params.topk), dtype=torch.int32, device=device),
        "mask": torch.empty((B, H, T, T), dtype=torch.uint8, device=device),
        "h_sum": torch.empty((B, H, d, d), dtype=torch.float32, device=device),
        "z_sum": torch.empty((B, H, d), dtype=torch.float32, device=device),
        "o": torch.empty((B, H, N, d), dtype=el, device=device),
        "workspace": torch.empty(max(sz["workspace"], 256), dtype=torch.uint8, device=device),
    }
    if params.qk_mode in (SLA2_QK_FP8_E4M3, SLA2_QK_PV_FP8_E4M3):
        out["q8"] = torch.empty((B, H, T * 64, d), dtype=torch.uint8, device=device)
        out["k8"] = torch.empty((B, H, T * 64, d), dtype=torch.uint8, device=device)
        out["q_scale"] = torch.empty((B, H, T), dtype=torch.float32, device=device)
        out["k_scale"] = torch.empty((B, H, T), dtype=torch.float32, device=device)
    if per_block_stats or params.dtype != SLA2_BF16:
        out["h"] = torch.empty((B, H, T, d, d), dtype=el, device=device)
        out["z"] = torch.empty((B, H, T, d), dtype=torch.float32, device=device)
    if with_lse:
        out["lse"] = torch.empty((B, H, N), dtype=torch.float32, device=device)
    if with_bwd:
        if sz["workspace_bwd"] == 0:
            raise SLA2Error("allocate", SLA2_ERR_UNSUPPORTED, "no backward pass for these params")
        out["workspace_bwd"] = torch.empty(sz["workspace_bwd"], dtype=torch.uint8, device=device)
    for name, t in out.items():
        want = sz[name]
        have = t.numel() * t.element_size()
        if name in ("workspace", "workspace_bwd"):
            if have < want:
                raise RuntimeError("workspace too small")
        elif have != want:
            raise RuntimeError(f"buffer {name}: {have} bytes allocated, library expects {want}")
    return out


def forward(params: Params, inputs: dict, buffers: Optional[dict] = None, stream=None) -> dict:
    """Run route -> linear precompute -> fused forward on one stream.

    inputs: device tensors q, k, v [B,H,N,d] (bf16 or fp32), alpha [H,d] fp32,
    and optionally wq, wk [d,d] fp32.  Returns the buffer dict (o holds the output).
    """
    if buffers is None:
        buffers = allocate(params, inputs["q"].device)
    t = dict(buffers)
    for key in ("q", "k", "v", "alpha", "wq", "wk"):
        t[key] = inputs.get(key)
    sla2_route(params, t, stream)
    sla2_linear_precompute(params, t, stream)
    sla2_attention_fwd(params, t, stream)
    return buffers
