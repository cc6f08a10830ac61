"""Condensate ("topological") attention for MI355X (gfx950): Python binding of libcondensate.so.

This module only marshals arguments into the C ABI declared in include/condensate.h: every
step of the computation runs in the library's HIP kernels. PyTorch provides device memory and
the stream (torch.cuda.current_stream()). There is no CPU fallback: if the library is missing
or the tensors are not on the GPU, the calls raise.

Entry points (same names as the C ABI, without the `ca_` prefix):
    condensate_attention(q, k, v, n, d, heads, kv_heads, W, topk, out, out_idx)   synchronous
    condensate_attention_ex(p, q, k, v, out, out_idx, ws, stream=None)           asynchronous
    condensate_select(p, q, k, out_idx, ws, stream=None)                         stage 1
    attention_on_subset(p, q, k, v, idx, out, stream=None)                       stage 2
    workspace_size(p), status_string(rc), last_error()
plus `params(...)` to fill the parameter struct and `condensate(...)`, which allocates the
outputs and workspace with torch and calls condensate_attention_ex on the current stream.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcondensate.so")

CA_OK, CA_ERR_INVALID_ARG, CA_ERR_UNSUPPORTED, CA_ERR_WORKSPACE, CA_ERR_HIP = 0, -1, -2, -3, -4
CA_F32, CA_BF16 = 0, 1
CA_MAX_SET = 4096

EXPORTED = ("ca_condensate_attention", "ca_workspace_size", "ca_condensate_attention_ex",
            "ca_condensate_attention_mass_ex", "ca_dense_attention_ex", "ca_condensate_select",
            "ca_attention_on_subset", "ca_condensate_attention_noscratch",
            "ca_profile_start", "ca_profile_stop", "ca_status_string", "ca_last_error")


class Params(ctypes.Structure):
    """Mirror of ca_params."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("d", ctypes.c_int32), ("n", ctypes.c_int64), ("nq", ctypes.c_int64),
        ("W", ctypes.c_int32), ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
    ]


class KernelTime(ctypes.Structure):
    """Mirror of ca_kernel_time."""
    _fields_ = [("kernel", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class CondensateError(RuntimeError):
    def __init__(self, rc: int, what: str):
        self.rc = rc
        super().__init__(f"{what}: {status_string(rc)} -- {last_error()}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libcondensate.so (built by sparse_transformer_attention_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_transformer_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, P = ctypes.c_void_p, ctypes.POINTER(Params)
        L.ca_condensate_attention.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, vp, vp]
        L.ca_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        L.ca_condensate_attention_ex.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ca_condensate_attention_mass_ex.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ca_dense_attention_ex.argtypes = [P, vp, vp, vp, vp, vp]
        L.ca_condensate_select.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ca_attention_on_subset.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.ca_condensate_attention_noscratch.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.ca_profile_start.argtypes = [ctypes.c_int32]
        L.ca_profile_stop.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32)]
        L.ca_status_string.argtypes = [ctypes.c_int]
        L.ca_status_string.restype = ctypes.c_char_p
        L.ca_last_error.argtypes = []
        L.ca_last_error.restype = ctypes.c_char_p
        for f in (L.ca_condensate_attention, L.ca_workspace_size, L.ca_condensate_attention_ex,
                  L.ca_condensate_attention_mass_ex, L.ca_dense_attention_ex, L.ca_condensate_select,
                  L.ca_attention_on_subset, L.ca_condensate_attention_noscratch, L.ca_profile_start,
                  L.ca_profile_stop):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return load().ca_status_string(rc).decode()


def last_error() -> str:
    return load().ca_last_error().decode()


def _check(rc: int, what: str):
    if rc != CA_OK:
        raise CondensateError(rc, what)


def _dev_ptr(t, name: str, dtype=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def params(batch, heads, kv_heads, d, n, nq, W, topk, dtype, chunk=0) -> Params:
    dt = {torch.float32: CA_F32, torch.bfloat16: CA_BF16, "f32": CA_F32, "bf16": CA_BF16}.get(dtype, dtype)
    return Params(batch, heads, kv_heads, d, n, nq, W, topk, dt, chunk)


def params_for(q, k, W: int, topk: int, chunk: int = 0) -> Params:
    """Parameters read off q [B][Hq][nq][d] and k [B][Hkv][n][d]."""
    B, Hq, nq, d = q.shape
    Bk, Hkv, n, dk = k.shape
    if B != Bk or d != dk:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    return params(B, Hq, Hkv, d, n, nq, W, topk, q.dtype, chunk)


def workspace_size(p: Params) -> int:
    n = ctypes.c_size_t(0)
    _check(load().ca_workspace_size(ctypes.byref(p), ctypes.byref(n)), "ca_workspace_size")
    return int(n.value)


def condensate_attention(q, k, v, n, d, heads, kv_heads, W, topk, out, out_idx):
    """Synchronous one-call form: float32, batch 1, nq = n (see include/condensate.h)."""
    f32 = torch.float32
    _check(load().ca_condensate_attention(
        _dev_ptr(q, "q", f32), _dev_ptr(k, "k", f32), _dev_ptr(v, "v", f32), n, d, heads,
        kv_heads, W, topk, _dev_ptr(out, "out", f32), _dev_ptr(out_idx, "out_idx", torch.int32)),
        "ca_condensate_attention")


def condensate_attention_ex(p: Params, q, k, v, out, out_idx, ws, stream=None):
    dt = q.dtype
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().ca_condensate_attention_ex(
        ctypes.byref(p), _dev_ptr(q, "q", dt), _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
        _dev_ptr(out, "out", torch.float32), _dev_ptr(out_idx, "out_idx", torch.int32),
        _dev_ptr(ws, "ws"), ws_bytes, _stream_ptr(stream)), "ca_condensate_attention_ex")


def condensate_attention_noscratch(p: Params, q, k, v, out, out_idx, stream=None):
    """ca_condensate_attention_noscratch: as condensate_attention_ex with the library's own
    device array as workspace (nothing allocated; calls on one GPU must not overlap)."""
    dt = q.dtype
    _check(load().ca_condensate_attention_noscratch(
        ctypes.byref(p), _dev_ptr(q, "q", dt), _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
        _dev_ptr(out, "out", torch.float32), _dev_ptr(out_idx, "out_idx", torch.int32),
        _stream_ptr(stream)), "ca_condensate_attention_noscratch")


def condensate_attention_mass_ex(p: Params, q, k, v, out, out_idx, mass, ws, stream=None):
    """ca_condensate_attention_mass_ex: also mass float32 [B][Hq][nq][4] = (excluded mass,
    anchor, window without position 0, top-k) of the full causal softmax."""
    dt = q.dtype
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().ca_condensate_attention_mass_ex(
        ctypes.byref(p), _dev_ptr(q, "q", dt), _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
        _dev_ptr(out, "out", torch.float32), _dev_ptr(out_idx, "out_idx", torch.int32),
        _dev_ptr(mass, "mass", torch.float32), _dev_ptr(ws, "ws"), ws_bytes, _stream_ptr(stream)),
        "ca_condensate_attention_mass_ex")


def dense_attention_ex(p: Params, q, k, v, out, stream=None):
    """ca_dense_attention_ex: dense causal attention (bf16), out float32 [B][Hq][nq][d]."""
    dt = q.dtype
    _check(load().ca_dense_attention_ex(
        ctypes.byref(p), _dev_ptr(q, "q", dt), _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
        _dev_ptr(out, "out", torch.float32), _stream_ptr(stream)), "ca_dense_attention_ex")


def dense_attention(q, k, v, stream=None):
    """Dense causal attention of the last nq positions over all n keys (bf16 inputs)."""
    p = params_for(q, k, 1, 0, 0)
    B, Hq, nq, d = q.shape
    out = torch.empty((B, Hq, nq, d), dtype=torch.float32, device=q.device)
    dense_attention_ex(p, q, k, v, out, stream)
    return out


def condensate_select(p: Params, q, k, out_idx, ws, stream=None):
    dt = q.dtype
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().ca_condensate_select(
        ctypes.byref(p), _dev_ptr(q, "q", dt), _dev_ptr(k, "k", dt),
        _dev_ptr(out_idx, "out_idx", torch.int32), _dev_ptr(ws, "ws"), ws_bytes,
        _stream_ptr(stream)), "ca_condensate_select")


def attention_on_subset(p: Params, q, k, v, idx, out, stream=None):
    dt = q.dtype
    _check(load().ca_attention_on_subset(
        ctypes.byref(p), _dev_ptr(q, "q", dt), _dev_ptr(k, "k", dt), _dev_ptr(v, "v", dt),
        _dev_ptr(idx, "idx", torch.int32), _dev_ptr(out, "out", torch.float32),
        _stream_ptr(stream)), "ca_attention_on_subset")


def alloc_workspace(p: Params, device="cuda"):
    """A workspace for problem p (uninitialised: the library needs none)."""
    nbytes = workspace_size(p)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes else None


def condensate(q, k, v, W: int, topk: int, chunk: int = 0, ws=None, stream=None):
    """Allocate outputs (and the workspace unless given) and run the whole method on the
    current stream. Returns (out float32 [B][Hq][nq][d], out_idx int32 [B][Hq][nq][1+W+topk])."""
    p = params_for(q, k, W, topk, chunk)
    B, Hq, nq, d = q.shape
    out = torch.empty((B, Hq, nq, d), dtype=torch.float32, device=q.device)
    out_idx = torch.empty((B, Hq, nq, 1 + W + topk), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = alloc_workspace(p, q.device)
    condensate_attention_ex(p, q, k, v, out, out_idx, ws, stream)
    return out, out_idx


def condensate_mass(q, k, v, W: int, topk: int, chunk: int = 0, ws=None, stream=None):
    """As condensate(), with the mass diagnostic: returns (out, out_idx, mass float32
    [B][Hq][nq][4] = excluded mass, anchor, window without position 0, top-k)."""
    p = params_for(q, k, W, topk, chunk)
    B, Hq, nq, d = q.shape
    out = torch.empty((B, Hq, nq, d), dtype=torch.float32, device=q.device)
    out_idx = torch.empty((B, Hq, nq, 1 + W + topk), dtype=torch.int32, device=q.device)
    mass = torch.empty((B, Hq, nq, 4), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = alloc_workspace(p, q.device)
    condensate_attention_mass_ex(p, q, k, v, out, out_idx, mass, ws, stream)
    return out, out_idx, mass


def profile_start(reserve_launches: int = 0):
    """Start bracketing every launch of this library with HIP events (see ca_profile_start)."""
    _check(load().ca_profile_start(reserve_launches), "ca_profile_start")


def profile_stop() -> dict:
    """Stop profiling; returns {kernel name: (launches, total milliseconds)}."""
    arr = (KernelTime * 16)()
    n = ctypes.c_int32(0)
    _check(load().ca_profile_stop(arr, 16, ctypes.byref(n)), "ca_profile_stop")
    return {arr[i].kernel.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n.value)}
