"""Python face of the CPU oracle for condensate attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg are the only callers allowed. The product path never imports this package, and this
package imports nothing from the product.

Functions take CPU torch tensors (float32 or bfloat16, contiguous) in the layouts
q [B][Hq][nq][d], k and v [B][Hkv][n][d], and return numpy/torch results in float64.
Each wraps one function of condensate_oracle.c, whose header maps every step to the
section of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "condensate_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
N_DIAG = 8


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("kv_heads", ctypes.c_int64),
        ("n", ctypes.c_int64), ("nq", ctypes.c_int64), ("d", ctypes.c_int64),
        ("W", ctypes.c_int64), ("topk", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("threads", ctypes.c_int32),
    ]


def build(force: bool = False) -> str:
    """Compile condensate_oracle.c with gcc into liboracle.so (next to the source)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("CONDENSATE_ORACLE_LIB")   # mutation tests load a planted variant
        if path is None:
            path = build()   # (re)compiled when missing or older than its source
        L = ctypes.CDLL(path)
        P = ctypes.POINTER(Problem)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_condensate.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.oracle_condensate_rows.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp]
        L.oracle_restricted.argtypes = [P, vp, vp, vp, vp, i64, vp]
        L.oracle_restricted_rows.argtypes = [P, vp, vp, vp, vp, i64, vp, i64, vp]
        L.oracle_full.argtypes = [P, vp, vp, vp, vp]
        L.oracle_full_rows.argtypes = [P, vp, vp, vp, vp, i64, vp]
        L.oracle_scores.argtypes = [P, vp, vp, ctypes.c_int64, vp]
        L.oracle_threads.argtypes = [ctypes.c_int32]
        for f in (L.oracle_condensate, L.oracle_condensate_rows, L.oracle_restricted,
                  L.oracle_restricted_rows, L.oracle_full, L.oracle_full_rows, L.oracle_scores,
                  L.oracle_threads):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _prep(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("oracle takes CPU tensors")
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"oracle takes float32 or bfloat16, got {t.dtype}")
    return t.contiguous()


def problem(q, k, W: int, topk: int, threads: int = 0) -> Problem:
    B, Hq, nq, d = q.shape
    Bk, Hkv, n, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q/k shapes disagree")
    if q.dtype != k.dtype:
        raise ValueError("q/k dtypes disagree")
    return Problem(B, Hq, Hkv, n, nq, d, W, topk, 0 if q.dtype == torch.float32 else 1, threads)


def _ptr(t) -> int:
    return t.data_ptr() if isinstance(t, torch.Tensor) else t.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def flat_rows(q, rows) -> np.ndarray:
    """Flat query indices b*Hq*nq + h*nq + r of (b, h, r) triples (int64, in the given order)."""
    B, Hq, nq, _ = q.shape
    a = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    bad = (a < 0).any() or (a[:, 0] >= B).any() or (a[:, 1] >= Hq).any() or (a[:, 2] >= nq).any()
    if bad:
        raise ValueError("row outside the problem")
    return np.ascontiguousarray((a[:, 0] * Hq + a[:, 1]) * nq + a[:, 2])


def condensate(q, k, v, W: int, topk: int, threads: int = 0, rows=None):
    """Full method. Returns (idx int32 [B][Hq][nq][1+W+topk], out float64 [B][Hq][nq][d],
    diag float64 [B][Hq][nq][8] = tau, max|s|, eps, |C|, k', and the full-softmax mass of
    position 0, of the window without 0, of the top-k positions).
    With rows (a list of (b, h, r)), only those queries: results [len(rows)][...]."""
    q, k, v = _prep(q), _prep(k), _prep(v)
    p = problem(q, k, W, topk, threads)
    B, Hq, nq, d = q.shape
    lead = (B, Hq, nq) if rows is None else (len(rows),)
    idx = np.empty(lead + (1 + W + topk,), dtype=np.int32)
    out = np.empty(lead + (d,), dtype=np.float64)
    diag = np.empty(lead + (N_DIAG,), dtype=np.float64)
    if rows is None:
        _check(lib().oracle_condensate(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                       _ptr(out), _ptr(diag)), "oracle_condensate")
    else:
        fr = flat_rows(q, rows)
        _check(lib().oracle_condensate_rows(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fr),
                                            len(fr), _ptr(idx), _ptr(out), _ptr(diag)),
               "oracle_condensate_rows")
    return idx, out, diag


def restricted(q, k, v, idx, threads: int = 0, rows=None):
    """Softmax over each supplied set (rows of idx, -1 padded), times V. float64 [B][Hq][nq][d].
    With rows (a list of (b, h, r)), idx is [len(rows)][cap] and so is the result."""
    q, k, v = _prep(q), _prep(k), _prep(v)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    B, Hq, nq, d = q.shape
    p = problem(q, k, 1, 0, threads)
    if rows is None:
        if idx.shape[:3] != (B, Hq, nq):
            raise ValueError("idx shape disagrees with q")
        out = np.empty((B, Hq, nq, d), dtype=np.float64)
        _check(lib().oracle_restricted(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                       idx.shape[3], _ptr(out)), "oracle_restricted")
        return out
    fr = flat_rows(q, rows)
    if idx.ndim != 2 or idx.shape[0] != len(fr):
        raise ValueError("idx must be [len(rows)][cap]")
    out = np.empty((len(fr), d), dtype=np.float64)
    _check(lib().oracle_restricted_rows(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fr),
                                        len(fr), _ptr(idx), idx.shape[1], _ptr(out)),
           "oracle_restricted_rows")
    return out


def full(q, k, v, threads: int = 0, rows=None):
    """Plain causal attention in float64: [B][Hq][nq][d] (with rows: [len(rows)][d])."""
    q, k, v = _prep(q), _prep(k), _prep(v)
    p = problem(q, k, 1, 0, threads)
    B, Hq, nq, d = q.shape
    if rows is None:
        out = np.empty((B, Hq, nq, d), dtype=np.float64)
        _check(lib().oracle_full(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out)), "oracle_full")
        return out
    fr = flat_rows(q, rows)
    out = np.empty((len(fr), d), dtype=np.float64)
    _check(lib().oracle_full_rows(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fr), len(fr),
                                  _ptr(out)), "oracle_full_rows")
    return out


def scores(q, k, b: int, h: int, r: int):
    """Scores s_0..s_i (float64) of query row r of head h in batch b."""
    q, k = _prep(q), _prep(k)
    p = problem(q, k, 1, 0)
    B, Hq, nq, d = q.shape
    i = k.shape[2] - nq + r
    s = np.empty(i + 1, dtype=np.float64)
    flat = (b * Hq + h) * nq + r
    _check(lib().oracle_scores(ctypes.byref(p), _ptr(q), _ptr(k), flat, _ptr(s)), "oracle_scores")
    return s


def threads_used(requested: int = 0) -> int:
    return int(lib().oracle_threads(requested))
