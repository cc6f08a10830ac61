"""Comparison of the HIP path's results with the oracle's, with the acceptance rule:

  index sets  -- the anchor and the window must match exactly; in the top-k part, a position
                 may differ only if its oracle score lies within 1e-5 * max_j |s_ij| of the
                 oracle's k-th selected score (the tie band); the part must have k' members;
  outputs     -- compared with the oracle's restricted softmax on the GPU's own set:
                 max_t |o_gpu - o_ref| / max_t |o_ref| <= 1e-5 (float32 inputs) or 2e-2
                 (bfloat16 inputs, float32 accumulation).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BAND = 1e-5
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def check_row_format(row: np.ndarray, i: int, W: int, topk: int):
    members = row[row >= 0]
    n_pad = len(row) - len(members)
    assert np.all(row[len(members):] == -1), "padding must be trailing -1"
    assert np.all(np.diff(members) > 0), "ascending, distinct"
    assert len(members) == min(i + 1, 1 + W + topk), (len(members), i, W, topk)
    assert n_pad == len(row) - len(members)
    return members


def compare_sets(gpu_idx, ref_idx, ref_diag, q, k, W, topk, rows=None):
    """gpu_idx/ref_idx: [B][Hq][nq][cap] int32 (numpy); ref_diag: oracle diagnostics.
    q, k: the CPU tensors the oracle read. rows: iterable of (b, h, r) to check (default all).
    Returns the number of rows whose top-k part differed inside the band."""
    B, Hq, nq, cap = gpu_idx.shape
    n = k.shape[2]
    if rows is None:
        rows = [(b, h, r) for b in range(B) for h in range(Hq) for r in range(nq)]
    banded = 0
    for (b, h, r) in rows:
        i = n - nq + r
        g = check_row_format(gpu_idx[b, h, r], i, W, topk)
        o = check_row_format(ref_idx[b, h, r], i, W, topk)
        gs, os_ = set(g.tolist()), set(o.tolist())
        wlo = max(0, i - W + 1)
        fixed = {0} | set(range(wlo, i + 1))
        assert fixed <= gs, f"anchor/window missing at {(b, h, r)}"
        gt = {j for j in gs if 1 <= j <= i - W}
        ot = {j for j in os_ if 1 <= j <= i - W}
        kp = min(topk, max(0, i - W))
        assert len(gt) == kp == len(ot)
        if gt != ot:
            s = oracle.scores(q, k, b, h, r)
            tau, mabs = ref_diag[b, h, r, 0], ref_diag[b, h, r, 1]
            for j in gt ^ ot:
                assert abs(s[j] - tau) <= BAND * mabs, (
                    f"row {(b, h, r)}: position {j} (score {s[j]!r}) differs outside the band "
                    f"around tau={tau!r} (band {BAND * mabs:.3g})")
            banded += 1
    return banded


def rel_err(gpu_out: np.ndarray, ref_out: np.ndarray) -> np.ndarray:
    """Per-row max-norm relative error."""
    num = np.abs(gpu_out.astype(np.float64) - ref_out).max(axis=-1)
    den = np.abs(ref_out).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def assert_outputs(gpu_out, ref_out, dtype):
    err = rel_err(gpu_out, ref_out)
    tol = TOL[dtype]
    assert np.all(err <= tol), f"max relative error {err.max():.3g} > {tol}"
    return float(err.max())
