"""Comparison of the HIP path's results with the oracle's, with the acceptance rule:

  index sets  -- the anchor and the window must match exactly; in the top-k part, a position
                 may differ only if its oracle score lies within 1e-5 * max_j |s_ij| of the
                 oracle's k-th selected score (the tie band); the part must have k' members;
  outputs     -- compared with the oracle's restricted softmax on the GPU's own set:
                 max_t |o_gpu - o_ref| / max_t |o_ref| <= 1e-5 (float32 inputs) or 2e-2
                 (bfloat16 inputs, float32 accumulation).

Beyond that acceptance bound each path also has a ceiling on the error it actually reaches
(CEILING): every path keeps its weights in fp32, so a dropped or double-counted row, or
weights rounded to bf16, shows up far below 2e-2.

Every check is vectorised over rows; the band test needs the oracle's scores only for the
rows whose sets differ.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BAND = 1e-5
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
# Achieved-error ceilings (relative, max-norm per row) of the method's outputs: fp32 scores,
# fp32 softmax weights and fp32 sums against the float64 oracle on the same input bits.
CEILING = {torch.float32: 1e-5, torch.bfloat16: 1e-4}


def check_format(arr: np.ndarray, pos: np.ndarray, W: int, topk: int):
    """Rows of out_idx ([R][cap]) at positions pos ([R]): C_i ascending, distinct, trailing -1
    padding, |C_i| = min(i+1, 1+W+k), position 0 first, the whole window {i-W+1..i} last, and
    k' = min(k, |R_i|) members in R_i = {1..i-W}."""
    R, cap = arr.shape
    assert cap == 1 + W + topk
    pos = np.asarray(pos, dtype=np.int64)
    valid = arr >= 0
    cnt = valid.sum(axis=1)
    want = np.minimum(pos + 1, cap)
    bad = np.nonzero(cnt != want)[0]
    assert bad.size == 0, f"set size: row {bad[0]} has {cnt[bad[0]]}, expected {want[bad[0]]}"
    prefix = np.arange(cap)[None, :] < cnt[:, None]
    assert np.array_equal(valid, prefix), "padding must be trailing -1"
    a = arr.astype(np.int64)
    asc = (np.diff(a, axis=1) > 0) | ~valid[:, 1:]
    assert asc.all(), f"row {np.nonzero(~asc.all(axis=1))[0][0]} not ascending and distinct"
    rr = np.arange(R)
    assert (a[:, 0] == 0).all(), "anchor (position 0) missing"
    assert (a[rr, cnt - 1] == pos).all(), "the query's own position must be the last member"
    wlo = np.maximum(0, pos - W + 1)
    wcount = pos - wlo + 1
    # Ascending distinct integers: wcount of them from wlo to i are exactly wlo..i.
    assert (a[rr, cnt - wcount] == wlo).all(), "window incomplete"
    in_r = (a >= 1) & (a <= (pos - W)[:, None])
    kp = np.minimum(topk, np.maximum(0, pos - W))
    assert (in_r.sum(axis=1) == kp).all(), "top-k part must have k' members"


def check_sets_rows(gpu: np.ndarray, ref: np.ndarray, diag: np.ndarray, pos, W: int, topk: int,
                    scores_of):
    """gpu, ref: [R][cap] int32 sets; diag: [R][8] oracle diagnostics; pos: [R] positions;
    scores_of(t): float64 oracle scores s_0..s_i of row t (asked only for rows whose sets
    differ). Both must be well-formed; they may differ only in the top-k part, and there only
    at positions inside the tie band. Returns the number of rows that differed."""
    pos = np.asarray(pos, dtype=np.int64)
    check_format(gpu, pos, W, topk)
    check_format(ref, pos, W, topk)
    differ = np.nonzero((gpu != ref).any(axis=1))[0]
    for t in differ:
        g = set(gpu[t][gpu[t] >= 0].tolist())
        o = set(ref[t][ref[t] >= 0].tolist())
        s = scores_of(int(t))
        tau, mabs = diag[t, 0], diag[t, 1]
        for j in g ^ o:
            assert 1 <= j <= pos[t] - W, f"row {t}: position {j} outside R_i differs"
            assert abs(s[j] - tau) <= BAND * mabs, (
                f"row {t}: position {j} (score {s[j]!r}) differs outside the band "
                f"around tau={tau!r} (band {BAND * mabs:.3g})")
    return int(differ.size)


def positions_of(nq: int, n: int, shape) -> np.ndarray:
    """Positions i = n - nq + r broadcast over an index array's leading [B][Hq][nq] shape."""
    r = np.arange(nq, dtype=np.int64)
    return np.broadcast_to(n - nq + r, shape).reshape(-1)


def compare_sets(gpu_idx, ref_idx, ref_diag, q, k, W, topk):
    """Whole problems: gpu_idx/ref_idx [B][Hq][nq][cap] int32, ref_diag [B][Hq][nq][8]; q, k:
    the CPU tensors the oracle read. Returns the number of rows that differed in the band."""
    B, Hq, nq, cap = gpu_idx.shape
    n = k.shape[2]
    pos = positions_of(nq, n, (B, Hq, nq))

    def scores_of(t):
        b, rest = divmod(t, Hq * nq)
        h, r = divmod(rest, nq)
        return oracle.scores(q, k, b, h, r)

    return check_sets_rows(gpu_idx.reshape(-1, cap), ref_idx.reshape(-1, cap),
                           ref_diag.reshape(-1, ref_diag.shape[-1]), pos, W, topk, scores_of)


def rel_err(gpu_out: np.ndarray, ref_out: np.ndarray) -> np.ndarray:
    """Per-row max-norm relative error."""
    num = np.abs(gpu_out.astype(np.float64) - ref_out).max(axis=-1)
    den = np.abs(ref_out).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def assert_outputs(gpu_out, ref_out, dtype, ceiling: float | None = None):
    """Acceptance (TOL) and the path's achieved-error ceiling (CEILING unless given)."""
    err = rel_err(gpu_out, ref_out)
    tol = TOL[dtype]
    assert np.all(err <= tol), f"max relative error {err.max():.3g} > {tol}"
    ceil = CEILING[dtype] if ceiling is None else ceiling
    assert np.all(err <= ceil), f"max relative error {err.max():.3g} above this path's ceiling {ceil}"
    return float(err.max())
