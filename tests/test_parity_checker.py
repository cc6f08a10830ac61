"""The parity checker itself (tests/parity.py), on the CPU: fed the oracle's own results it
accepts them; fed planted mistakes of the kinds a kernel could make (a window row dropped, a
top-k member swapped for one far outside the tie band, a padding hole, an output row with a row
dropped from its softmax, weights rounded to bf16) it rejects them."""
import numpy as np
import pytest
import torch

import oracle
from sparse_transformer_attention_amd import synth

from parity import assert_outputs, check_format, check_sets_rows, compare_sets, positions_of


def case(dtype="bf16"):
    w = synth.Workload("t", batch=2, heads=4, kv_heads=2, d=32, n=400, nq=24, dtype=dtype, W=20,
                       topk=12, q_scale=2.0, needles_per_kv_head=3)
    x = synth.make_inputs(w, seed=17)
    idx, out, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    return w, x, idx, out, diag


def test_accepts_the_oracles_own_results():
    w, x, idx, out, diag = case()
    assert compare_sets(idx.copy(), idx, diag, x["q"], x["k"], w.W, w.topk) == 0
    assert assert_outputs(out.astype(np.float32), out, torch.bfloat16) < 1e-6
    rows = [(1, 3, 23), (0, 0, 0), (1, 2, 7)]
    ri, ro, rd = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk, rows=rows)
    pos = np.array([w.n - w.nq + r for (_, _, r) in rows])
    assert check_sets_rows(ri.copy(), ri, rd, pos, w.W, w.topk, lambda t: None) == 0


def test_rejects_a_dropped_window_row():
    w, x, idx, _, diag = case()
    bad = idx.copy()
    row = bad[0, 1, 5]
    i = w.n - w.nq + 5
    members = row[row >= 0]
    # Replace window position i-1 by a candidate not in the set (same size, still ascending
    # after re-sorting).
    outside = next(j for j in range(1, i - w.W + 1) if j not in set(members.tolist()))
    m = sorted((set(members.tolist()) - {i - 1}) | {outside})
    row[: len(m)] = m
    with pytest.raises(AssertionError):
        compare_sets(bad, idx, diag, x["q"], x["k"], w.W, w.topk)


def test_rejects_a_topk_swap_outside_the_band():
    w, x, idx, _, diag = case()
    bad = idx.copy()
    b, h, r = 1, 2, 9
    i = w.n - w.nq + r
    s = oracle.scores(x["q"], x["k"], b, h, r)
    row = bad[b, h, r]
    members = set(row[row >= 0].tolist())
    top = [j for j in members if 1 <= j <= i - w.W]
    # The best selected position swapped for the worst candidate: far outside the band.
    best = max(top, key=lambda j: s[j])
    worst = min((j for j in range(1, i - w.W + 1) if j not in members), key=lambda j: s[j])
    m = sorted((members - {best}) | {worst})
    row[: len(m)] = m
    with pytest.raises(AssertionError, match="outside the band"):
        compare_sets(bad, idx, diag, x["q"], x["k"], w.W, w.topk)


def test_rejects_padding_holes_and_wrong_sizes():
    w, _, idx, _, _ = case()
    pos = positions_of(w.nq, w.n, idx.shape[:3])
    flat = idx.reshape(-1, idx.shape[-1]).copy()
    check_format(flat, pos, w.W, w.topk)
    hole = flat.copy()
    hole[3, 1] = -1            # a hole inside the members
    with pytest.raises(AssertionError):
        check_format(hole, pos, w.W, w.topk)
    short = flat.copy()
    short[4, int((short[4] >= 0).sum()) - 1] = -1
    with pytest.raises(AssertionError, match="set size"):
        check_format(short, pos, w.W, w.topk)


def test_output_ceiling_catches_a_dropped_row_and_bf16_weights():
    w, x, idx, out, _ = case()
    # The softmax without one top-k member of each row.
    less = idx.copy()
    for row in less.reshape(-1, less.shape[-1]):
        members = row[row >= 0]
        if len(members) > 2:
            row[:] = np.concatenate([members[:1], members[2:], [-1] * (len(row) - len(members) + 1)])
    dropped = oracle.restricted(x["q"], x["k"], x["v"], less)
    with pytest.raises(AssertionError):
        assert_outputs(dropped.astype(np.float32), out, torch.bfloat16)
    # Weights rounded to bf16 before the V product, the sum kept in fp64: the numerator and
    # denominator disagree by up to 2^-9 per weight.
    q = x["q"].double()
    k = x["k"].double().repeat_interleave(w.group, dim=1)
    v = x["v"].double().repeat_interleave(w.group, dim=1)
    s = q @ k.transpose(-1, -2) / np.sqrt(w.d)
    mask = torch.zeros_like(s, dtype=torch.bool)
    ii = torch.from_numpy(idx.astype(np.int64))
    mask.scatter_(3, torch.where(ii >= 0, ii, torch.zeros_like(ii)), True)
    s = s.masked_fill(~mask, -np.inf)
    p = torch.exp(s - s.amax(dim=-1, keepdim=True))
    rounded = (p.float().to(torch.bfloat16).double() @ v) / p.sum(dim=-1, keepdim=True)
    with pytest.raises(AssertionError, match="ceiling"):
        assert_outputs(rounded.numpy().astype(np.float32), out, torch.bfloat16)
