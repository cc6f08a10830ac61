"""Pins of the CPU oracle to facts fixed by the pages and by the mathematics.

Each test checks the oracle against something other than itself: the set-size closed form
of Corollary 2 and the counts printed in the section 4.2 tables, the exclusion lemma of
section 3.2.1, brute-force enumeration of top-k subsets on tiny inputs, torch.topk, and
torch's scaled_dot_product_attention in float64 with membership masks (the special cases
"full attention" of section 1.1 and "Static (Anchor+Window)" of section 4.3 among them).
Page sections are those of the metaphor-xennon blog page on "The Condensate Theorem".
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from sparse_transformer_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make(B=1, Hq=2, Hkv=1, n=200, nq=1, d=16, W=16, topk=8, dtype="f32", seed=0, needles=0,
         q_scale=1.0, k_scale=1.0):
    w = synth.Workload("t", batch=B, heads=Hq, kv_heads=Hkv, d=d, n=n, nq=nq, dtype=dtype, W=W,
                       topk=topk, q_scale=q_scale, k_scale=k_scale, needles_per_kv_head=needles)
    return w, synth.make_inputs(w, seed)


def scores64(w, x):
    """Scores from torch's float64 matmul (independent of the oracle): [B][Hq][nq][n]."""
    q = x["q"].double()
    k = x["k"].double().repeat_interleave(w.group, dim=1)
    return torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(w.d)


def member_mask(w, idx):
    m = torch.zeros((w.batch, w.heads, w.nq, w.n + 1), dtype=torch.bool)
    ii = torch.from_numpy(idx.astype(np.int64))
    ii = torch.where(ii >= 0, ii, torch.full_like(ii, w.n))   # padding -> a spare column
    m.scatter_(3, ii, True)
    return m[..., : w.n]


def sdpa64(w, x, mask):
    q = x["q"].double()
    k = x["k"].double().repeat_interleave(w.group, dim=1)
    v = x["v"].double().repeat_interleave(w.group, dim=1)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask).numpy()


def positions(w):
    return [w.n - w.nq + r for r in range(w.nq)]


CASES = [
    dict(Hq=2, Hkv=1, n=200, nq=1, d=16, W=16, topk=8),
    dict(Hq=4, Hkv=2, n=300, nq=40, d=32, W=20, topk=12, dtype="bf16"),
    dict(Hq=1, Hkv=1, n=97, nq=97, d=8, W=8, topk=4),            # prefill with i < W rows
    dict(Hq=3, Hkv=3, n=64, nq=64, d=8, W=1, topk=5),             # W = 1
    dict(Hq=2, Hkv=2, n=50, nq=10, d=8, W=40, topk=30),           # k larger than |R|
    dict(Hq=2, Hkv=1, n=120, nq=7, d=16, W=10, topk=0),           # k = 0
    dict(B=2, Hq=8, Hkv=2, n=150, nq=3, d=64, W=32, topk=16, dtype="bf16"),
]


@pytest.mark.parametrize("case", CASES)
def test_set_structure_closed_form(case):
    """|C_i| = min(i+1, 1+W+k) <= 1+W+k (Corollary 2, section 2.4); C_i holds {0}, the whole
    window {i-W+1..i} and k' = min(k, |R_i|) positions of R_i = {1..i-W} (Definition 1)."""
    w, x = make(**case)
    idx, out, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    cap = 1 + w.W + w.topk
    for b, h, r in itertools.product(range(w.batch), range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        row = idx[b, h, r]
        members = row[row >= 0]
        assert np.all(row[len(members):] == -1), "padding must be trailing -1"
        assert np.all(np.diff(members) > 0), "ascending and distinct"
        assert len(members) == min(i + 1, cap) == diag[b, h, r, 3]
        assert members[0] == 0 and members[-1] == i
        wlo = max(0, i - w.W + 1)
        assert set(range(wlo, i + 1)) <= set(members.tolist())
        n_r = max(0, i - w.W)
        rest = [j for j in members.tolist() if 1 <= j <= i - w.W]
        assert len(rest) == min(w.topk, n_r) == diag[b, h, r, 4]


def test_golden_counts_section_4_2():
    """The pages print |C| = 97 for W=64, k=32 at every listed length (section 4.2.2 table),
    split 1 anchor + 64 window + 32 top-k (section 4.2.1 table)."""
    g = json.load(open(os.path.join(GOLDEN, "sec4_set_sizes.json")))
    W, topk = g["W"], g["topk"]
    for n_str, expect in g["set_size_by_sequence_length"].items():
        n = int(n_str)
        w, x = make(Hq=1, Hkv=1, n=n, nq=1, d=8, W=W, topk=topk, seed=n)
        idx, _, diag = oracle.condensate(x["q"], x["k"], x["v"], W, topk)
        members = idx[0, 0, 0][idx[0, 0, 0] >= 0]
        i = n - 1
        assert len(members) == expect == int(diag[0, 0, 0, 3])
        assert int(np.sum(members == 0)) == g["parts"]["anchor"]
        assert int(np.sum(members >= i - W + 1)) == g["parts"]["window"]
        assert int(np.sum((members >= 1) & (members <= i - W))) == g["parts"]["topk"]


@pytest.mark.parametrize("case", CASES[:5])
def test_exclusion_lemma(case):
    """Every excluded candidate scores at most tau_min, the k-th selected score (section 3.2.1),
    and tau is the k-th largest candidate score."""
    w, x = make(**case)
    idx, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    for b, h, r in itertools.product(range(w.batch), range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        if i - w.W < 1 or w.topk == 0:
            continue
        s = oracle.scores(x["q"], x["k"], b, h, r)
        members = set(idx[b, h, r][idx[b, h, r] >= 0].tolist())
        T = [j for j in range(1, i - w.W + 1) if j in members]
        X = [j for j in range(1, i - w.W + 1) if j not in members]
        tau = diag[b, h, r, 0]
        assert min(s[T]) == tau
        if X:
            assert max(s[X]) <= tau


def test_scores_match_library_matmul():
    """Step 1 against torch's float64 matmul: scale 1/sqrt(d), GQA head map, query position."""
    w, x = make(B=2, Hq=6, Hkv=2, n=90, nq=5, d=32, W=4, topk=3, dtype="bf16", seed=3)
    ref = scores64(w, x)
    for b, h, r in itertools.product(range(w.batch), range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        s = oracle.scores(x["q"], x["k"], b, h, r)
        assert len(s) == i + 1
        np.testing.assert_allclose(s, ref[b, h, r, : i + 1].numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_tie_band_width_is_largest_absolute_score(case):
    """The half-width of the tie band around the k-th selected score (the Top-k of section
    2.2.3; tau_min of the section 3.2.1 lemma) is 1e-5 * max_{j <= i} |s_ij|. The oracle's
    diag[1] must be that maximum, taken over the causal positions only, against torch's
    float64 matmul: a signed or halved maximum would widen or narrow what parity accepts."""
    w, x = make(**case)
    _, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    S = scores64(w, x)
    from_negative = 0
    for b, h, r in itertools.product(range(w.batch), range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        s = S[b, h, r, : i + 1]
        want = s.abs().max().item()
        assert abs(diag[b, h, r, 1] - want) <= 1e-12, (b, h, r, diag[b, h, r, 1], want)
        from_negative += int(-s.min().item() > s.max().item())
    # The inputs exercise the absolute value: in some row the largest |s| is a negative score.
    assert from_negative > 0


def _beats(sa, a, sb, b):
    return sa > sb or (sa == sb and a < b)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    """n <= 12 with small-integer inputs (many exact ties): the oracle's top-k part is the one
    k'-subset of R whose every member beats every non-member (higher score, then lower index)."""
    g = torch.Generator().manual_seed(seed)
    n = 6 + seed % 7
    d = 4
    W = 1 + seed % 3
    topk = 1 + seed % 4
    nq = n
    q = torch.randint(-1, 2, (1, 1, nq, d), generator=g).float()
    k = torch.randint(-1, 2, (1, 1, n, d), generator=g).float()
    v = torch.randn((1, 1, n, d), generator=g)
    idx, _, _ = oracle.condensate(q, k, v, W, topk)
    s_all = (q[0, 0].double() @ k[0, 0].double().T) / 2.0   # 1/sqrt(4) is exact
    for r in range(nq):
        i = r
        R = list(range(1, i - W + 1))
        kp = min(topk, len(R))
        s = s_all[r]
        winners = []
        for S in itertools.combinations(R, kp):
            rest = [b for b in R if b not in S]
            if all(_beats(s[a].item(), a, s[b].item(), b) for a in S for b in rest):
                winners.append(set(S))
        assert len(winners) == 1
        members = set(idx[0, 0, r][idx[0, 0, r] >= 0].tolist())
        assert {j for j in members if 1 <= j <= i - W} == winners[0]


@pytest.mark.parametrize("seed", range(4))
def test_topk_matches_torch_topk_outside_ties(seed):
    w, x = make(Hq=4, Hkv=2, n=2000, nq=3, d=32, W=50, topk=40, seed=seed, needles=5)
    idx, _, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    S = scores64(w, x)
    for h, r in itertools.product(range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        cand = S[0, h, r, 1 : i - w.W + 1]
        vals, pos = torch.topk(cand, w.topk + 1)
        assert vals[w.topk - 1] > vals[w.topk], "no tie at the boundary for these seeds"
        want = set((pos[: w.topk] + 1).tolist())
        members = set(idx[0, h, r][idx[0, h, r] >= 0].tolist())
        assert {j for j in members if 1 <= j <= i - w.W} == want


@pytest.mark.parametrize("case", CASES)
def test_restricted_softmax_matches_sdpa(case):
    """Step 5 (softmax restricted to C_i, times V; Theorem 1's Attention_C, section 2.3)
    equals torch's float64 attention with a membership mask."""
    w, x = make(**case)
    idx, out, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    ref = sdpa64(w, x, member_mask(w, idx))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    again = oracle.restricted(x["q"], x["k"], x["v"], idx)
    assert np.array_equal(again, out)


def causal_mask(w):
    pos = torch.tensor(positions(w))
    return torch.arange(w.n)[None, :] <= pos[:, None]


@pytest.mark.parametrize("case", [dict(Hq=2, Hkv=1, n=40, nq=40, d=16, W=20, topk=19),
                                  dict(Hq=4, Hkv=2, n=60, nq=9, d=8, W=59, topk=0, dtype="bf16"),
                                  dict(Hq=1, Hkv=1, n=33, nq=1, d=8, W=8, topk=24)])
def test_full_attention_special_case(case):
    """When 1+W+k >= i+1 the set is all of {0..i}: the method is plain causal attention
    (section 1.1 equation), bit for bit the oracle's own full attention, and equal to torch's."""
    w, x = make(**case)
    assert 1 + w.W + w.topk >= w.n
    idx, out, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    full = oracle.full(x["q"], x["k"], x["v"])
    assert np.array_equal(out, full)
    assert np.all(diag[..., 2] == 0.0)
    ref = sdpa64(w, x, causal_mask(w).expand(w.batch, w.heads, w.nq, w.n))
    np.testing.assert_allclose(full, ref, rtol=0, atol=1e-12)


def test_full_attention_rows_inside_prefill():
    """Rows with i+1 <= 1+W+k of a longer prefill are also plain causal attention."""
    w, x = make(Hq=1, Hkv=1, n=300, nq=300, d=16, W=24, topk=10, seed=5)
    idx, out, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    full = oracle.full(x["q"], x["k"], x["v"])
    cut = 1 + w.W + w.topk
    assert np.array_equal(out[:, :, :cut], full[:, :, :cut])
    assert not np.array_equal(out[:, :, cut:], full[:, :, cut:])


def test_static_anchor_window_special_case():
    """k = 0 is the "Static (Anchor+Window)" baseline of section 4.3: attention sink plus a
    sliding window, checked against torch's attention with that mask."""
    w, x = make(Hq=4, Hkv=2, n=180, nq=30, d=16, W=12, topk=0, seed=7)
    _, out, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, 0)
    pos = torch.tensor(positions(w))
    j = torch.arange(w.n)[None, :]
    mask = (j == 0) | ((j <= pos[:, None]) & (j >= pos[:, None] - w.W + 1))
    ref = sdpa64(w, x, mask.expand(w.batch, w.heads, w.nq, w.n))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_excluded_mass_identity_and_theorem4_bound(seed):
    """Full attention splits exactly into the restricted output and the excluded rows' output,
    weighted by the excluded mass eps (section 3.2.2): A = (1-eps) Abar + eps Abar_excl.
    Hence |Abar - A|_2 <= 2 eps max_j |v_j|_2, the checkable form of Theorem 4 (section 3.2.4)."""
    w, x = make(Hq=2, Hkv=1, n=400, nq=20, d=16, W=32, topk=16, seed=seed, needles=4)
    idx, out, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    full = oracle.full(x["q"], x["k"], x["v"])
    comp = np.full((w.batch, w.heads, w.nq, w.n), -1, dtype=np.int32)
    for b, h, r in itertools.product(range(w.batch), range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        members = set(idx[b, h, r][idx[b, h, r] >= 0].tolist())
        rest = [j for j in range(i + 1) if j not in members]
        comp[b, h, r, : len(rest)] = rest
    excl = oracle.restricted(x["q"], x["k"], x["v"], comp)
    eps = diag[..., 2:3]
    assert np.all(eps > 0)
    np.testing.assert_allclose((1 - eps) * out + eps * excl, full, rtol=0, atol=1e-13)
    vmax = x["v"].double().norm(dim=-1).max().item()
    gap = np.linalg.norm(out - full, axis=-1)
    assert np.all(gap <= 2 * eps[..., 0] * vmax)


def test_bf16_is_widened_exactly():
    """A bf16 problem and the same values stored as float32 give identical results."""
    w, x = make(Hq=4, Hkv=2, n=250, nq=6, d=32, W=20, topk=10, dtype="bf16", seed=11)
    a = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    b = oracle.condensate(x["q"].float(), x["k"].float(), x["v"].float(), w.W, w.topk)
    for u, v in zip(a, b):
        assert np.array_equal(u, v, equal_nan=True)


def test_planted_needles_closed_form():
    """A planted key equals 4 q/|q| for its query, so its score is 4 |q| / sqrt(d) (scale of
    section 1.1); it is in the set exactly when it ranks within the top-k (section 2.2.3)."""
    w = synth.WORKLOADS["prefill_1k_f32"]
    x = synth.make_inputs(w)
    idx, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    assert int(diag[..., 3].sum()) == 79704   # sum over rows of min(i+1, 81)
    for (j, h, r) in x["needles"][(0, 0)]:
        s = oracle.scores(x["q"], x["k"], 0, h, r)
        qn = x["q"][0, h, r].double().norm().item()
        assert abs(s[j] - 4.0 * qn / math.sqrt(w.d)) < 1e-5
        cand = s[1 : w.n - w.nq + r - w.W + 1]
        rank = int(np.sum(cand > s[j]))
        assert (j in set(idx[0, h, r].tolist())) == (rank < w.topk)


def test_restricted_rejects_bad_sets():
    w, x = make(n=20, nq=2, d=8, W=4, topk=2)
    bad = np.full((1, 2, 2, 4), -1, dtype=np.int32)
    bad[..., 0] = 0
    bad[0, 0, 0, 1] = 0          # repeated position
    with pytest.raises(RuntimeError):
        oracle.restricted(x["q"], x["k"], x["v"], bad)
    bad2 = np.full((1, 2, 2, 4), -1, dtype=np.int32)
    bad2[..., 0] = 0
    bad2[0, 1, 0, 1] = 19        # beyond the query's position (18)
    with pytest.raises(RuntimeError):
        oracle.restricted(x["q"], x["k"], x["v"], bad2)


def test_threads_do_not_change_results():
    w, x = make(Hq=4, Hkv=4, n=500, nq=16, d=16, W=16, topk=8, seed=2)
    a = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk, threads=1)
    b = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk, threads=4)
    for u, v in zip(a, b):
        assert np.array_equal(u, v, equal_nan=True)


@pytest.mark.parametrize("case", [
    dict(n=300, nq=5, W=32, topk=16),       # all three parts present
    dict(n=40, nq=40, W=8, topk=4),         # prefill: early rows with window over 0, |R| < k
    dict(n=300, nq=2, W=16, topk=0),        # k = 0: no top-k mass
    dict(n=50, nq=3, W=64, topk=8),         # the window covers every position
])
def test_mass_parts_partition_one(case):
    """The full-softmax masses of the anchor, of the window without position 0, of the top-k
    positions and outside C (eps) are those of disjoint sets covering 0..i: they sum to 1. With
    k = 0 or an empty R the top-k mass is 0; with C = {0..i} eps is 0 as well."""
    w, x = make(Hq=2, Hkv=1, d=16, **case)
    _, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    eps, anchor, window, topk = diag[..., 2], diag[..., 5], diag[..., 6], diag[..., 7]
    assert np.allclose(eps + anchor + window + topk, 1.0, rtol=0, atol=1e-12)
    assert np.all(anchor > 0) and np.all(window >= 0) and np.all(topk >= 0)
    kp = diag[..., 4]
    assert np.all(topk[kp == 0] == 0.0)
    full = diag[..., 3] == (w.n - w.nq + np.arange(w.nq) + 1)[None, None, :]
    assert np.all(eps[full] == 0.0)


def test_mass_parts_hand_computed():
    """Scores built so that exp(s_j) = 1, 2, 8, 4, 1, 2 at positions 0..5 (q = e_0, k_j =
    sqrt(d) ln(e^{s_j}) e_0). For the query at 5 with W = 2, k = 1: window {4, 5}, R = {1, 2, 3},
    top-1 = position 2; Z = 18, so anchor 1/18, window 3/18, top-k 8/18, eps (positions 1, 3)
    6/18."""
    d, n = 64, 6
    ez = [1.0, 2.0, 8.0, 4.0, 1.0, 2.0]
    q = torch.zeros(1, 1, 1, d, dtype=torch.float64)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, n, d, dtype=torch.float64)
    for j, e in enumerate(ez):
        k[0, 0, j, 0] = math.sqrt(d) * math.log(e)
    v = torch.zeros(1, 1, n, d, dtype=torch.float64)
    idx, _, diag = oracle.condensate(q.float(), k.float(), v.float(), 2, 1)
    assert sorted(j for j in idx[0, 0, 0].tolist() if j >= 0) == [0, 2, 4, 5]
    got = diag[0, 0, 0]
    expect = {2: 6 / 18, 5: 1 / 18, 6: 3 / 18, 7: 8 / 18}
    for col, val in expect.items():
        assert abs(got[col] - val) < 1e-6, (col, got[col], val)


def test_row_subsets_equal_the_whole_call():
    """The row-subset entry points (used for sampled parity at full sizes) return, for each
    listed (b, h, r) and in the listed order, exactly the whole call's results for that query."""
    w, x = make(B=2, Hq=4, Hkv=2, n=260, nq=30, d=32, W=20, topk=12, dtype="bf16", seed=4)
    idx, out, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    full = oracle.full(x["q"], x["k"], x["v"])
    rows = [(1, 3, 29), (0, 0, 0), (0, 2, 17), (1, 0, 5), (0, 2, 17)]
    i2, o2, d2 = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk, rows=rows)
    f2 = oracle.full(x["q"], x["k"], x["v"], rows=rows)
    r2 = oracle.restricted(x["q"], x["k"], x["v"], np.stack([idx[t] for t in rows]), rows=rows)
    for t, key in enumerate(rows):
        assert np.array_equal(i2[t], idx[key])
        assert np.array_equal(o2[t], out[key]) and np.array_equal(r2[t], out[key])
        assert np.array_equal(d2[t], diag[key], equal_nan=True)
        assert np.array_equal(f2[t], full[key])
    with pytest.raises(ValueError):
        oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk, rows=[(0, 4, 0)])
