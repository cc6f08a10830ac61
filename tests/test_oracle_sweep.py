"""Property sweep of the oracle's pins over random shapes (Hypothesis): batch, heads and GQA
group, n, the query rows, d, W, k, dtype, planted needles and the seed.

Every drawn problem is checked against facts that do not come from the oracle (page sections
are those of the metaphor-xennon blog page on "The Condensate Theorem"):
- the set structure of Definition 1 (section 2.1) and the size bound of Corollary 2 (section 2.4);
- the scores of step 1 against torch's float64 matmul, then on them the exclusion lemma of
  section 3.2.1 and the top-k rule of section 2.2.3 (ties to the smaller position);
- the restricted softmax of section 2.3 against torch's float64 attention with a membership mask;
- the tie-band width max_{j <= i} |s_ij| and the mass partition (section 3.2.2) summing to one.
The examples are derandomized, so a failure reproduces from the printed case.
"""
import itertools

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from test_oracle_pins import make, member_mask, scores64, sdpa64


@st.composite
def problems(draw):
    Hkv = draw(st.sampled_from([1, 2]))
    g = draw(st.sampled_from([1, 2, 4]))
    n = draw(st.integers(min_value=1, max_value=160))
    nq = draw(st.integers(min_value=1, max_value=min(n, 12)))
    return dict(B=draw(st.sampled_from([1, 2])), Hq=Hkv * g, Hkv=Hkv, n=n, nq=nq,
                d=draw(st.sampled_from([4, 8, 16, 32, 64])),
                W=draw(st.integers(min_value=1, max_value=70)),
                topk=draw(st.integers(min_value=0, max_value=40)),
                dtype=draw(st.sampled_from(["f32", "bf16"])),
                needles=draw(st.sampled_from([0, 2])),
                seed=draw(st.integers(min_value=0, max_value=2**31 - 1)))


SWEEP = settings(max_examples=150, deadline=None, derandomize=True,
                 suppress_health_check=[HealthCheck.too_slow])


@SWEEP
@given(problems())
def test_sweep_pins(case):
    w, x = make(**case)
    idx, out, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    S = scores64(w, x)
    cap = 1 + w.W + w.topk
    for b, h, r in itertools.product(range(w.batch), range(w.heads), range(w.nq)):
        i = w.n - w.nq + r
        row = idx[b, h, r]
        members = row[row >= 0]
        # Definition 1 and Corollary 2: {0}, the whole window, k' = min(k, |R_i|) of R_i.
        assert np.all(row[len(members):] == -1)
        assert np.all(np.diff(members) > 0)
        assert len(members) == min(i + 1, cap) == diag[b, h, r, 3]
        assert members[0] == 0 and members[-1] == i
        assert set(range(max(0, i - w.W + 1), i + 1)) <= set(members.tolist())
        n_r = max(0, i - w.W)
        top = [j for j in members.tolist() if 1 <= j <= i - w.W]
        assert len(top) == min(w.topk, n_r) == diag[b, h, r, 4]
        # Step 1 against torch's float64 matmul, and the tie-band width from it.
        s_ref = S[b, h, r, : i + 1].numpy()
        M = np.abs(s_ref).max()
        s = oracle.scores(x["q"], x["k"], b, h, r)
        np.testing.assert_allclose(s, s_ref, rtol=0, atol=1e-12 * max(1.0, M))
        assert abs(diag[b, h, r, 1] - M) <= 1e-12 * max(1.0, M)
        # Sections 3.2.1 / 2.2.3 on those scores: no excluded candidate beats a selected one,
        # and at an exact tie the smaller position is the selected one.
        excl = sorted(set(range(1, n_r + 1)) - set(top))
        if top and excl:
            t_min, x_max = min(s[top]), max(s[excl])
            assert x_max <= t_min
            if x_max == t_min:
                assert max(j for j in top if s[j] == t_min) < min(j for j in excl if s[j] == x_max)
    # Section 2.3: the softmax restricted to C_i times V.
    ref = sdpa64(w, x, member_mask(w, idx))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # Section 3.2.2: eps and the anchor / window / top-k masses partition the full softmax.
    eps, anchor, window, topk = diag[..., 2], diag[..., 5], diag[..., 6], diag[..., 7]
    assert np.allclose(eps + anchor + window + topk, 1.0, rtol=0, atol=1e-12)
    assert np.all(eps >= -1e-15) and np.all(anchor > 0) and np.all(window >= 0) and np.all(topk >= 0)
