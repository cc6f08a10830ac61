"""The mass diagnostic (ca_condensate_attention_mass_ex) against the oracle: the full causal
softmax weight outside C_i (section 3.2.2 of the metaphor-xennon page on "The Condensate
Theorem") and of the anchor, the window without position 0 and the top-k positions (sections
2.2.1-2.2.3). The oracle's float64 values are pinned by the partition identity, special cases
and a hand-computed example (test_oracle_pins.py). The set and output must be those of the
plain call, bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_transformer_attention_amd as ca
from sparse_transformer_attention_amd import synth

pytestmark = pytest.mark.gpu

# fp32 sums over up to n terms against float64: relative 1e-3 with an absolute floor.
RTOL, ATOL = 1e-3, 1e-5
MASS_COLS = [2, 5, 6, 7]   # oracle diag columns: eps, anchor, window, top-k


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def W_(**kw):
    base = dict(name="t", batch=1, heads=4, kv_heads=1, d=128, n=4000, nq=1, dtype="bf16", W=64,
                topk=32, q_scale=2.0, needles_per_kv_head=8)
    base.update(kw)
    return synth.Workload(**base)


CASES = {
    "gqa4_b2_bf16": W_(batch=2, heads=8, kv_heads=2, n=5000, W=64, topk=32),
    "f32_d128_multi_query": W_(dtype="f32", heads=4, kv_heads=1, n=2500, nq=3, W=33, topk=17),
    "bf16_d64_gqa8": W_(d=64, heads=16, kv_heads=2, n=2100, nq=5, W=50, topk=100),
    "f32_W1_prefill": W_(dtype="f32", d=64, heads=1, kv_heads=1, n=700, nq=700, W=1, topk=5),
}


def run_both(w, x):
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    out, idx, mass = ca.condensate_mass(q, k, v, w.W, w.topk)
    out2, idx2 = ca.condensate(q, k, v, w.W, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))
    return out.cpu().numpy(), idx.cpu().numpy(), mass.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_mass_matches_oracle(name):
    w = CASES[name]
    x = synth.make_inputs(w, seed=11)
    announce(f"mass {name}")
    _, _, mass = run_both(w, x)
    _, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    ref = diag[..., MASS_COLS]
    assert np.allclose(mass, ref, rtol=RTOL, atol=ATOL), np.abs(mass - ref).max()
    assert np.allclose(mass.sum(axis=-1), 1.0, atol=1e-5)


def test_mass_full_size_decode_131k():
    w = synth.WORKLOADS["decode_131k_gqa_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("mass full-size decode 131k")
    _, _, mass = run_both(w, x)
    for h in range(w.heads):
        kvh = h // w.group
        q1 = x["q"][0, h, 0].reshape(1, 1, 1, w.d).cpu()
        k1 = x["k"][0, kvh].reshape(1, 1, w.n, w.d).cpu()
        v1 = x["v"][0, kvh].reshape(1, 1, w.n, w.d).cpu()
        _, _, diag = oracle.condensate(q1, k1, v1, w.W, w.topk)
        ref = diag[0, 0, 0, MASS_COLS]
        assert np.allclose(mass[0, h, 0], ref, rtol=RTOL, atol=ATOL), (h, mass[0, h, 0], ref)
