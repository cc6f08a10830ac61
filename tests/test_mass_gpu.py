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
    # W >= 512: the window part comes from the chunk partials of extra stream workgroups.
    "long_window_bf16": W_(heads=8, kv_heads=2, n=5000, W=600, topk=32),
    "long_window_f32_d64": W_(dtype="f32", d=64, heads=2, kv_heads=1, n=900, nq=600, W=512, topk=16),
}


# bf16 with at least 64 query vectors per KV head and topk <= 128: the matrix-core prefill
# path, where the bound pass also sums each query's softmax over R_i and finish adds the parts.
MFMA_CASES = {
    "mfma_mha_d128_ragged": W_(heads=2, kv_heads=2, n=2000, nq=600, W=64, topk=64),
    # Every position a query: the first rows have no candidates (R_i empty) and share
    # wavefronts with rows that have them.
    "mfma_full_causal_d64": W_(d=64, heads=2, kv_heads=1, n=700, nq=700, W=16, topk=8),
    "mfma_gqa4_d64_w1024": W_(d=64, heads=8, kv_heads=2, n=2600, nq=300, W=1024, topk=32),
    "mfma_gqa8_b2_d128": W_(batch=2, heads=16, kv_heads=2, n=1800, nq=90, W=40, topk=24),
}


# The chunked path (chunk = 256 / 512): one sum per workgroup of a unit, merged in finish. The
# decode-shaped cases spread a unit's chunks over many workgroups.
CHUNKED_CASES = {
    "chunked_decode_gqa4_bf16": (W_(n=6000, heads=8, kv_heads=2, W=64, topk=32), 256),
    "chunked_decode_f32_multi": (W_(dtype="f32", n=3000, nq=3, W=33, topk=17), 512),
    "chunked_prefill_bf16_d64": (W_(d=64, heads=2, kv_heads=1, n=900, nq=300, W=40, topk=24), 256),
    "chunked_prefill_f32_early_rows": (W_(dtype="f32", d=64, heads=2, kv_heads=2, n=500, nq=500, W=16, topk=8), 256),
}


def run_both(w, x, path=None, chunk=0):
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    if path:
        ca.profile_start(8)
    out, idx, mass = ca.condensate_mass(q, k, v, w.W, w.topk, chunk=chunk)
    torch.cuda.synchronize()
    if path:
        prof = ca.profile_stop()
        assert path in prof, f"{path} not taken: {sorted(prof)}"
    out2, idx2 = ca.condensate(q, k, v, w.W, w.topk, chunk=chunk)
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


@pytest.mark.parametrize("name", list(MFMA_CASES))
def test_mass_mfma_path_matches_oracle(name):
    w = MFMA_CASES[name]
    x = synth.make_inputs(w, seed=13)
    announce(f"mass {name}")
    _, _, mass = run_both(w, x, path="mfma_bound")
    _, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    ref = diag[..., MASS_COLS]
    assert np.allclose(mass, ref, rtol=RTOL, atol=ATOL), np.abs(mass - ref).max()
    assert np.allclose(mass.sum(axis=-1), 1.0, atol=1e-5)


@pytest.mark.parametrize("name", list(CHUNKED_CASES))
def test_mass_chunked_path_matches_oracle(name):
    w, chunk = CHUNKED_CASES[name]
    x = synth.make_inputs(w, seed=17)
    announce(f"mass {name}")
    _, _, mass = run_both(w, x, path="score_select", chunk=chunk)
    _, _, diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    ref = diag[..., MASS_COLS]
    assert np.allclose(mass, ref, rtol=RTOL, atol=ATOL), np.abs(mass - ref).max()
    assert np.allclose(mass.sum(axis=-1), 1.0, atol=1e-5)


def test_mass_full_size_prefill_chunk_4k_32k_sampled_rows():
    """The 4,096-position chunk at 32K context (the MFMA path at its full size): 24 rows spread
    over heads and positions, each against the oracle row by row."""
    w = synth.WORKLOADS["prefill_chunk_4k_32k_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("mass full-size prefill chunk 4k x 32k")
    _, _, mass = run_both(w, x, path="mfma_bound")
    xh = {t: x[t].cpu() for t in ("q", "k", "v")}
    g = np.random.default_rng(5)
    rows = [(0, int(h), int(r)) for h, r in zip(g.integers(0, w.heads, 24), g.integers(0, w.nq, 24))]
    rows += [(0, 0, 0), (0, w.heads - 1, w.nq - 1)]
    _, _, diag = oracle.condensate(xh["q"], xh["k"], xh["v"], w.W, w.topk, rows=rows)
    ref = diag[:, MASS_COLS]
    got = np.stack([mass[b, h, r] for b, h, r in rows])
    assert np.allclose(got, ref, rtol=RTOL, atol=ATOL), np.abs(got - ref).max()


def test_mass_full_size_decode_131k_all_32_vectors():
    w = synth.WORKLOADS["decode_131k_gqa_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("mass full-size decode 131k")
    _, _, mass = run_both(w, x)
    xh = {t: x[t].cpu() for t in ("q", "k", "v")}
    rows = [(0, h, 0) for h in range(w.heads)]
    _, _, diag = oracle.condensate(xh["q"], xh["k"], xh["v"], w.W, w.topk, rows=rows)
    ref = diag[:, MASS_COLS]
    got = mass[0, :, 0]
    assert np.allclose(got, ref, rtol=RTOL, atol=ATOL), np.abs(got - ref).max()
