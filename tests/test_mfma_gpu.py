"""Parity of the MFMA prefill path (bf16, many query vectors per KV head) with the CPU oracle.

The library takes this path by itself for bf16 problems with at least 64 query vectors per KV
head and topk <= 128; every test checks through the library's profiler that its two kernels
(mfma_bound, mfma_cand) ran. The shapes cover the three bound-pass tilings: 2 of every 4 key
tiles (topk <= 32), 3 of 4 (topk <= 64) and all of them (topk > 64). Index sets must match the oracle's outside the tie band (exactly,
with integer inputs), outputs the oracle's restricted softmax on the GPU's own set.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_transformer_attention_amd as ca
from sparse_transformer_attention_amd import synth

from parity import assert_outputs, compare_sets

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def W_(**kw):
    base = dict(name="t", batch=1, heads=2, kv_heads=2, d=128, n=2000, nq=600, dtype="bf16", W=64,
                topk=64, q_scale=2.0, needles_per_kv_head=8)
    base.update(kw)
    return synth.Workload(**base)


SHAPES = {
    # 600 vectors per KV head: two full workgroups of 256 and a ragged third.
    "mha_d128_ragged": W_(),
    # GQA (4 query heads per KV head) at d = 64, the largest topk of the path.
    "gqa4_d64_topk128": W_(d=64, heads=8, kv_heads=2, n=1500, nq=40, W=32, topk=128),
    # Every position a query: the first rows have no candidates, later ones fewer than topk.
    "full_causal_d64": W_(d=64, heads=2, kv_heads=1, n=700, nq=700, W=16, topk=8),
    "batch2_topk1": W_(batch=2, heads=4, kv_heads=2, n=1200, nq=100, W=100, topk=1),
    "topk_exceeds_R": W_(heads=1, kv_heads=1, n=400, nq=400, W=64, topk=100),
    # 4096 query vectors or more: the merge and attend stage runs one workgroup of 64 threads
    # (topk <= 32) or 128 threads per vector instead of 1024.
    "many_vectors_wave64": W_(d=64, heads=8, kv_heads=2, n=1024, nq=560, W=64, topk=16),
    "many_vectors_wave128": W_(heads=8, kv_heads=8, n=1024, nq=520, W=64, topk=64),
    # 8 query heads per KV head, batch 2: the vectors of a KV head interleave heads and rows.
    "gqa8_b2_d128": W_(batch=2, heads=16, kv_heads=2, n=1800, nq=90, W=40, topk=24),
    # The windows of the pages' per-layer schedule (sections 6.1-6.2): W = 1024 (1,025-row
    # anchor-and-window sets in mfma_window and finish), 256 and 64.
    "window_1024_mha": W_(heads=2, kv_heads=2, n=3000, nq=800, W=1024, topk=64),
    "window_1024_gqa4_d64": W_(d=64, heads=8, kv_heads=2, n=2600, nq=300, W=1024, topk=32),
    "window_256_gqa2": W_(heads=4, kv_heads=2, n=2000, nq=500, W=256, topk=64),
    "window_64_gqa4_d64": W_(d=64, heads=8, kv_heads=2, n=2400, nq=400, W=64, topk=32),
}


def run_mfma(w, x):
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    ca.profile_start(8)
    out, idx = ca.condensate(q, k, v, w.W, w.topk)
    torch.cuda.synchronize()
    prof = ca.profile_stop()
    assert "mfma_bound" in prof and "mfma_cand" in prof, f"MFMA path not taken: {sorted(prof)}"
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("name", list(SHAPES))
def test_mfma_path_matches_oracle(name):
    w = SHAPES[name]
    x = synth.make_inputs(w, seed=21)
    announce(f"mfma {name}")
    out, idx = run_mfma(w, x)
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


def integer_inputs(w, seed, levels=2):
    """Small-integer q/k: every product and sum is exact in fp32, so scores tie exactly."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-levels, levels + 1, (w.batch, w.heads, w.nq, w.d), generator=g).float()
    k = torch.randint(-levels, levels + 1, (w.batch, w.kv_heads, w.n, w.d), generator=g).float()
    v = torch.randn((w.batch, w.kv_heads, w.n, w.d), generator=g)
    return {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16)}


@pytest.mark.parametrize("shape", [
    dict(d=64, heads=2, kv_heads=2, n=3000, nq=128, W=30, topk=20),
    dict(d=128, heads=4, kv_heads=1, n=2500, nq=70, W=10, topk=128),
    # Over 1024 rows per kept key: the candidate pass with its block pre-test (and here the
    # pre-test lets every block of a tied bound through to the exact compare).
    dict(d=128, heads=2, kv_heads=2, n=3000, nq=64, W=30, topk=2),
    # 32 < k <= 64: the bound pass reads 3 of every 4 tiles (k <= 32 above: 2 of 4; k = 128:
    # every tile), and many more rows than k tie at that looser bound.
    dict(d=128, heads=4, kv_heads=2, n=2800, nq=96, W=40, topk=48),
])
def test_mfma_exact_ties_follow_the_tie_break(shape):
    """Many keys tie at the bound, so candidate lists fill and are cut to their exact top-k'
    while the rows stream; equal scores must still go to the smaller position."""
    w = W_(**shape)
    x = integer_inputs(w, seed=3)
    announce(f"mfma ties {shape}")
    out, idx = run_mfma(w, x)
    ref_idx, _, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    assert np.array_equal(idx, ref_idx)
    assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


@pytest.mark.parametrize("length,topk", [(60, 48), (1500, 128)])
def test_mfma_clustered_best_rows(length, topk):
    """A run of key rows aligned with the queries: far more rows than k reach the bound."""
    w = W_(heads=2, kv_heads=1, n=4000, nq=64, W=64, topk=topk)
    x = synth.make_inputs(w, seed=13)
    q = x["q"].float()
    k = x["k"].float().clone()
    d = q.sum(dim=(1, 2))
    d = d / d.norm(dim=-1, keepdim=True) * 24.0
    j = torch.arange(length, dtype=torch.float32)
    gains = 1.0 + 0.5 * ((j * 7919.0) % length if length > 256 else j) / length
    k[:, 0, 1001:1001 + length] = d[:, None, :] * gains[None, :, None]
    x["k"] = k.to(torch.bfloat16)
    announce(f"mfma clustered {length} {topk}")
    out, idx = run_mfma(w, x)
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


def test_mfma_matches_chunked_path():
    """The chunked VALU path (chunk = 256) on the same inputs: both sets are the oracle's
    outside the band."""
    w = SHAPES["mha_d128_ragged"]
    x = synth.make_inputs(w, seed=8)
    announce("mfma vs chunked")
    out, idx = run_mfma(w, x)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    out2, idx2 = ca.condensate(q, k, v, w.W, w.topk, chunk=256)
    torch.cuda.synchronize()
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    compare_sets(idx2.cpu().numpy(), ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)


def test_mfma_deterministic():
    w = SHAPES["gqa4_d64_topk128"]
    x = synth.make_inputs(w, seed=2)
    announce("mfma determinism")
    a = run_mfma(w, x)
    b = run_mfma(w, x)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
