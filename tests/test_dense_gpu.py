"""The dense causal-attention baseline (ca_dense_attention_ex) against the oracle's full
attention (softmax over every j <= i, times V; section 1.1 of the metaphor-xennon page on "The
Condensate Theorem"), which the oracle pins match to library attention (test_oracle_pins.py).
bf16 inputs, fp32 accumulation; tolerance that of bf16 outputs. The dense kernel multiplies V by
the softmax weights rounded to bf16 (a relative error of up to 2^-9 per weight), so its
achieved-error ceiling is that of bf16 weights, not of the method's fp32 ones."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_transformer_attention_amd as ca
from sparse_transformer_attention_amd import synth

from parity import assert_outputs

# bf16 weights: errors of a few 2^-9 in a convex combination of V rows.
DENSE_CEILING = 1e-2

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def W_(**kw):
    base = dict(name="t", batch=1, heads=2, kv_heads=2, d=128, n=1500, nq=300, dtype="bf16", W=64,
                topk=16, q_scale=1.0, needles_per_kv_head=4)
    base.update(kw)
    return synth.Workload(**base)


CASES = {
    "prefill_mha_d128_ragged": W_(),
    "prefill_gqa4_d64": W_(d=64, heads=8, kv_heads=2, n=900, nq=900),
    "decode_gqa_b2": W_(batch=2, heads=8, kv_heads=2, n=3000, nq=1),
    # 8 query heads per KV head at d = 128, batch 2: several workgroups per KV head, the last
    # one ragged (dispatched first: it has the most rows).
    "prefill_gqa8_d128_b2": W_(batch=2, heads=16, kv_heads=2, n=1300, nq=170),
}


@pytest.mark.parametrize("name", list(CASES))
def test_dense_matches_oracle_full_attention(name):
    w = CASES[name]
    x = synth.make_inputs(w, seed=5)
    announce(f"dense {name}")
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    out = ca.dense_attention(q, k, v)
    torch.cuda.synchronize()
    ref = oracle.full(x["q"], x["k"], x["v"])
    err = assert_outputs(out.cpu().numpy(), ref, torch.bfloat16, ceiling=DENSE_CEILING)
    announce(f"dense {name}: max relative error {err:.3g}")


def test_dense_full_size_prefill_131k_stratified():
    """The full 131K prefill (8 heads, d = 64): the first and last rows, the row at every
    256-vector boundary for every head, and 512 random rows, against the oracle's full
    attention on those rows."""
    w = synth.WORKLOADS["prefill_131k_h8_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("dense full-size prefill 131k")
    out = ca.dense_attention(x["q"], x["k"], x["v"])
    rows = set()
    for h in range(w.heads):
        rows.update({(0, h, 0), (0, h, w.nq - 1)})
        rows.update((0, h, m) for m in range(256, w.nq, 256))
    g = np.random.default_rng(3)
    rows.update((0, int(h), int(r)) for h, r in zip(g.integers(0, w.heads, 512), g.integers(0, w.nq, 512)))
    rows = sorted(rows)
    a = torch.tensor(rows, dtype=torch.int64, device="cuda")
    g_out = out[a[:, 0], a[:, 1], a[:, 2]].cpu().numpy()
    xh = {t: x[t].cpu() for t in ("q", "k", "v")}
    del x, out
    ref = oracle.full(xh["q"], xh["k"], xh["v"], rows=rows)
    err = assert_outputs(g_out, ref, torch.bfloat16, ceiling=DENSE_CEILING)
    announce(f"dense 131k: {len(rows)} rows, max relative error {err:.3g}")
