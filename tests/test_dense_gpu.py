"""The dense causal-attention baseline (ca_dense_attention_ex) against the oracle's full
attention (softmax over every j <= i, times V; section 1.1 of the metaphor-xennon page on "The
Condensate Theorem"), which the oracle pins match to library attention (test_oracle_pins.py).
bf16 inputs, fp32 accumulation; tolerance that of bf16 outputs."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_transformer_attention_amd as ca
from sparse_transformer_attention_amd import synth

from parity import assert_outputs

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
    assert_outputs(out.cpu().numpy(), ref, torch.bfloat16)


def test_dense_full_size_prefill_131k_sampled():
    w = synth.WORKLOADS["prefill_131k_h8_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("dense full-size prefill 131k")
    out = ca.dense_attention(x["q"], x["k"], x["v"]).cpu().numpy()
    g = torch.Generator().manual_seed(3)
    rows = [(0, 0, 0), (0, 7, w.nq - 1)] + [
        (0, int(torch.randint(w.heads, (1,), generator=g)), int(torch.randint(w.nq, (1,), generator=g)))
        for _ in range(6)]
    for (b, h, r) in rows:
        i = w.n - w.nq + r
        q1 = x["q"][b, h, r].reshape(1, 1, 1, w.d).cpu()
        k1 = x["k"][b, h, : i + 1].reshape(1, 1, i + 1, w.d).cpu()
        v1 = x["v"][b, h, : i + 1].reshape(1, 1, i + 1, w.d).cpu()
        ref = oracle.full(q1, k1, v1)
        assert_outputs(out[b, h, r].reshape(1, 1, 1, -1), ref, torch.bfloat16)
