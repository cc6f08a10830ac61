"""ca_condensate_attention_noscratch (the entry point that allocates nothing: its workspace is the
library's per-GPU device array) against ca_condensate_attention_ex with a caller workspace, through
the C ABI, on consecutive calls whose problems shrink: the 131K GQA decode step, then smaller
problems on the other paths (matrix-core prefill, chunked select). Same kernels, same order:
the sets and the output bits must be equal."""
import sys

import pytest
import torch

import sparse_transformer_attention_amd as ca
from sparse_transformer_attention_amd import synth

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def W_(**kw):
    base = dict(name="t", batch=1, heads=4, kv_heads=1, d=128, n=4000, nq=1, dtype="bf16", W=64,
                topk=32, q_scale=2.0, needles_per_kv_head=8)
    base.update(kw)
    return synth.Workload(**base)


CASES = [
    ("prefill_mfma", W_(heads=4, kv_heads=2, d=64, n=3000, nq=3000, W=48, topk=32, q_scale=1.0), 0),
    ("decode_131k_gqa_bf16", synth.WORKLOADS["decode_131k_gqa_bf16"], 0),
    ("decode_f32_chunked", W_(dtype="f32", heads=8, kv_heads=2, n=9000, nq=2, W=100, topk=40), 256),
]


def test_noscratch_matches_ex_on_shrinking_calls():
    sizes = []
    for name, w, chunk in CASES:
        x = synth.make_inputs(w, seed=7, device="cuda")
        q, k, v = x["q"], x["k"], x["v"]
        p = ca.params_for(q, k, w.W, w.topk, chunk=chunk)
        need = ca.workspace_size(p)
        sizes.append(need)
        announce(f"noscratch {name} (workspace {need} bytes)")
        out_a = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device="cuda")
        idx_a = torch.empty((w.batch, w.heads, w.nq, w.set_cap), dtype=torch.int32, device="cuda")
        out_b, idx_b = torch.empty_like(out_a), torch.empty_like(idx_a)
        ws = ca.alloc_workspace(p)
        ca.condensate_attention_ex(p, q, k, v, out_a, idx_a, ws)
        for _ in range(2):  # twice: the second call finds the first one's contents
            out_b.fill_(float("nan"))
            idx_b.fill_(-7)
            ca.condensate_attention_noscratch(p, q, k, v, out_b, idx_b)
            torch.cuda.synchronize()
            assert torch.equal(idx_a, idx_b), name
            assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32)), name
    assert sizes[0] > sizes[1] > sizes[2] > 0
