"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded synthetic inputs.

Index sets must match outside the tie band; outputs must match the oracle's restricted softmax
on the GPU's own set within 1e-5 (float32) or 2e-2 (bfloat16) relative (see parity.py).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_transformer_attention_amd as ca
from sparse_transformer_attention_amd import synth

from parity import TOL, assert_outputs, compare_sets

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def W_(**kw):
    base = dict(name="t", batch=1, heads=4, kv_heads=1, d=128, n=4000, nq=1, dtype="bf16", W=64,
                topk=32, q_scale=2.0, needles_per_kv_head=8)
    base.update(kw)
    return synth.Workload(**base)


SMALL = {
    "prefill_1k_f32": synth.WORKLOADS["prefill_1k_f32"],
    "decode_8k_mha_f32": synth.WORKLOADS["decode_8k_mha_f32"],
    "gqa4_b2_bf16": W_(batch=2, heads=8, kv_heads=2, n=5000, W=64, topk=32),
    "prefill_bf16_ragged": W_(heads=4, kv_heads=4, n=3000, nq=300, W=100, topk=40, q_scale=1.0),
    "f32_d128_gqa4": W_(dtype="f32", heads=4, kv_heads=1, n=2500, nq=3, W=33, topk=17),
    "bf16_d64_gqa8": W_(d=64, heads=16, kv_heads=2, n=2100, nq=5, W=50, topk=100),
    "topk_exceeds_R": W_(heads=2, kv_heads=2, n=300, nq=10, W=250, topk=100),
    "topk_zero": W_(heads=2, kv_heads=1, n=1000, nq=4, W=20, topk=0),
    "window_covers_all": W_(dtype="f32", d=64, heads=2, kv_heads=2, n=200, nq=200, W=512, topk=8),
    "single_key": W_(dtype="f32", d=64, heads=2, kv_heads=1, n=1, nq=1, W=1, topk=4, needles_per_kv_head=0),
    "W1_prefill": W_(dtype="f32", d=64, heads=1, kv_heads=1, n=700, nq=700, W=1, topk=5),
}


def run_gpu(w, x, chunk=0):
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    out, idx = ca.condensate(q, k, v, w.W, w.topk, chunk=chunk)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end_small(name):
    w = SMALL[name]
    x = synth.make_inputs(w, seed=7)
    announce(f"end_to_end {name}")
    out, idx = run_gpu(w, x)
    ref_idx, ref_out, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    ref_on_gpu_set = oracle.restricted(x["q"], x["k"], x["v"], idx)
    assert_outputs(out, ref_on_gpu_set, w.torch_dtype)


@pytest.mark.parametrize("name", ["prefill_1k_f32", "decode_8k_mha_f32", "gqa4_b2_bf16", "bf16_d64_gqa8",
                                  "f32_d128_gqa4"])
def test_attention_on_subset_with_oracle_sets(name):
    """Stage 2 alone, fed the oracle's own index sets."""
    w = SMALL[name]
    x = synth.make_inputs(w, seed=11)
    ref_idx, ref_out, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    announce(f"subset {name}")
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    p = ca.params_for(q, k, w.W, w.topk)
    out = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device="cuda")
    ca.attention_on_subset(p, q, k, v, torch.from_numpy(ref_idx).cuda(), out)
    torch.cuda.synchronize()
    assert_outputs(out.cpu().numpy(), ref_out, w.torch_dtype)


def test_attention_on_subset_any_order_and_padding():
    """Stage 2 ignores -1 and out-of-range entries and does not depend on entry order
    beyond rounding."""
    w = SMALL["gqa4_b2_bf16"]
    x = synth.make_inputs(w, seed=3)
    ref_idx, ref_out, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    rng = np.random.default_rng(0)
    shuffled = ref_idx.copy()
    for row in shuffled.reshape(-1, shuffled.shape[-1]):
        rng.shuffle(row)
    shuffled[..., -1] = np.where(shuffled[..., -1] < 0, w.n + 5, shuffled[..., -1])
    announce("subset shuffled")
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    p = ca.params_for(q, k, w.W, w.topk)
    out = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device="cuda")
    ca.attention_on_subset(p, q, k, v, torch.from_numpy(shuffled).cuda(), out)
    torch.cuda.synchronize()
    assert_outputs(out.cpu().numpy(), ref_out, w.torch_dtype)
    empty = torch.full_like(torch.from_numpy(ref_idx), -1).cuda()
    ca.attention_on_subset(p, q, k, v, empty, out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("chunk", [256, 512, 1024])
def test_chunk_size_does_not_change_results(chunk):
    w = W_(heads=8, kv_heads=2, n=9000, nq=2, W=64, topk=48)
    x = synth.make_inputs(w, seed=5)
    announce(f"chunk {chunk}")
    out, idx = run_gpu(w, x, chunk=chunk)
    out0, idx0 = run_gpu(w, x, chunk=0)
    assert np.array_equal(idx, idx0)
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


def integer_inputs(w, seed, levels=2):
    """Small-integer q/k so that every fp32 score is exact: many exact ties."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-levels, levels + 1, (w.batch, w.heads, w.nq, w.d), generator=g).float()
    k = torch.randint(-levels, levels + 1, (w.batch, w.kv_heads, w.n, w.d), generator=g).float()
    v = torch.randn((w.batch, w.kv_heads, w.n, w.d), generator=g)
    dt = w.torch_dtype
    return {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt)}


@pytest.mark.parametrize("shape", [
    dict(heads=4, kv_heads=1, n=20000, nq=1, W=64, topk=50),
    dict(heads=2, kv_heads=2, n=3000, nq=64, W=30, topk=20, dtype="f32", d=64),
    dict(heads=8, kv_heads=2, n=6000, nq=3, W=10, topk=300, d=64),
])
@pytest.mark.parametrize("chunk", [0, 256])
def test_exact_ties_follow_the_tie_break(shape, chunk):
    """With exact scores the GPU must reproduce the oracle's sets exactly: equal scores are
    broken toward the smaller position, with no band."""
    w = W_(**shape)
    x = integer_inputs(w, seed=1)
    announce(f"ties {shape} chunk {chunk}")
    out, idx = run_gpu(w, x, chunk=chunk)
    ref_idx, _, _ = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    assert np.array_equal(idx, ref_idx)
    assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


def test_deterministic():
    w = SMALL["gqa4_b2_bf16"]
    x = synth.make_inputs(w, seed=2)
    announce("determinism")
    a = run_gpu(w, x)
    b = run_gpu(w, x)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


def clustered_inputs(w, seed, start, length):
    """Random q/k/v, then K rows [start, start+length) aligned with the sum of each KV head's
    query rows, with distinct gains: the best scores of every query sit in that run, many per
    tile of rows."""
    x = synth.make_inputs(w, seed=seed)
    q = x["q"].float()
    k = x["k"].float().clone()
    g = w.heads // w.kv_heads
    j = torch.arange(length, dtype=torch.float32)
    # Distinct gains; for long runs permuted, so that the best rows spread over many tiles.
    gains = 1.0 + 0.5 * ((j * 7919.0) % length if length > 256 else j) / length
    for kvh in range(w.kv_heads):
        d = q[:, kvh * g:(kvh + 1) * g].sum(dim=(1, 2))  # [B][d]
        d = d / d.norm(dim=-1, keepdim=True) * 24.0
        k[:, kvh, start:start + length] = d[:, None, :] * gains[None, :, None]
    x["k"] = k.to(w.torch_dtype)
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("length,topk", [(60, 48), (1500, 300)])
def test_clustered_best_rows(dtype, length, topk):
    """Best rows packed into consecutive tiles: with a few such tiles the decode path scores
    them again (more than two keys of a tile reach the bound); with many (here > 64 tiles) it
    scores every passing tile into its scratch keys and selects from there. Either way the
    sets must match the oracle's."""
    w = W_(dtype=dtype, heads=4, kv_heads=1, n=8000, nq=2, W=64, topk=topk)
    x = clustered_inputs(w, seed=13, start=3001, length=length)
    announce(f"clustered {dtype} {length} {topk}")
    out, idx = run_gpu(w, x)
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


@pytest.mark.parametrize("name", ["prefill_bf16_ragged", "mfma_wave64", "mfma_wave128"])
def test_select_stage_alone_matches_full_call(name):
    # (The last two: over 4096 bf16 query vectors, the MFMA path with its 64- and 128-thread
    # merge workgroups, here without the attend part.)
    w = {"prefill_bf16_ragged": SMALL["prefill_bf16_ragged"],
         "mfma_wave64": W_(d=64, heads=8, kv_heads=2, n=1024, nq=560, W=64, topk=16),
         "mfma_wave128": W_(heads=8, kv_heads=8, n=1024, nq=520, W=64, topk=64)}[name]
    x = synth.make_inputs(w, seed=4)
    announce(f"select alone {name}")
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    p = ca.params_for(q, k, w.W, w.topk)
    ws = ca.alloc_workspace(p)
    idx = torch.empty((w.batch, w.heads, w.nq, w.set_cap), dtype=torch.int32, device="cuda")
    ca.condensate_select(p, q, k, idx, ws)
    out, idx2 = ca.condensate(q, k, v, w.W, w.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


def test_synchronous_one_call_form():
    """ca_condensate_attention: float32, batch 1, every position a query."""
    w = synth.WORKLOADS["prefill_1k_f32"]
    x = synth.make_inputs(w, seed=9)
    announce("one-call form")
    q, k, v = (x[t][0].contiguous().cuda() for t in ("q", "k", "v"))
    out = torch.empty((w.heads, w.n, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.heads, w.n, w.set_cap), dtype=torch.int32, device="cuda")
    ca.condensate_attention(q, k, v, w.n, w.d, w.heads, w.kv_heads, w.W, w.topk, out, idx)
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(idx.cpu().numpy()[None], ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    assert_outputs(out.cpu().numpy()[None], oracle.restricted(x["q"], x["k"], x["v"], idx.cpu().numpy()[None]),
                   torch.float32)


def test_workspace_too_small_is_rejected():
    w = SMALL["gqa4_b2_bf16"]
    x = synth.make_inputs(w, seed=1)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    p = ca.params_for(q, k, w.W, w.topk)
    need = ca.workspace_size(p)
    ws = torch.empty(need - 8, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.heads, w.nq, w.set_cap), dtype=torch.int32, device="cuda")
    with pytest.raises(ca.CondensateError) as e:
        ca.condensate_attention_ex(p, q, k, v, out, idx, ws)
    assert e.value.rc == ca.CA_ERR_WORKSPACE


# ---- full-size workloads --------------------------------------------------------------------

def sampled_oracle(w, x_gpu, rows):
    """Oracle on sampled query vectors: each (b, h, r) is solved as a decode over keys 0..i,
    with only that KV slice copied to the host."""
    out_idx, out_ref, diag, qs, ks = {}, {}, {}, {}, {}
    for (b, h, r) in rows:
        i = w.n - w.nq + r
        kvh = h // w.group
        q1 = x_gpu["q"][b, h, r].reshape(1, 1, 1, w.d).cpu()
        k1 = x_gpu["k"][b, kvh, : i + 1].reshape(1, 1, i + 1, w.d).cpu()
        v1 = x_gpu["v"][b, kvh, : i + 1].reshape(1, 1, i + 1, w.d).cpu()
        idx, out, dg = oracle.condensate(q1, k1, v1, w.W, w.topk)
        out_idx[(b, h, r)], out_ref[(b, h, r)], diag[(b, h, r)] = idx, (q1, k1, v1), dg
    return out_idx, out_ref, diag


def check_sampled(w, x_gpu, gpu_out, gpu_idx, rows):
    ref_idx, ref_in, ref_diag = sampled_oracle(w, x_gpu, rows)
    worst = 0.0
    for key in rows:
        b, h, r = key
        q1, k1, v1 = ref_in[key]
        g_idx = gpu_idx[b, h, r].reshape(1, 1, 1, -1)
        compare_sets(g_idx, ref_idx[key], ref_diag[key], q1, k1, w.W, w.topk)
        ref = oracle.restricted(q1, k1, v1, g_idx)
        worst = max(worst, assert_outputs(gpu_out[b, h, r].reshape(1, 1, 1, -1), ref, w.torch_dtype))
    return worst


def test_full_size_decode_131k():
    """The 131K-token GQA decode, in the launch configuration the benchmark times; every query
    vector checked."""
    w = synth.WORKLOADS["decode_131k_gqa_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("full-size decode 131k")
    out, idx = ca.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    torch.cuda.synchronize()
    rows = [(0, h, 0) for h in range(w.heads)]
    check_sampled(w, x, out.cpu().numpy(), idx.cpu().numpy(), rows)
    # The planted needles of each KV head rank high for their query; most are selected.
    idx_np = idx.cpu().numpy()
    found = sum(j in set(idx_np[0, h, r].tolist()) for kv in range(w.kv_heads)
                for (j, h, r) in x["needles"][(0, kv)])
    assert found >= 0.5 * w.kv_heads * w.needles_per_kv_head


def test_full_size_decode_1m_batch4():
    w = synth.WORKLOADS["decode_1m_b4_gqa_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("full-size decode 1m b4")
    out, idx = ca.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    torch.cuda.synchronize()
    rows = [(0, 0, 0), (0, 7, 0), (1, 13, 0), (2, 22, 0), (3, 31, 0), (3, 4, 0)]
    check_sampled(w, x, out.cpu().numpy(), idx.cpu().numpy(), rows)


def test_full_size_prefill_chunk_4k_32k():
    w = synth.WORKLOADS["prefill_chunk_4k_32k_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("full-size prefill chunk 4k x 32k")
    out, idx = ca.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(0)
    rows = [(0, 0, 0), (0, 31, w.nq - 1), (0, 5, 255), (0, 17, 256)]
    rows += [(0, int(torch.randint(w.heads, (1,), generator=g)), int(torch.randint(w.nq, (1,), generator=g)))
             for _ in range(12)]
    check_sampled(w, x, out.cpu().numpy(), idx.cpu().numpy(), rows)


def test_full_size_prefill_131k():
    """Full causal prefill, 8 heads, d = 64, 131,072 positions (every position a query): the
    first W rows have no candidates, the next ones fewer than k."""
    w = synth.WORKLOADS["prefill_131k_h8_bf16"]
    x = synth.make_inputs(w, device="cuda")
    announce("full-size prefill 131k")
    out, idx = ca.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(1)
    rows = [(0, 0, 0), (0, 1, w.W), (0, 2, w.W + 1), (0, 3, w.W + w.topk), (0, 7, w.nq - 1)]
    rows += [(0, int(torch.randint(w.heads, (1,), generator=g)), int(torch.randint(w.nq, (1,), generator=g)))
             for _ in range(11)]
    check_sampled(w, x, out.cpu().numpy(), idx.cpu().numpy(), rows)


@pytest.mark.parametrize("name", ["decode_131k_gqa_w64_bf16", "decode_131k_gqa_w1024_bf16"])
def test_full_size_decode_131k_other_windows(name):
    """The 131K GQA decode with W = 64 and W = 1024; every query vector checked."""
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w, device="cuda")
    announce(f"full-size {name}")
    out, idx = ca.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    torch.cuda.synchronize()
    check_sampled(w, x, out.cpu().numpy(), idx.cpu().numpy(), [(0, h, 0) for h in range(w.heads)])
