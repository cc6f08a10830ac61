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

from parity import TOL, assert_outputs, check_sets_rows, compare_sets

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
    # Long windows on the decode path: the anchor-and-window rows go through decode_stream's
    # window workgroups in chunks of 64 (10 chunks here, 5 in the 131K decode and 47 in the
    # near-limit cases): a last chunk of 25 rows, windows that reach position 0 (the first 212
    # rows of the fp32 case, with no candidates, beside rows that have them), and 768 rows in
    # exactly 12 chunks, more than the 7 that decode_finish's wavefronts take at once.
    "long_window_bf16_d128": W_(heads=8, kv_heads=2, n=5000, W=600, topk=32),
    "long_window_f32_d64_early": W_(dtype="f32", d=64, heads=2, kv_heads=1, n=900, nq=600, W=512, topk=16),
    "long_window_bf16_d64_full_chunks": W_(d=64, heads=4, kv_heads=2, n=3000, nq=2, W=767, topk=24),
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


def test_attention_on_subset_more_than_65536_query_vectors():
    """Stage 2 with 2 x 40,000 query vectors (a grid of two rows of workgroups): a set that
    holds only the query's own position gives its own V row back exactly (float32, one weight
    of 1), and a set of the query and the anchor the two-row softmax."""
    n, heads, d = 40000, 2, 64
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, heads, n, d, generator=g)
    k = torch.randn(1, 1, n, d, generator=g)
    v = torch.randn(1, 1, n, d, generator=g)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    p = ca.params(1, heads, 1, d, n, n, 1, 0, "f32")
    pos = torch.arange(n, dtype=torch.int32).view(1, 1, n, 1).expand(1, heads, n, 1)
    idx = torch.cat([pos, torch.full_like(pos, -1)], dim=-1).contiguous()
    announce("subset 80000 query vectors")
    out = torch.empty((1, heads, n, d), dtype=torch.float32, device="cuda")
    ca.attention_on_subset(p, qc, kc, vc, idx.cuda(), out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), v.expand(1, heads, n, d))
    idx2 = torch.cat([pos, -(pos == 0).to(torch.int32)], dim=-1).contiguous()  # no repeats
    ca.attention_on_subset(p, qc, kc, vc, idx2.cuda(), out)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 65535, 65536, 65537, 79999])  # flat query vectors, both heads
    s_self = (q.view(-1, d)[rows].double() * k[0, 0, rows % n].double()).sum(-1) / d ** 0.5
    s_zero = (q.view(-1, d)[rows].double() * k[0, 0, 0].double()).sum(-1) / d ** 0.5
    w0 = torch.sigmoid(s_zero - s_self)  # weight of position 0 (row 0 of each head: itself)
    ref = (1 - w0)[:, None] * v[0, 0, rows % n].double() + w0[:, None] * v[0, 0, 0].double()
    ref[rows % n == 0] = v[0, 0, 0].double()
    got = out.view(-1, d)[torch.from_numpy(rows).cuda()].cpu().double()
    assert torch.allclose(got, ref, rtol=1e-5, atol=1e-5)


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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_clustered_best_rows_then_a_second_round_of_records(dtype):
    """A decode over 140,000 keys reads its block records in two rounds of 512 blocks. The
    cluster sits in the first round, so its blocks are still listed for a second scoring when
    the second round's candidates are cut (by rank counting: fewer than 257 candidates); the
    cut must drop the listed blocks whose rows can no longer rank and keep the others."""
    w = W_(dtype=dtype, heads=4, kv_heads=1, n=140000, nq=1, W=64, topk=48)
    x = clustered_inputs(w, seed=17, start=3001, length=60)
    # A second, shorter run in the second round, scaled to displace part of the first: its rows
    # enter the second round's cut while the first run's block is still listed.
    q = x["q"].float()
    k = x["k"].float()
    d = q[:, 0:4].sum(dim=(1, 2))
    d = d / d.norm(dim=-1, keepdim=True) * 24.0
    gains = 1.3 + 0.01 * torch.arange(20, dtype=torch.float32)
    k[:, 0, 135001:135021] = d[:, None, :] * gains[None, :, None]
    x["k"] = k.to(w.torch_dtype)
    announce(f"clustered two rounds {dtype}")
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

def to_host(x):
    return {t: x[t].cpu() for t in ("q", "k", "v")}


def check_rows(w, xh, gpu_out, gpu_idx, rows):
    """Oracle on the listed (b, h, r) queries (one call over the full tensors, no copies per
    row), sets compared row by row within the band, outputs against the oracle's restricted
    softmax on the GPU's own sets. gpu_out/gpu_idx: [B][Hq][nq][..] numpy. Returns the largest
    relative output error."""
    a = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    ref_idx, _, ref_diag = oracle.condensate(xh["q"], xh["k"], xh["v"], w.W, w.topk, rows=rows)
    g_idx = np.ascontiguousarray(gpu_idx[a[:, 0], a[:, 1], a[:, 2]])
    g_out = gpu_out[a[:, 0], a[:, 1], a[:, 2]]
    pos = w.n - w.nq + a[:, 2]
    check_sets_rows(g_idx, ref_idx, ref_diag, pos, w.W, w.topk,
                    lambda t: oracle.scores(xh["q"], xh["k"], *map(int, a[t])))
    ref = oracle.restricted(xh["q"], xh["k"], xh["v"], g_idx, rows=rows)
    return assert_outputs(g_out, ref, w.torch_dtype)


def run_full_size(w):
    x = synth.make_inputs(w, device="cuda")
    out, idx = ca.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    torch.cuda.synchronize()
    return x, out, idx


def test_full_size_decode_131k_all_32_vectors():
    """The 131K-token GQA decode, in the launch configuration the benchmark times; every query
    vector checked."""
    w = synth.WORKLOADS["decode_131k_gqa_bf16"]
    announce("full-size decode 131k")
    x, out, idx = run_full_size(w)
    idx_np = idx.cpu().numpy()
    check_rows(w, to_host(x), out.cpu().numpy(), idx_np, [(0, h, 0) for h in range(w.heads)])
    # The planted needles of each KV head rank high for their query; most are selected.
    found = sum(j in set(idx_np[0, h, r].tolist()) for kv in range(w.kv_heads)
                for (j, h, r) in x["needles"][(0, kv)])
    assert found >= 0.5 * w.kv_heads * w.needles_per_kv_head


def test_full_size_decode_1m_batch4_all_128_vectors():
    w = synth.WORKLOADS["decode_1m_b4_gqa_bf16"]
    announce("full-size decode 1m b4 (all 128 query vectors)")
    x, out, idx = run_full_size(w)
    out_np, idx_np = out.cpu().numpy(), idx.cpu().numpy()
    xh = to_host(x)
    del x, out, idx
    torch.cuda.empty_cache()
    rows = [(b, h, 0) for b in range(w.batch) for h in range(w.heads)]
    check_rows(w, xh, out_np, idx_np, rows)


def test_full_size_prefill_chunk_4k_32k_all_131072_rows():
    """The 4K x 32K prefill chunk on the MFMA path: every one of the 32 x 4096 query rows."""
    w = synth.WORKLOADS["prefill_chunk_4k_32k_bf16"]
    announce("full-size prefill chunk 4k x 32k (all rows)")
    x, out, idx = run_full_size(w)
    out_np, idx_np = out.cpu().numpy(), idx.cpu().numpy()
    xh = to_host(x)
    ref_idx, _, ref_diag = oracle.condensate(xh["q"], xh["k"], xh["v"], w.W, w.topk)
    compare_sets(idx_np, ref_idx, ref_diag, xh["q"], xh["k"], w.W, w.topk)
    del ref_idx, ref_diag
    ref = oracle.restricted(xh["q"], xh["k"], xh["v"], idx_np)
    assert_outputs(out_np, ref, w.torch_dtype)


def prefill_strata(w, seed, extra_random):
    """Stratified query rows of a full prefill (nq = n): for every head, the rows where R_i
    grows from empty to k (W-2 .. W+k+13), the last and the first row at every 256-vector
    boundary of the MFMA candidate-pass workgroups (vector = row for one query head per KV
    head), the last 16 rows; plus extra_random uniform (head, row) draws."""
    assert w.group == 1
    rows = set()
    for h in range(w.heads):
        rows.update((0, h, r) for r in range(max(0, w.W - 2), min(w.nq, w.W + w.topk + 14)))
        for m in range(256, w.nq, 256):
            rows.update({(0, h, m - 1), (0, h, m)})
        rows.update((0, h, r) for r in range(w.nq - 16, w.nq))
    g = np.random.default_rng(seed)
    rows.update((0, int(h), int(r)) for h, r in zip(g.integers(0, w.heads, extra_random),
                                                     g.integers(0, w.nq, extra_random)))
    return sorted(rows)


def test_full_size_prefill_131k_stratified_9k_rows():
    """Full causal prefill, 8 heads, d = 64, 131,072 positions (every position a query) on the
    MFMA path: about 9,000 stratified rows over all 8 heads (see prefill_strata)."""
    w = synth.WORKLOADS["prefill_131k_h8_bf16"]
    rows = prefill_strata(w, seed=1, extra_random=512)
    announce(f"full-size prefill 131k ({len(rows)} stratified rows)")
    assert len(rows) > 8500
    x, out, idx = run_full_size(w)
    a = np.asarray(rows, dtype=np.int64)
    sel = torch.from_numpy(a).cuda()
    g_out = out[sel[:, 0], sel[:, 1], sel[:, 2]].cpu().numpy()
    g_idx = idx[sel[:, 0], sel[:, 1], sel[:, 2]].cpu().numpy()
    xh = to_host(x)
    del x, out, idx
    ref_idx, _, ref_diag = oracle.condensate(xh["q"], xh["k"], xh["v"], w.W, w.topk, rows=rows)
    pos = w.n - w.nq + a[:, 2]
    check_sets_rows(g_idx, ref_idx, ref_diag, pos, w.W, w.topk,
                    lambda t: oracle.scores(xh["q"], xh["k"], *map(int, a[t])))
    ref = oracle.restricted(xh["q"], xh["k"], xh["v"], g_idx, rows=rows)
    assert_outputs(g_out, ref, w.torch_dtype)


@pytest.mark.parametrize("name", ["prefill_chunk_4k_32k_w1024_bf16", "prefill_chunk_4k_32k_w64_bf16"])
def test_full_size_prefill_chunk_4k_32k_other_windows_2k_rows(name):
    """The 4K x 32K prefill chunk on the MFMA path with W = 1024 and W = 64, in the launch
    configuration of the benchmark: per head the first and last 16 rows and 32 uniform draws
    (2,048 rows over the 32 heads)."""
    w = synth.WORKLOADS[name]
    g = np.random.default_rng(5)
    rows = sorted({(0, h, int(r)) for h in range(w.heads)
                   for r in list(range(16)) + list(range(w.nq - 16, w.nq)) + list(g.integers(16, w.nq - 16, 32))})
    announce(f"full-size {name} ({len(rows)} rows)")
    ca.profile_start(8)
    x, out, idx = run_full_size(w)
    prof = ca.profile_stop()
    assert "mfma_cand" in prof and "mfma_window" in prof, sorted(prof)
    out_np, idx_np = out.cpu().numpy(), idx.cpu().numpy()
    xh = to_host(x)
    del x, out, idx
    check_rows(w, xh, out_np, idx_np, rows)


@pytest.mark.parametrize("W,topk", [(3000, 256), (3000, 512)])
def test_decode_near_the_limits(W, topk):
    """Decode with a 3,000-row window: topk = 256, the largest of the two-kernel decode path
    (1 + W + k = 3,257 entries per set), and topk = 512, the largest of the library (the chunked
    path; 3,513 entries)."""
    w = W_(heads=8, kv_heads=2, n=24000, nq=2, W=W, topk=topk, needles_per_kv_head=32)
    x = synth.make_inputs(w, seed=31)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    announce(f"decode near the limits W={W} topk={topk}")
    ca.profile_start(8)
    out, idx = ca.condensate(q, k, v, w.W, w.topk)
    torch.cuda.synchronize()
    prof = ca.profile_stop()
    assert ("decode_finish" in prof) == (topk <= 256), sorted(prof)
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    idx_np = idx.cpu().numpy()
    compare_sets(idx_np, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
    assert_outputs(out.cpu().numpy(), oracle.restricted(x["q"], x["k"], x["v"], idx_np), w.torch_dtype)


@pytest.mark.parametrize("name", ["decode_131k_gqa_w64_bf16", "decode_131k_gqa_w1024_bf16"])
def test_full_size_decode_131k_other_windows(name):
    """The 131K GQA decode with W = 64 and W = 1024; every query vector checked."""
    w = synth.WORKLOADS[name]
    announce(f"full-size {name}")
    x, out, idx = run_full_size(w)
    check_rows(w, to_host(x), out.cpu().numpy(), idx.cpu().numpy(), [(0, h, 0) for h in range(w.heads)])


def test_workspace_reused_across_calls_shapes_and_paths():
    """One workspace, filled with random bytes before its first use, serves a sequence of calls
    on changing inputs: two decode shapes (the two-kernel decode path, whose records the second
    kernel reads) and a bf16 prefill (the matrix-core path) in between. Every call's sets and
    outputs must match the oracle's."""
    shapes = {
        "A": W_(heads=8, kv_heads=2, n=5000, nq=1, W=64, topk=32),
        "B": W_(heads=4, kv_heads=1, n=9000, nq=2, W=40, topk=48),
        "C": W_(heads=2, kv_heads=2, n=1500, nq=300, W=64, topk=32),
    }
    need = max(ca.workspace_size(ca.params(w.batch, w.heads, w.kv_heads, w.d, w.n, w.nq, w.W, w.topk, "bf16"))
               for w in shapes.values())
    g = torch.Generator(device="cuda").manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)
    for step, (name, seed) in enumerate([("A", 1), ("B", 2), ("A", 3), ("C", 4), ("A", 5), ("B", 6), ("A", 5)]):
        w = shapes[name]
        x = synth.make_inputs(w, seed=seed)
        announce(f"workspace reuse step {step} shape {name}")
        q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
        out, idx = ca.condensate(q, k, v, w.W, w.topk, ws=ws)
        torch.cuda.synchronize()
        out, idx = out.cpu().numpy(), idx.cpu().numpy()
        ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
        compare_sets(idx, ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
        assert_outputs(out, oracle.restricted(x["q"], x["k"], x["v"], idx), w.torch_dtype)


def test_graph_replays_take_fresh_inputs():
    """A decode call captured in a graph and replayed on new inputs copied into the captured
    buffers (the kernel's tags come from the workspace, not from the launch): every replay
    equals an eager call on the same inputs, with the program's own work between replays."""
    w = W_(heads=8, kv_heads=2, n=6000, nq=1, W=64, topk=32)
    xs = [synth.make_inputs(w, seed=s) for s in (11, 12, 13)]
    q, k, v = (xs[0][t].cuda() for t in ("q", "k", "v"))
    p = ca.params_for(q, k, w.W, w.topk)
    ws = ca.alloc_workspace(p)
    out = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.heads, w.nq, w.set_cap), dtype=torch.int32, device="cuda")
    announce("graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ca.condensate_attention_ex(p, q, k, v, out, idx, ws)   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ca.condensate_attention_ex(p, q, k, v, out, idx, ws)
    torch.cuda.synchronize()
    for rep in range(6):
        x = xs[rep % 3]
        q.copy_(x["q"]); k.copy_(x["k"]); v.copy_(x["v"])
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_idx = out.clone(), idx.clone()
        eager_out, eager_idx = ca.condensate(q, k, v, w.W, w.topk)
        torch.cuda.synchronize()
        assert torch.equal(got_idx, eager_idx), f"replay {rep}: sets differ from the eager call"
        assert torch.equal(got_out.view(torch.int32), eager_out.view(torch.int32)), f"replay {rep}: outputs differ"
    ref_idx, _, ref_diag = oracle.condensate(x["q"], x["k"], x["v"], w.W, w.topk)
    compare_sets(got_idx.cpu().numpy(), ref_idx, ref_diag, x["q"], x["k"], w.W, w.topk)
