"""Seeded synthetic inputs shaped like the workloads of the condensate-attention pages.

This module only draws and places numbers: Gaussian Q/K/V, the anchor bias on key 0,
the query bias, and planted "needle" keys. It holds none of the method's arithmetic
(no scores, no selection, no softmax), so both the CPU oracle and the HIP path can be
fed from it without sharing any part of the computation.

Recipe, per tensor, in this order: draw N(0,1) in float32 -> scale -> anchor bias
(key 0 += anchor_bias*u) and query bias (every query += query_bias*u) -> needles
(a key set to needle_norm * q/|q| for a chosen query q, at a position that query can
only reach through its top-k part) -> cast to the workload dtype.

u is a fixed unit vector (a normalised N(0, I_d) draw). Every tensor slice has its own
seeded generator, so a slice can be rebuilt alone and on any device. The bytes depend on
the device the big tensors are drawn on (torch's CPU and GPU generators differ); both
sides of a parity check always read the same bytes, copied from wherever they were drawn.

The shapes come from "The Condensate Theorem" pages (metaphor-xennon blog, sections 2.1
(Definition 1), 4.3 (multi-needle haystack) and 5.1.2 (H=8, d_k=64 timing setup)); the
distributions are the synthetic stand-ins described above, since the pages' prompts and
trained checkpoints are not available.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

_MASK64 = (1 << 64) - 1


def _mix(*parts: int) -> int:
    """SplitMix64-style mixing of integers into a 63-bit torch seed."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h = (h ^ (p & _MASK64)) & _MASK64
        h = (h + 0x9E3779B97F4A7C15) & _MASK64
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        h = z ^ (z >> 31)
    return h & ((1 << 63) - 1)


_TAG = {"u": 1, "q": 2, "k": 3, "v": 4, "needle": 5}


@dataclass(frozen=True)
class Workload:
    """One synthetic problem: sizes, method parameters and the input recipe."""

    name: str
    batch: int
    heads: int
    kv_heads: int
    d: int
    n: int          # keys in the cache (positions 0..n-1)
    nq: int         # queries = the last nq positions
    dtype: str      # "f32" or "bf16"
    W: int          # local window
    topk: int       # dynamic top-k
    q_scale: float = 1.0
    k_scale: float = 1.0
    anchor_bias: float = 3.0
    query_bias: float = 1.0
    needles_per_kv_head: int = 0
    needle_norm: float = 4.0
    mode: str = "decode"  # "decode" or "prefill" (informational)

    @property
    def group(self) -> int:
        return self.heads // self.kv_heads

    @property
    def set_cap(self) -> int:
        return 1 + self.W + self.topk

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a small prefill the oracle finishes in seconds, an 8K MHA decode,
# the 131K GQA decode, a 4K-query prefill chunk over 32K keys and a 1M-token batch-4 decode;
# then a full 131K prefill and the 131K decode at other window sizes.
WORKLOADS = {
    "prefill_1k_f32": Workload(
        "prefill_1k_f32", batch=1, heads=1, kv_heads=1, d=64, n=1024, nq=1024, dtype="f32",
        W=64, topk=16, q_scale=2.0, k_scale=2.0, needles_per_kv_head=8, mode="prefill"),
    "decode_8k_mha_f32": Workload(
        "decode_8k_mha_f32", batch=1, heads=12, kv_heads=12, d=64, n=8192, nq=1, dtype="f32",
        W=128, topk=32, q_scale=2.0, needles_per_kv_head=16),
    "decode_131k_gqa_bf16": Workload(
        "decode_131k_gqa_bf16", batch=1, heads=32, kv_heads=8, d=128, n=131072, nq=1,
        dtype="bf16", W=256, topk=64, q_scale=2.0, needles_per_kv_head=64),
    "prefill_chunk_4k_32k_bf16": Workload(
        "prefill_chunk_4k_32k_bf16", batch=1, heads=32, kv_heads=32, d=128, n=32768, nq=4096,
        dtype="bf16", W=256, topk=64, q_scale=1.0, needles_per_kv_head=256, mode="prefill"),
    "decode_1m_b4_gqa_bf16": Workload(
        "decode_1m_b4_gqa_bf16", batch=4, heads=32, kv_heads=8, d=128, n=1048576, nq=1,
        dtype="bf16", W=256, topk=128, q_scale=2.0, needles_per_kv_head=512),
    # Full causal prefill at the shape of the pages' timing table (section 5.1.2: 8 heads,
    # d = 64, 131,072 tokens), with the defaults of their two-stage sketch (section 5.2.2:
    # W = 64, k = 32).
    "prefill_131k_h8_bf16": Workload(
        "prefill_131k_h8_bf16", batch=1, heads=8, kv_heads=8, d=64, n=131072, nq=131072,
        dtype="bf16", W=64, topk=32, q_scale=1.0, needles_per_kv_head=64, mode="prefill"),
    # The 131K GQA decode with the other windows of the pages' per-layer schedule (sections
    # 6.1-6.2: W = 1024 in the shallow quarter of the layers, 256 in the next quarter, 64 in
    # the deep half).
    "decode_131k_gqa_w64_bf16": Workload(
        "decode_131k_gqa_w64_bf16", batch=1, heads=32, kv_heads=8, d=128, n=131072, nq=1,
        dtype="bf16", W=64, topk=64, q_scale=2.0, needles_per_kv_head=64),
    "decode_131k_gqa_w1024_bf16": Workload(
        "decode_131k_gqa_w1024_bf16", batch=1, heads=32, kv_heads=8, d=128, n=131072, nq=1,
        dtype="bf16", W=1024, topk=64, q_scale=2.0, needles_per_kv_head=64),
    # The 4K x 32K prefill chunk with the shallow layers' window (W = 1024) and the deep
    # layers' (W = 64).
    "prefill_chunk_4k_32k_w1024_bf16": Workload(
        "prefill_chunk_4k_32k_w1024_bf16", batch=1, heads=32, kv_heads=32, d=128, n=32768, nq=4096,
        dtype="bf16", W=1024, topk=64, q_scale=1.0, needles_per_kv_head=256, mode="prefill"),
    "prefill_chunk_4k_32k_w64_bf16": Workload(
        "prefill_chunk_4k_32k_w64_bf16", batch=1, heads=32, kv_heads=32, d=128, n=32768, nq=4096,
        dtype="bf16", W=64, topk=64, q_scale=1.0, needles_per_kv_head=256, mode="prefill"),
}

WORKLOAD_ORDER = list(WORKLOADS)


def default_seed(w: Workload) -> int:
    return 1000 + (WORKLOAD_ORDER.index(w.name) if w.name in WORKLOADS else 99)


def _gen(device, seed: int, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(seed, *parts))
    return g


def unit_vector(w: Workload, seed: int) -> torch.Tensor:
    """The fixed unit vector u (float32, CPU)."""
    g = _gen("cpu", seed, _TAG["u"])
    u = torch.randn(w.d, generator=g, dtype=torch.float32)
    return u / u.norm()


def _needle_plan(w: Workload, seed: int):
    """Needle placements: list per (b, kv head) of (key position j, query head h, query row r).

    Each needle picks a query uniformly among those whose candidate range {1..i-W} is
    non-empty, then a key position uniformly in that range; positions within one
    (b, kv head) are distinct.
    """
    plan = {}
    first_pos = w.n - w.nq
    rows = [r for r in range(w.nq) if first_pos + r - w.W >= 1]
    for b in range(w.batch):
        for kvh in range(w.kv_heads):
            out = []
            if rows and w.needles_per_kv_head > 0:
                g = _gen("cpu", seed, _TAG["needle"], b, kvh)
                used = set()
                tries = 0
                while len(out) < w.needles_per_kv_head and tries < 50 * w.needles_per_kv_head:
                    tries += 1
                    h = kvh * w.group + int(torch.randint(w.group, (1,), generator=g))
                    r = rows[int(torch.randint(len(rows), (1,), generator=g))]
                    i = first_pos + r
                    j = 1 + int(torch.randint(i - w.W, (1,), generator=g))
                    if j in used:
                        continue
                    used.add(j)
                    out.append((j, h, r))
            plan[(b, kvh)] = out
    return plan


def make_inputs(w: Workload, seed: int | None = None, device="cpu"):
    """Draw q [B][Hq][nq][d], k and v [B][Hkv][n][d] in w.dtype on `device`.

    Returns a dict with 'q', 'k', 'v' (contiguous tensors), 'u' and 'needles'
    ({(b, kv_head): [(j, h, r), ...]}).
    """
    if seed is None:
        seed = default_seed(w)
    dev = torch.device(device)
    u = unit_vector(w, seed)
    u_dev = u.to(dev)
    dt = w.torch_dtype

    q32 = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device=dev)
    for b in range(w.batch):
        for h in range(w.heads):
            g = _gen(dev, seed, _TAG["q"], b, h)
            x = torch.randn((w.nq, w.d), generator=g, dtype=torch.float32, device=dev)
            q32[b, h] = x * w.q_scale + w.query_bias * u_dev
    plan = _needle_plan(w, seed)

    k = torch.empty((w.batch, w.kv_heads, w.n, w.d), dtype=dt, device=dev)
    v = torch.empty((w.batch, w.kv_heads, w.n, w.d), dtype=dt, device=dev)
    for b in range(w.batch):
        for kvh in range(w.kv_heads):
            g = _gen(dev, seed, _TAG["k"], b, kvh)
            x = torch.randn((w.n, w.d), generator=g, dtype=torch.float32, device=dev)
            if w.k_scale != 1.0:
                x.mul_(w.k_scale)
            x[0] += w.anchor_bias * u_dev
            for (j, h, r) in plan[(b, kvh)]:
                qv = q32[b, h, r]
                x[j] = w.needle_norm * qv / qv.norm()
            k[b, kvh] = x.to(dt)
            del x
            g = _gen(dev, seed, _TAG["v"], b, kvh)
            v[b, kvh] = torch.randn((w.n, w.d), generator=g, dtype=torch.float32, device=dev).to(dt)
    q = q32.to(dt).contiguous()
    return {"q": q, "k": k, "v": v, "u": u, "needles": plan}


def query_position(w: Workload, r: int) -> int:
    """Absolute position of query row r (queries are the last nq positions)."""
    return w.n - w.nq + r
