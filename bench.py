"""Benchmark of the condensate-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--chunk C] [--rotate R]

A step is one call of ca_condensate_attention_ex: scores over every causal key, the anchor /
window / exact top-k set, and the restricted softmax times V -- the whole path, on one batch of
synthetic inputs already resident in HBM. The default workload is the 131,072-token GQA decode
step (32 query heads, 8 KV heads, d=128, bf16, W=256, k=64). Distinct KV buffer sets are rotated
between steps so that the key stream comes from HBM and not from the 256 MB last-level cache.

Prints one JSON line: query vectors/s from a clean timed loop, the step's algorithmic HBM GB/s,
the roofline of the dominant kernel (on the decode path decode_stream, which reads every key row;
on the prefill paths the score stage; durations from HIP events the library records around its
own launches on the stream it uses, in a second pass over the same steps), and the CPU oracle
timed on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "condensate-attn decode queries/sec + achieved HBM GB/s at 131K ctx (1 GPU)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of the chip
# HBM bytes per launch of decode_stream (the dominant kernel of the decode step) from rocprofv3
# FETCH_SIZE / WRITE_SIZE counters, valid while the kernel's sources hash to the recorded value.
COUNTERS = os.path.join(ROOT, "profiles", "decode_stream_decode_131k_gqa_bf16_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_transformer_attention_amd", "csrc", f)
                  for f in ("decode_stream.hip", "decode_core.h", "score_core.h", "device_utils.h")]


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per score-stage launch from the committed counter summary, or None when the
    summary is absent, is for another workload, or predates the current kernel sources."""
    if not os.path.exists(COUNTERS):
        return None
    text = open(COUNTERS).read()
    m_sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]+)", text)
    m_wl = re.search(r"workload:\s*(\S+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_wl and m_b) or m_wl.group(1) != workload or m_sha.group(1) != kernel_sources_sha():
        return None
    return float(m_b.group(1))


def cpu_info():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_131k_gqa_bf16")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=0, help="KV buffer sets (0 = enough for 1 GiB of K)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mass", action="store_true",
                    help="time the call with the mass diagnostic (decode and MFMA prefill paths)")
    ap.add_argument("--dense", action="store_true",
                    help="time dense causal attention (bf16) on the workload instead of the method")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.mul(src, 1.0, out=dst)   # one elementwise kernel: reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        e0.record()
        for _ in range(9):
            torch.mul(src, 1.0, out=dst)
        e1.record()
        torch.cuda.synchronize()
        copy_s = e0.elapsed_time(e1) / 1e3 / 9
        # (Context for the achievable HBM bandwidth: GB/s moved by this plain copy.)
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "launches": 10,
                          "copy_gbps": 2 * (1 << 30) / copy_s / 1e9}))
        return

    import numpy as np
    import sparse_transformer_attention_amd as ca
    from sparse_transformer_attention_amd import synth

    w = synth.WORKLOADS[args.workload]
    seed = synth.default_seed(w) if args.seed is None else args.seed
    x = synth.make_inputs(w, seed=seed, device="cuda")
    eb = w.elem_bytes
    k_bytes = w.batch * w.kv_heads * w.n * w.d * eb
    rotate = args.rotate or max(1, -(-(1 << 30) // k_bytes))
    sets = [(x["k"], x["v"])] + [(x["k"].clone(), x["v"].clone()) for _ in range(rotate - 1)]
    q = x["q"]
    p = ca.params_for(q, x["k"], w.W, w.topk, args.chunk)
    ws = ca.alloc_workspace(p)
    out = torch.empty((w.batch, w.heads, w.nq, w.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.heads, w.nq, w.set_cap), dtype=torch.int32, device="cuda")

    mass = torch.empty((w.batch, w.heads, w.nq, 4), dtype=torch.float32, device="cuda") if args.mass else None

    def step(s):
        kk, vv = sets[s % rotate]
        if args.dense:
            ca.dense_attention_ex(p, q, kk, vv, out)
        elif args.mass:
            ca.condensate_attention_mass_ex(p, q, kk, vv, out, idx, mass, ws)
        else:
            ca.condensate_attention_ex(p, q, kk, vv, out, idx, ws)

    for s in range(args.warmup):
        step(s)
    # Timed region: K steps back to back, nothing else on the stream.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in range(args.steps):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    # The same K steps again with the library's profiler on: HIP events recorded around each of
    # its launches, on the stream it launches on, give every kernel's average duration (the
    # events themselves add a little time per step, so this pass is not the one timed above).
    torch.cuda.synchronize()
    ca.profile_start(4 * args.steps)
    t1 = time.perf_counter()
    for s in range(args.steps):
        step(s)
    torch.cuda.synchronize()
    ms_per_step_profiled = (time.perf_counter() - t1) * 1e3 / args.steps
    prof = ca.profile_stop()
    # Per-step spread: a third pass with an event pair around every step on the stream the
    # library launches on (torch's current stream), for the median and the 10th / 90th
    # percentiles of the step's GPU time.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s, (e0, e1) in enumerate(evs):
        e0.record()
        step(s)
        e1.record()
    torch.cuda.synchronize()
    per_step_us = np.sort(np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]))
    step_spread = {"median": float(np.median(per_step_us)),
                   "p10": float(np.percentile(per_step_us, 10)),
                   "p90": float(np.percentile(per_step_us, 90))}

    # Algorithmic bytes. The score stage reads the key rows of the candidate range once per KV
    # head plus the queries; the whole step reads all of K, the distinct V rows of the sets,
    # the queries, and writes the outputs and index sets.
    rmax = max(0, w.n - 1 - w.W)
    q_bytes = w.batch * w.heads * w.nq * w.d * eb
    score_bytes = w.batch * w.kv_heads * rmax * w.d * eb + q_bytes
    idx_np = idx.cpu().numpy() if not args.dense else np.full(idx.shape, -1, dtype=np.int32)
    v_rows = 0
    for b in range(w.batch):
        for kvh in range(w.kv_heads):
            rows = idx_np[b, kvh * w.group:(kvh + 1) * w.group].reshape(-1)
            v_rows += len(np.unique(rows[rows >= 0]))
    step_bytes = (k_bytes + v_rows * w.d * eb + q_bytes + w.batch * w.heads * w.nq * w.d * 4
                  + idx_np.size * 4)
    nqv = w.batch * w.heads * w.nq

    if args.dense:
        # Dense causal attention: q.k and the weights times V for every causal pair.
        nd, td = prof.get("dense", (0, 0.0))
        dense_s = td / max(1, nd) / 1e3
        pos0 = w.n - w.nq
        pairs = w.batch * w.heads * (w.nq * (pos0 + 1) + w.nq * (w.nq - 1) // 2)
        flops = 4 * w.d * pairs
        ach = flops / dense_s / 1e12 if nd else None
        roofline = {
            "kernel": "dense (mfma_window over every causal row)",
            "bound": "mfma",
            "achieved": ach,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": ach / MFMA_BF16_PEAK_TFLOPS if ach else None,
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": dense_s * 1e6,
        }
    elif "mfma_bound" in prof:
        # Prefill path: the scores of every causal pair j <= i are a dense bf16 product run on
        # the matrix cores, twice (bound pass, candidate pass); the algorithmic work is one.
        nb, tb = prof["mfma_bound"]
        nc, tc = prof["mfma_cand"]
        pass_s = (tb / max(1, nb) + tc / max(1, nc)) / 1e3
        pos0 = w.n - w.nq
        pairs = w.batch * w.heads * (w.nq * (pos0 + 1) + w.nq * (w.nq - 1) // 2)
        flops = 2 * w.d * pairs
        ach = flops / pass_s / 1e12
        roofline = {
            "kernel": "mfma_bound + mfma_cand (score stage)",
            "bound": "mfma",
            "achieved": ach,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": ach / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": pass_s * 1e6,
        }
    if "decode_stream" in prof and not args.dense:
        # Decode path: decode_stream reads every candidate key row once (the score stage) and,
        # in its last workgroups, the K and V rows of the anchors and windows (the distinct
        # rows: the windows of the nq query rows of a KV head overlap, position 0 once);
        # decode_finish (selection, set assembly, attend) follows it.
        launches, dec_ms = prof["decode_stream"]
        dec_avg_s = dec_ms / max(1, launches) / 1e3
        win_rows = min(w.n, w.W + w.nq - 1)
        win_rows += 1 if w.n - w.nq - w.W + 1 > 0 else 0
        score_bytes += w.batch * w.kv_heads * win_rows * 2 * w.d * eb
        achieved = score_bytes / dec_avg_s / 1e9
        # The recorded counters are those of the kernel without the mass diagnostic.
        traffic = recorded_traffic(w.name) if not args.mass else None
        roofline = {
            "kernel": "decode_stream (score stage: every key row once, block records; "
                      "anchor-and-window partials)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": score_bytes,
            "avg_launch_us": dec_avg_s * 1e6,
        }
    elif "mfma_bound" not in prof and not args.dense:
        # Chunked path: score_topk (profiled as score_select) is the score stage.
        launches, score_ms = prof.get("score_select", (0, 0.0))
        score_avg_s = score_ms / max(1, launches) / 1e3
        achieved = score_bytes / score_avg_s / 1e9 if launches else None
        roofline = {
            "kernel": "score_topk (score stage)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": (achieved / HBM_PEAK_GBPS) if achieved else None,
            "traffic": None,
            "algorithmic_bytes_per_launch": score_bytes,
            "avg_launch_us": score_avg_s * 1e6,
        }
    kernels = {name: {"launches": n, "avg_us": round(t / max(1, n) * 1e3, 3)} for name, (n, t) in prof.items()}

    record = {
        "metric": METRIC,
        "value": nqv / (ms_per_step / 1e3),
        "unit": "query vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "kv_heads": w.kv_heads,
                   "d": w.d, "n": w.n, "nq": w.nq, "W": w.W, "topk": w.topk, "accumulate": "f32",
                   "chunk": args.chunk or "auto", "kv_sets_rotated": rotate, "seed": seed,
                   "mass_diagnostic": bool(args.mass), "dense_baseline": bool(args.dense)},
        "hbm_gbps": step_bytes / (ms_per_step / 1e3) / 1e9,
        "step_algorithmic_bytes": step_bytes,
        "gpu_ms_per_step": gpu_ms / args.steps,
        "ms_per_step_profiled": ms_per_step_profiled,
        "step_us_events": step_spread,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        import oracle
        qc, kc, vc = q.cpu(), x["k"].cpu(), x["v"].cpu()

        def oracle_rate(threads, seconds):
            """Query vectors per second of the oracle on `threads` threads (0: all), over about
            `seconds` of CPU work on the same workload, and what the sample was."""
            reps, t_cpu, vectors = 0, 0.0, 0
            if nqv * w.n <= (1 << 28):
                # Whole steps.
                while t_cpu < seconds:
                    t1 = time.perf_counter()
                    oracle.condensate(qc, kc, vc, w.W, w.topk, threads)
                    t_cpu += time.perf_counter() - t1
                    reps += 1
                vectors = reps * nqv
                sample = (f"{reps} whole steps of the same workload ({nqv} query vectors each "
                          f"over {w.n} keys), float64, {t_cpu:.1f} s")
            else:
                # A whole step is far beyond the time budget: blocks of m consecutive query
                # positions at random places, all heads, each block solved as the last m
                # positions of the keys up to its last one (the same computation as inside a
                # whole step).
                m = min(16, w.nq)
                rng = np.random.default_rng(seed)
                while t_cpu < seconds:
                    r0 = int(rng.integers(0, w.nq - m + 1))
                    last = w.n - w.nq + r0 + m - 1
                    qb = qc[:, :, r0:r0 + m].contiguous()
                    kb, vb = kc[:, :, :last + 1].contiguous(), vc[:, :, :last + 1].contiguous()
                    t1 = time.perf_counter()
                    oracle.condensate(qb, kb, vb, w.W, w.topk, threads)
                    t_cpu += time.perf_counter() - t1
                    vectors += w.batch * w.heads * m
                    reps += 1
                sample = (f"{reps} blocks of {m} consecutive query positions x "
                          f"{w.batch * w.heads} query heads at random positions of the workload "
                          f"({vectors} query vectors, each over its causal keys), float64, "
                          f"{t_cpu:.1f} s")
            return vectors / t_cpu, sample

        value_all, sample = oracle_rate(0, args.cpu_seconds)
        cores = oracle.threads_used()
        # (Last: a thread count set for one call stays set for the process.)
        value_one, sample_one = oracle_rate(1, max(2.0, args.cpu_seconds / 4))
        record["cpu_baseline"] = {
            "value": value_all,
            "unit": "query vectors/s",
            "cores": cores,
            "kind": "oracle",
            "sample": sample,
            "cpu": cpu_info(),
            "single_thread_value": value_one,
            "single_thread_sample": sample_one,
        }
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
