"""Host logic of bench.py (no GPU): the one-GPU guard and the lookup of the recorded HBM
counters, which must name the timed workload and the current kernel sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_matches_workload_and_sources(tmp_path, monkeypatch):
    # The committed summary names the decode workload and the current sources' hash.
    t = bench.recorded_traffic("decode_131k_gqa_bf16")
    assert t is not None and 2.5e8 < t < 3.0e8
    assert bench.recorded_traffic("prefill_chunk_4k_32k_bf16") is None
    # A summary taken on other sources is not used.
    stale = tmp_path / "counters.md"
    text = open(bench.COUNTERS).read()
    stale.write_text(text.replace(bench.kernel_sources_sha(), "0" * 16))
    monkeypatch.setattr(bench, "COUNTERS", str(stale))
    assert bench.recorded_traffic("decode_131k_gqa_bf16") is None
