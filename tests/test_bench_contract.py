"""bench.py's contract pieces that run without a GPU: the one-GPU guard, the
oracle CPU baseline object, and the stale-profile rule for the traffic field."""
import json
import os
import subprocess
import sys

import bench
import attn_inputs as ai

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_object():
    w = ai.WORKLOADS["single_head_fwd_n256_d64_f16"]
    dr = ai.draw_workload(w)
    cb = bench.cpu_baseline(w, dr, budget_s=0.01, workers=2)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] == 2
    # two 128-row units, one per worker (each worker does at least one)
    assert "2 of 2 (head, 128-query-row block) units" in cb["sample"]


def test_cpu_pool_size_follows_the_affinity_mask():
    n = bench.cpu_pool_size()
    assert 1 <= n <= 16 and n <= len(os.sched_getaffinity(0))


def test_traffic_is_null_unless_taken_on_these_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    entry = {"bytes_per_launch": 12345}
    f.write_text(json.dumps({"wl": {"fa_fwd": dict(entry, source_hash=bench.kernel_source_hash()),
                                    "fa_bwd": dict(entry, source_hash="0" * 16)}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("wl", "fa_fwd") == 12345
    assert bench.measured_traffic("wl", "fa_bwd") is None       # taken on other kernel sources
    assert bench.measured_traffic("other", "fa_fwd") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("wl", "fa_fwd") is None
