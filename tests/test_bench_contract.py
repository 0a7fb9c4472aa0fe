"""bench.py's reporting contract, checked on the CPU: the multi-GPU refusal, the CPU-baseline record
and the rule that counter traffic is reported only for the kernel source it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_traffic_only_for_the_profiled_source(monkeypatch, tmp_path):
    rec = {"kernel_sha256_16": "0123456789abcdef", "bytes_per_launch": {"prefill_65536": 123.0}}
    path = tmp_path / "counters.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "COUNTERS", str(path))
    monkeypatch.setattr(bench, "kernel_digest", lambda *a: "0123456789abcdef")
    assert bench.counter_traffic("prefill_65536") == 123.0
    assert bench.counter_traffic("decode_64") is None
    monkeypatch.setattr(bench, "kernel_digest", lambda *a: "fedcba9876543210")
    assert bench.counter_traffic("prefill_65536") is None


def test_committed_counters_name_the_digest_they_were_taken_on():
    with open(bench.COUNTERS) as f:
        rec = json.load(f)
    assert len(rec["kernel_sha256_16"]) == 16
    for key in ("prefill_65536", "decode_64"):
        assert rec["bytes_per_launch"][key] > rec["algorithmic_bytes_per_launch"][key] * 0.99


def test_cpu_baseline_record():
    from paged_kv_cache_msa_amd import workloads as W
    rec = bench.cpu_baseline(W, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and "tokens" in rec["sample"]
