"""bench.py's contract pieces that run without a GPU: the one-GPU refusal and
the gate that reports measured HBM traffic only for the kernel sources the
counters were taken on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_committed_traffic_matches_current_kernel_sources():
    """Every committed traffic record names the hash of the sources it was
    measured on; the decode ones must match the sources as they stand."""
    for w in ("llama13b", "llama70b", "llama13b_fp8"):
        with open(os.path.join(ROOT, "profiles", f"traffic_{w}.json")) as f:
            t = json.load(f)
        assert t["kernel_source_hash"] == bench.kernel_source_hash("decode"), w
        assert bench.load_traffic(w) == t["bytes_per_call"]
        # reads within a few percent of the algorithmic bytes
        assert 0.95 < t["read_bytes"] / t["algorithmic_bytes"] < 1.05, w


def test_traffic_is_withheld_for_other_sources(tmp_path, monkeypatch):
    rec = {"workload": "llama13b", "kernel_source_hash": "0" * 16, "bytes_per_call": 123}
    (tmp_path / "traffic_llama13b.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.load_traffic("llama13b") is None
    rec["kernel_source_hash"] = bench.kernel_source_hash("decode")
    (tmp_path / "traffic_llama13b.json").write_text(json.dumps(rec))
    assert bench.load_traffic("llama13b") == 123
    assert bench.load_traffic("no_such_workload") is None


def test_kernel_source_hash_covers_each_family():
    hashes = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert all(len(h) == 16 for h in hashes.values())
    assert len(set(hashes.values())) == len(hashes)  # families hash differently
