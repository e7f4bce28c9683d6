"""Host-side logic of bench.py: the one-GPU guard and the lookup of counter
figures recorded for a kernel's exact sources.  No GPU is used."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (its main() runs only as a script)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus must be 1" in r.stderr


def _fake_root(tmp_path, body=b"kernel source v1"):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_bytes(body)
    rec = {"kernels": {"k": {"sources": ["k.hip"],
                             "sha256": hashlib.sha256(body).hexdigest(),
                             "traffic_bytes": 1234.0,
                             "mfma_busy_frac": 0.25}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))


def test_counter_figures_follow_the_recorded_sources(tmp_path, monkeypatch):
    _fake_root(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("k") == 1234.0
    assert bench.profiled_traffic("k", "mfma_busy_frac") == 0.25
    assert bench.profiled_traffic("k", "no_such_field") is None
    assert bench.profiled_traffic("other_kernel") is None
    # a changed source invalidates every figure taken from the old build
    (tmp_path / "k.hip").write_bytes(b"kernel source v2")
    assert bench.profiled_traffic("k") is None
    assert bench.profiled_traffic("k", "mfma_busy_frac") is None


def test_missing_profile_gives_none(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("k") is None


@pytest.mark.parametrize("kernel", ["chunked_mfma_kernel", "recurrent_kernel"])
def test_committed_profile_has_the_bench_kernels(kernel):
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["kernels"][kernel]
    assert rec["traffic_bytes"] > 0 and rec["sources"]
