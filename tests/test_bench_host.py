"""Host-side logic of bench.py (no GPU): the algorithmic byte count of a GEMV launch, the
counter summary gate on the GEMV source hash, and the refusal of more than one GPU."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_gemv_bytes_model():
    # codes N*K/2 + fp16 scale and zero 4*N*K/g + X 2*M*K + Y 4*M*N
    assert bench.gemv_bytes(1, 2048, 2048, 128) == 2048 * 1024 + 4 * 2048 * 16 + 2 * 2048 + 4 * 2048
    assert bench.gemv_bytes(4, 16384, 16384, 128) == 16384 * 8192 + 4 * 16384 * 128 + 8 * 16384 + 16 * 16384
    # 0.53125 bytes per weight at g = 128 before X and Y
    n, k = 12288, 4096
    assert (bench.gemv_bytes(1, n, k, 128) - 2 * k - 4 * n) / (n * k) == pytest.approx(0.53125)


def test_step_bytes_of_the_sweep():
    total = sum(bench.gemv_bytes(m, n, k, bench.DECODE_G) for n, k in bench.DECODE_SHAPES for m in (1, 2, 3, 4))
    assert total == 1155755008


def test_traffic_needs_matching_source_hash(tmp_path, monkeypatch):
    d = {"source_hash": bench.source_hash("gemv.hip", "common.h"), "traffic_bytes_per_launch": 123}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gemv_decode_sweep_counters.json").write_text(json.dumps(d))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda *names: d["source_hash"])
    assert bench.load_traffic(0.0) == 123
    monkeypatch.setattr(bench, "source_hash", lambda *names: "0" * 16)
    assert bench.load_traffic(0.0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""
