"""Host-side logic of bench.py (CPU only): the one-GPU guard, the byte counts it prices the
kernels against, and the traffic figure it reads from the committed rocprofv3 summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_workloads():
    # fwd_b8_t2048: per token-head q, k, z (bf16, M = 64), v (bf16, 128), f (fp32), o (fp32,
    # 128); per head the fp32 final state 64 x 128
    rows, heads = 8 * 2048 * 8, 8 * 8
    assert bench.forward_bytes(8, 2048, 8, 64, 128, 2) == rows * (3 * 64 * 2 + 128 * 2 + 4 + 128 * 4) \
        + heads * 64 * 128 * 4
    assert round(bench.forward_bytes(8, 2048, 8, 64, 128, 2) / 1e6, 1) == 153.6
    # decode_b256: the state read, K = 16 rows written back, the step's inputs and o
    assert round(bench.decode_bytes(256, 16, 64, 128, 16, 2) / 1e6, 1) == 172.5


def test_traffic_is_read_only_for_the_profiled_sources(monkeypatch):
    if not os.path.exists(bench.TRAFFIC_FILE):
        pytest.skip("no traffic summary")
    text = open(bench.TRAFFIC_FILE).read()
    sha = [ln.split(":", 1)[1].strip() for ln in text.splitlines() if ln.startswith("source_sha256:")][0]
    want = float([ln.split(":", 1)[1] for ln in text.splitlines() if ln.startswith("hbm_bytes_per_call:")][0])
    monkeypatch.setattr(bench, "forward_sources_sha256", lambda: sha)
    assert bench.measured_traffic() == want
    monkeypatch.setattr(bench, "forward_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic() is None
