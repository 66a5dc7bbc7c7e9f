"""Host-side logic of bench.py (no GPU): the one-GPU guard, the recorded
Stage-2 traffic and its source digest, the popcount used for selection
statistics, and the oracle CPU-baseline leg on a tiny workload."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from differentiable_adaptive_block_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_matches_committed_sources():
    # the committed counter summary was taken on the committed Stage-2 sources
    t = bench.recorded_traffic()
    assert t is not None and t > 0


def test_recorded_traffic_ignores_other_sources(tmp_path, monkeypatch):
    good = open(bench.TRAFFIC_FILE).read()
    bad = good.replace(bench.stage2_digest(), "0" * 16)
    assert bad != good
    f = tmp_path / "traffic.md"
    f.write_text(bad)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic() is None


def test_popcount32(monkeypatch):
    monkeypatch.setattr(bench, "torch", torch, raising=False)
    rng = np.random.default_rng(3)
    x = rng.integers(0, 2**32, size=4096, dtype=np.uint64)
    x[:4] = [0, 1, 2**32 - 1, 2**31]
    got = bench._popcount32(torch.from_numpy(x.astype(np.int64)).to(torch.int32)).tolist()
    assert got == [bin(int(v)).count("1") for v in x]


def test_cpu_baseline_leg_tiny(monkeypatch):
    monkeypatch.setattr(bench, "torch", torch, raising=False)
    wl = inputs.CONFIGS["prefill16k"]
    w = inputs.make_prefill(1, 2, 256, 64, "bf16", True, (1, 2), seed=5, device="cpu", with_dout=False)
    r = bench.cpu_baseline(w, wl, 1.5, rows_per_worker=8, workers=2)
    assert set(r) == {"value", "unit", "cores", "kind", "sample", "host_cpu_count", "blas_threads_per_process"}
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["unit"] == "tokens/s"
    assert r["value"] > 0 and "16 query rows" in r["sample"]


def test_median_and_columns():
    assert bench._median([3.0, 1.0, 2.0]) == 2.0
    assert bench._median([4.0, 1.0, 2.0, 3.0]) == 2.5
    assert bench._col([[1, 2], [3, 4]], 1) == [2, 4]
