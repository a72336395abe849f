"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the cold-cache
replica count, the percentiles, and the HBM-traffic figure taken from the
committed counter summary only while the kernel sources match it."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_replicas_cover_the_requested_bytes():
    for touched in (1, 12_640_256, 202_244_096, 711_784_448, 3 << 30):
        r = bench.replicas_for(touched, 1.0)
        assert r >= 1 and r * touched >= 2 ** 30
        assert r == 1 or (r - 1) * touched < 2 ** 30      # no more than needed
    assert bench.replicas_for(12_640_256, 1.0) == 85     # the one-sequence 32K step


def test_percentiles():
    p = bench.percentiles(np.arange(1, 101, dtype=float))
    assert p["median"] == 50.5 and p["n"] == 100
    assert abs(p["p10"] - 10.9) < 1e-9 and abs(p["p90"] - 90.1) < 1e-9


def test_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    good = tmp_path / "good.txt"
    good.write_text(f"kernel_source_sha1: {bench.kernel_source_hash()}\ntraffic_bytes_per_launch: 9556781\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(good))
    assert bench.measured_traffic() == 9556781.0
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha1: 0000\ntraffic_bytes_per_launch: 9556781\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(stale))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_committed_traffic_summary_matches_the_current_kernel():
    """The summary under profiles/ was taken on the fused kernel as it is now
    (otherwise the bench reports traffic as null and the summary is stale)."""
    assert bench.measured_traffic() is not None
