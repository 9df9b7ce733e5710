"""Host-side logic of bench.py (no GPU): the one-GPU guard, the exact-pair accounting of a
selection, and the rule that the traffic figure is reported only for the kernel sources it was
measured on."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gen import workload  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_selection_stats_counts_exact_pairs_and_centroids():
    # four query blocks of 64 rows over M = 4 key blocks; query block 1 is dense
    w = workload(1, T=1, Hh=16, Ww=16, H=1, dense_rows=(64, 128))
    assert w.N == 256
    M = 4
    sel = {
        "kept_cnt": np.array([[1, 4, 2, 3]], dtype=np.int32),
        "extra_cnt": np.array([[5, 7, 0, 1]], dtype=np.int32),
        "mult": np.zeros((1, 4, 64), dtype=np.uint8),
    }
    # centroid terms: query block 0 has 3 skipped blocks, 2 has 2, 3 has 1 (dense block 1 none)
    for i, c in enumerate([3, 0, 2, 1]):
        sel["mult"][0, i, :c] = 60
    pairs, cent, frac = bench.selection_stats(sel, w, 1, 1)
    # exact keys per row: (kept * 64 + extra), extras ignored on the dense query block
    keys = [1 * 64 + 5, 4 * 64, 2 * 64 + 0, 3 * 64 + 1]
    assert pairs == 64 * sum(keys)
    assert cent == 64 * (3 + 0 + 2 + 1)
    assert abs(frac - (1 + 2 + 3) / (3 * M)) < 1e-12


def test_traffic_is_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    f.write_text(f"sources_sha256 (common.h, flash.hip, launch.h): `{bench.sources_digest()}`\n\n"
                 "traffic_bytes_per_launch: `123456`\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("sol-full-bf16-n64k") == 123456.0
    assert bench.measured_traffic("sol-long-bf16-n203k") is None
    f.write_text("sources_sha256 (common.h, flash.hip, launch.h): `0000000000000000`\n\n"
                 "traffic_bytes_per_launch: `123456`\n")
    assert bench.measured_traffic("sol-full-bf16-n64k") is None
