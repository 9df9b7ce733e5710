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


def test_kernel_rooflines_use_the_algorithmic_bytes():
    # pool against the hot-path table's bytes (read Q, K, V; write three fp32 means), with the
    # implementation's extra writes beside it; select against the score read plus its outputs
    w = workload(4)
    kern = {n: {"avg_ms": 1.0} for n in ("block_pool", "block_score", "block_select", "extra_select",
                                         "sparse_flash_fwd")}
    stats = {"exact_pairs": 10 ** 9}
    peaks = {"bf16_mfma_TFLOPs": 2000.0, "fp32_mfma_TFLOPs": 120.0, "copy_GBs": 5000.0}
    roof = bench.kernel_rooflines(w, kern, None, stats, False, peaks)
    BH, Mq, M, N, d = 24, 1024, 1024, 65536, 128
    alg = BH * (3 * N * d * 2 + (Mq + 2 * M) * d * 4)
    assert kern["block_pool"]["algorithmic_bytes"] == alg
    assert abs(kern["block_pool"]["frac"] - alg / 1e-3 / 1e9 / bench.PEAK_HBM_GBS) < 1e-4
    assert kern["block_pool"]["impl_bytes"] > alg
    assert kern["block_select"]["algorithmic_bytes"] == BH * Mq * (M * 4 + 8 + M // 8)
    assert abs(kern["block_pool"]["frac_measured"] - alg / 1e-3 / 1e9 / 5000.0) < 1e-4
    f = 4.0 * d * 10 ** 9
    assert roof["algorithmic_flop"] == f and roof["frac_measured_peak"] == round(f / 1e-3 / 1e12 / 2000.0, 4)


def test_selection_check_counts_flips():
    # one head, two sparse query blocks over M = 4 key blocks: one mask bit differs in block 0,
    # block 1's masks agree and its extra sets differ by one token each way
    w = workload(1, T=1, Hh=16, Ww=16, H=1, extra_tokens=2)
    M = w.N // 64
    assert M == 4
    kept_gpu = np.array([[1, 1, 0, 0], [0, 1, 0, 1], [0, 0, 1, 0], [0, 0, 0, 1]], dtype=bool)
    words = (kept_gpu * (1 << np.arange(4))).sum(axis=1).astype(np.int64)
    sel = {"kept_bm": words.reshape(1, 4, 1), "extra_cnt": np.array([[0, 2, 0, 0]]),
           "extra_idx": np.zeros((1, 4, 256), dtype=np.int32)}
    sel["extra_idx"][0, 1, :2] = [3, 130]
    ref = {"kept": kept_gpu.copy(), "extra": [np.array([], int), np.array([3, 140]), np.array([], int),
                                              np.array([], int)],
           "dense": np.array([False, False, True, True]), "scores": np.zeros((4, 4))}
    ref["kept"][0, 2] = True
    out = bench.selection_check(w, sel, {0: ref})
    assert out["rows"] == 2 and out["mask_flips"] == 1 and out["extra_flips"] == 2


def test_cpu_baseline_names_its_threads_and_blas():
    # the oracle leg on a tiny sample: the fields the bench line reports beside the time
    from gen import make_inputs
    w = workload(1)
    x = make_inputs(w, heads=[0])
    cb, refs = bench.cpu_baseline(w, x, heads=(0,), n_sparse=2, n_dense=0)
    assert cb["kind"] == "oracle" and cb["unit"] == "ms" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["host_cpus"] >= 1 and cb["blas"]
    assert 0 in refs and refs[0]["kept"].shape == (w.N // w.block_q, w.N // w.block_k)
