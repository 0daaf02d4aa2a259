"""Host logic of bench.py (CPU only): the one-GPU contract, the sources'
fingerprint and the recorded-traffic lookup, the attainable-peak choice and
the algorithmic work the roofline divides by, checked on the tiny workload
against counts written out by hand."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_defaults_are_the_driver_workload_and_the_separate_top_k():
    a = bench.parse_args([])
    assert a.workload == "70b-80layer-8req" and a.gpus == 1
    assert a.steps is None and a.warmup is None
    assert a.select_in_launch == 0 and a.graph == 0


def test_source_fingerprint_is_stable_and_printed():
    sha = bench.source_fingerprint()
    assert len(sha) == 64 and int(sha, 16) >= 0
    assert bench.source_fingerprint() == sha
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--print-source-sha"],
                         capture_output=True, text=True, timeout=120, check=True).stdout.strip()
    assert out == sha


def test_recorded_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("partial_attn", "w") is None          # no summary
    (tmp_path / "traffic_partial_attn_w.txt").write_text(
        "# comment: 1\nhbm_bytes_per_launch: 12345\nsource_sha256: "
        + bench.source_fingerprint() + "\n")
    assert bench.recorded_traffic("partial_attn", "w") == 12345.0
    (tmp_path / "traffic_partial_attn_w.txt").write_text(
        "hbm_bytes_per_launch: 12345\nsource_sha256: " + "0" * 64 + "\n")
    assert bench.recorded_traffic("partial_attn", "w") is None          # stale sources


def test_attainable_mfma_prefers_the_random_operand_figure():
    assert bench.mfma_attainable({"mfma_bf16_32x32x16_tflops": 2080.0,
                                  "mfma_bf16_32x32x16_random_tflops": 1760.0}) == 1760.0
    assert bench.mfma_attainable({"mfma_bf16_32x32x16_tflops": 2080.0}) == 2080.0


def test_algorithmic_work_of_the_tiny_layer():
    """tiny: one request of two 64-token chunks, 4 Q / 2 KV heads, head_dim
    16, fp32: a KV row is 2 * 16 * 4 = 128 bytes; the second chunk's 64
    tokens have delta 64; all 128 tokens are candidates, 20 are selected."""
    from types import SimpleNamespace

    from selective_recompute_amd import workloads as W
    wl = W.make_workload("tiny")
    runner = SimpleNamespace(batches=[SimpleNamespace(n_cand=128)])
    sel = np.sort(np.array([0, 5, 63, 64, 100, 127] + list(range(70, 84)), dtype=np.int64))
    assert len(sel) == 20
    (w,) = bench.algorithmic_work(wl, runner, [sel])
    row = 128
    assert w["rerotate"] == 2 * row * 64 + 4 * 128
    assert w["deviation_topk"] == 2 * row * 128 + 8 * 128
    assert w["fuse_scatter"] == 4 * row * 20 + 8 * 20
    kept_turned = 64 - int(np.count_nonzero(sel >= 64))   # rows with delta != 0 not in S
    assert w["rerotate_fuse"] == 2 * row * kept_turned + 4 * 128 + 4 * row * 20 + 8 * 20
    assert w["partial_attn"] == 4.0 * 16 * 4 * float(np.sum(sel + 1))
