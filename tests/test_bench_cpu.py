"""Host logic of bench.py, on the CPU: the one-GPU guard, the work and peak
tables behind `value` and `roofline`, the spread statistics and the lookup of
the committed traffic summary."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_counts_of_the_workloads():
    w = bench.WORKLOADS["hunyuan"]
    # MLP delta: two products of 2*n*d*k each; attention delta: s = Q K_S^T and
    # P V_S, 2*n*kk*128 each per head.
    assert bench.flops_mlp(w) == 4.0 * 118800 * 3072 * 860
    assert bench.flops_attn(w) == 4.0 * 118800 * 8316 * 128 * 24
    assert bench.flops_attn(w, reident=True) == 2 * bench.flops_attn(w)
    amount, bound = bench.kernel_work("sparse_step_fused", w)
    assert bound == "mfma" and amount == 2.0 * 118800 * 860 * 3072 + bench.flops_attn(w)
    amount, bound = bench.kernel_work("mlp_gemm1_sparse", w, fp8=True)
    assert bound == "mfma_fp8" and amount == 2.0 * 118800 * 3072 * 860


def test_topk_work_counts_only_launches_in_the_step():
    w = bench.WORKLOADS["flux"]
    nb = (w["n"] + 127) // 128
    assert bench.kernel_work("topk_rows", w) == (None, None)
    mlp = nb * w["h"] * 4 + nb * w["k"] * 4
    att = w["heads"] * nb * w["n"] * 4 + w["heads"] * nb * w["kk"] * 4
    assert bench.kernel_work("topk_rows", w, rescore=True) == (float(mlp), "hbm")
    assert bench.kernel_work("topk_rows", w, reident=True) == (float(att), "hbm")
    assert bench.kernel_work("topk_rows", w, reident=True, rescore=True) == ((mlp + att) / 2.0, "hbm")


def test_mixed_peak_is_the_harmonic_combination():
    assert bench.peak_for("mfma", 1.0) == bench.PEAK_BF16_TFLOPS
    assert bench.peak_for("mfma_fp8", 1.0) == bench.PEAK_FP8_TFLOPS
    # half the flops at each rate: total / (f/2/fp8 + f/2/bf16)
    f = 1e12
    expect = f / (f / 2 / bench.PEAK_FP8_TFLOPS + f / 2 / bench.PEAK_BF16_TFLOPS)
    assert bench.peak_for(("mfma_mix", f / 2), f) == pytest.approx(expect)
    assert bench.PEAK_BF16_TFLOPS < bench.peak_for(("mfma_mix", f / 2), f) < bench.PEAK_FP8_TFLOPS


def test_spread_statistics():
    vals = list(np.arange(1.0, 11.0))          # 1 .. 10
    st = bench.stats_ms(vals)
    assert st["count"] == 10 and st["median"] == 5.5 and st["mean"] == 5.5
    assert st["p10"] == pytest.approx(1.9) and st["p90"] == pytest.approx(9.1)
    assert bench.stats_ms([]) is None


def test_traffic_lookup_follows_the_source_digest(tmp_path, monkeypatch):
    digest = bench.source_digest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_tiny.md").write_text(
        "| Kernel | Source digest | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled bytes per launch | part of |\n"
        "|---|---|---:|---:|---:|---|\n"
        f"| sparse_step_fused | {digest} | 10 | 5 | 12345 | sparse step |\n"
        "| mlp_gemm1_sparse | 0000000000000000 | 10 | 5 | 999 | sparse step |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("sparse_step_fused", "tiny") == 12345
    assert bench.traffic_for("mlp_gemm1_sparse", "tiny") is None      # taken on other sources
    assert bench.traffic_for("attn_dense", "tiny") is None            # no row
    assert bench.traffic_for("sparse_step_fused", "flux_2304") is None  # no such file here


def test_committed_traffic_rows_name_their_digest():
    # Every row of the committed summaries carries a 16-hex-digit source digest.
    for wl in ("hunyuan", "flux"):
        path = os.path.join(ROOT, "profiles", f"traffic_{wl}.md")
        rows = [l for l in open(path) if l.startswith("| ") and "Source digest" not in l and "---" not in l]
        assert rows, wl
        for l in rows:
            cells = [c.strip() for c in l.strip().strip("|").split("|")]
            assert len(cells[1]) == 16 and int(cells[1], 16) >= 0
            assert int(float(cells[4])) > 0
