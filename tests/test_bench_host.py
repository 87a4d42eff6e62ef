"""Host-side logic of bench.py (no GPU): roofline pricing, the source hash that
ties committed counter summaries to the kernel sources, the traffic record
lookup, and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_hbm_stage_is_priced_against_8_tb_per_s():
    r = bench.roof_entry(1.0, "hbm", 2e9)  # 2 GB in 1 ms
    assert r["bound"] == "hbm" and r["GB/s"] == 2000.0 and r["frac"] == 0.25


def test_gemm_above_the_ridge_is_mfma_bound():
    flops = 0.5 * bench.PEAK_BF16_TFLOPS * 1e12 * 1e-3  # half of peak for 1 ms
    r = bench.roof_entry(1.0, "gemm", (flops, flops / 1000.0))  # 1000 flop/byte
    assert r["bound"] == "mfma" and r["frac"] == 0.5 and r["mfma_frac"] == 0.5


def test_gemm_below_the_ridge_is_hbm_bound():
    nbytes = 4e9  # 4 GB in 1 ms: half of the HBM peak
    r = bench.roof_entry(1.0, "gemm", (100.0 * nbytes, nbytes))  # 100 flop/byte
    assert r["bound"] == "hbm" and r["frac"] == 0.5


def test_ridge_point_is_about_315_flop_per_byte():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert 314 < ridge < 316


def test_source_hash_ignores_comments_but_not_code(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f() {\n  return 1;  // one\n}\n")
    h = bench.source_hash(str(a))
    a.write_text("// header comment\nint f() {\n\n  return 1;  // a different comment\n}\n")
    assert bench.source_hash(str(a)) == h
    a.write_text("int f() {\n  return 2;\n}\n")
    assert bench.source_hash(str(a)) != h


def test_traffic_record_needs_a_matching_hash(tmp_path, monkeypatch):
    csrc = tmp_path / "combine_top_router_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.GEMM_SOURCES:
        (csrc / f).write_text(f"int {f.split('.')[0]}_x = 1;\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.gemm_source_hash()
    md = tmp_path / "profiles" / "gate_up_w_counters.md"
    md.write_text(f"- source_sha256_16: `{sha}`\n- hbm_bytes_per_launch: `1.5e+09`\n")
    assert bench.traffic_record("gate_up", "w") == 1.5e9
    assert bench.traffic_record("gate_up", "other") is None  # no summary for it
    (csrc / bench.GEMM_SOURCES[-1]).write_text("int changed = 2;\n")
    assert bench.traffic_record("gate_up", "w") is None  # taken on other code


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr
