"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic FLOP and byte counts behind the roofline, and the guard that keeps
stale HBM counters out of the report."""
import json
import os
import shutil
import subprocess
import sys

import numpy as np

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_dense_counts_match_the_operand_sizes():
    wl = workloads.dense(64, 300, 1536, seed=0)
    flops, nbytes, rows = bench.algorithmic_counts(wl)
    KB = 1536 // 128
    assert rows == 64 and flops == 2.0 * 64 * 300 * 1536
    # codes of X and W, FP32 scales (1x128 of X, 128x128 blocks of W, ragged N), BF16 Y
    expect = 64 * 1536 + 4 * 64 * KB + 300 * 1536 + 4 * 3 * KB + 2 * 64 * 300
    assert nbytes == expect


def test_grouped_counts_take_valid_rows_and_used_experts_only():
    wl = workloads.masked(4, 256, 256, 256, seed=0)
    valid = np.clip(np.asarray(wl.masked_m), 0, 256)
    flops, nbytes, rows = bench.algorithmic_counts(wl)
    assert rows == int(valid.sum())
    assert flops == 2.0 * rows * 256 * 256
    used = int((valid > 0).sum())
    expect = rows * 256 + 4 * rows * 2 + used * 256 * 256 + 4 * used * 2 * 2 + 2 * rows * 256
    assert nbytes == expect
    wl = workloads.contiguous(4, 512, 256, 256, seed=1)
    counts = np.bincount(wl.m_indices[wl.m_indices >= 0], minlength=4)
    flops, nbytes, rows = bench.algorithmic_counts(wl)
    assert rows == int(counts.sum()) == 512


def test_mx_counts():
    wl = workloads.dense(32, 256, 512, seed=0)
    f8 = bench.algorithmic_counts_mx(wl, w4=False)
    f4 = bench.algorithmic_counts_mx(wl, w4=True)
    assert f8[0] == f4[0] == 2.0 * 32 * 256 * 512
    assert f8[1] - f4[1] == 256 * 512 / 2          # E2M1 weights: half a byte per element


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "fine_grained_block_e4m3_amd", "csrc")
    dst = tmp_path / "fine_grained_block_e4m3_amd" / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_sha()
    name = sorted(p for p in os.listdir(dst) if p.endswith(".h"))[0]
    text = (dst / name).read_text()
    (dst / name).write_text("// a comment\n/* and a\n   block comment */\n" + text + "\n\n")
    assert bench.kernel_source_sha() == base
    (dst / name).write_text(text + "\nstatic const int kBenchHashProbe = 1;\n")
    assert bench.kernel_source_sha() != base


def test_stale_counters_are_not_reported(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    entry = {"source_sha": "abc", "hbm_bytes_per_dispatch": 123.0, "clock_mhz_grbm": 2000.0,
             "mfma_busy_frac": 0.5}
    (tmp_path / "profiles" / "counters.json").write_text(json.dumps({"gemm_exact_cfg2": entry}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_counters("gemm_exact_cfg2", "abc")["hbm_bytes_per_dispatch"] == 123.0
    assert bench.load_counters("gemm_exact_cfg2", "def") is None
    assert bench.load_counters("gemm_exact_cfg9", "abc") is None
    r = bench.roofline(1e12, 1e9, 1e-3, "f16", True, bench.load_counters("gemm_exact_cfg2", "abc"))
    assert r["bound"] == "mfma" and r["peak"] == 2500.0 and abs(r["frac"] - 1000 / 2500) < 1e-12
    assert r["frac_of_fp8_peak"] == r["achieved"] / 5000.0
    assert r["traffic"] == 123.0 and r["traffic_ratio"] == 123.0 / 1e9 and r["clock_mhz_counters"] == 2000.0
    r = bench.roofline(1e12, 1e9, 1e-3, "fp8", False, None)
    assert r["bound"] == "hbm" and r["traffic"] is None and abs(r["frac"] - 1000 / 8000) < 1e-12


def test_stats_and_cpu_model():
    s = bench.stats([3.0, 1.0, 2.0, 10.0])
    assert s == {"mean": 4.0, "median": 2.5, "min": 1.0, "n": 4}
    assert bench._cpu_model().get("model name") is not None


def test_cpu_baseline_splits_quantization_and_gemm():
    wl = workloads.dense(64, 256, 512, seed=0)
    r = bench.cpu_baseline(wl, 0.2)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["nproc"] >= 1
    assert r["quant_seconds"] > 0 and r["gemm_seconds"] > 0
    assert r["one_thread"]["gemm_seconds"] > 0 and "1 thread" in r["one_thread"]["sample"]
    import oracle
    assert oracle.num_threads() == r["cores"]          # the thread count is restored
