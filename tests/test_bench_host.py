"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
guard that drops a counter-based traffic figure taken on other kernel
source."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_figure_needs_the_recorded_kernel_source(tmp_path):
    good = tmp_path / "good.md"
    good.write_text(f"- source_sha256: {bench.kernel_source_sha()}\n"
                    "- fetch_bytes_per_launch: 1000\n- write_bytes_per_launch: 24\n")
    assert bench.read_traffic(str(good)) == 1024.0
    stale = tmp_path / "stale.md"
    stale.write_text("- source_sha256: 0000000000000000\n"
                     "- fetch_bytes_per_launch: 1000\n- write_bytes_per_launch: 24\n")
    assert bench.read_traffic(str(stale)) is None
    assert bench.read_traffic(str(tmp_path / "missing.md")) is None



def test_launch_stats_median_min_p90():
    import numpy as np
    st = bench.launch_stats(np, [0.2, 0.1, 0.3, 0.5, 0.4])   # ms
    assert st == {"n": 5, "median": 300.0, "min": 100.0, "p90": 460.0, "mean": 300.0}


def test_summary_keeps_the_secondary_headline_figures():
    sec = {"fp8_gemm_4096x4096x8192": {"us": 100.0, "TFLOP/s": 2748.8, "frac_of_peak": 0.55},
           "bf16_gemm_128x256x256": {"us": 5.0, "launch_us": {"min": 4.8, "p90": 5.3}},
           "decode_cold_cache": {"best tensor M=16 N=16384": {"split": 1, "GB/s": 6000.0, "frac_hbm": 0.75,
                                                              "frac_measured_wall": 0.9},
                                 "tensor M=16 N=16384 K=7168 split=2": {"us": 30.0}},
           "vendor_library_same_process": {"bf16_4096x4096x8192_TFLOP/s": 1300.0}}
    s = bench.summarize(sec)
    assert s["fp8 tensor 4096x4096x8192"]["us_median"] == 100.0
    assert s["bf16 128x256x256"] == {"us_median": 5.0, "us_min": 4.8, "us_p90": 5.3}
    assert s["decode cold tensor M=16 N=16384"]["GB/s"] == 6000.0
    assert not any("split=2" in k for k in s)
    assert s["context: vendor library, same process"] == {"bf16_4096x4096x8192_TFLOP/s": 1300.0}
