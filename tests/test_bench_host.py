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

