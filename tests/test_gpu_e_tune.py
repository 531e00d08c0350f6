"""The kernel sweep tool on the device: every compiled kernel that accepts
the shape is timed, the built-in selection is among them, and the reported
ratio is consistent with the timings."""
import pytest

from dense_gemm_packer_amd import tune

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("spec", ["bf16:512x512x512", "fp8:16x2048x7168:4"])
def test_sweep_reports_every_accepting_kernel(spec):
    r = tune.sweep(spec, iters=4)
    names = [k["kernel"] for k in r["kernels"]]
    assert names and len(names) == len(set(names))
    assert r["builtin_choice"] in names
    times = [k["us"] for k in r["kernels"]]
    assert times == sorted(times) and all(t > 0 for t in times)
    assert r["builtin_time_over_fastest"] >= 1.0
    assert r["cold"] == (r["M"] <= 32)
