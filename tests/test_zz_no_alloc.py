"""dgp_gemm_preshuffle_splitk_noalloc, through the C ABI: the split-K GEMM
whose fp32 partials go to the library's fixed per-GPU scratch gives the
same output, bit for bit, as dgp_gemm_preshuffle_splitk with a caller
workspace (same kernels, same summation order) -- on two calls in a row, the
second smaller than the first, so the second reads a scratch that still
holds the first call's partials.  Sizes past the scratch are refused with
nothing enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import dense_gemm_packer_amd as dgp
import synth
from gpu_common import DEV, dev_codes, dev_scales, dmode

pytestmark = pytest.mark.gpu


def _call_noalloc(a, Bs, out, M, N, K, dtype, mode, sA, sB, split_k):
    L = dgp.lib()
    ptr = lambda t: None if t is None else t.data_ptr()   # noqa: E731
    return L.dgp_gemm_preshuffle_splitk_noalloc(ptr(a), ptr(Bs), ptr(out), M, N, K, dtype, mode, ptr(sA),
                                                ptr(sB), split_k, None, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("name,dtype_s,big,small", [
    ("fp8_decode", "fp8", (16, 16384, 8), (5, 2048, 4)),
    ("fp8_blockscale", "fp8", (16, 16384, 4), (16, 2048, 2)),
    ("bf16_decode", "bf16", (16, 16384, 8), (1, 2048, 2)),
    ("fp4_mx32", "fp4", (16, 16384, 7), (3, 4096, 4)),
])
def test_noalloc_matches_workspace_entry_point(name, dtype_s, big, small):
    for M, N, split in (big, small):
        print(f"noalloc {name} M={M} N={N} split={split}", flush=True)
        w = synth.workload_inputs(name, M=16, N=N)
        mode = w["scale_mode"]
        a = dev_codes(w["A"][:M], dtype_s)
        Bs = dgp.preshuffle_b(dev_codes(w["B"], dtype_s))
        sA = None if w["sA"] is None else (w["sA"] if mode == "tensor" else w["sA"][:M])
        dA, dB = dev_scales(sA, mode), dev_scales(w["sB"], mode)
        K = w["K"]
        want = dgp.gemm_preshuffle_splitk(a, Bs, split, dA, dB, dmode(mode))
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        st = _call_noalloc(a, Bs, out, M, N, K, dgp.dtype_code(a), dmode(mode), dA, dB, split)
        assert st == 0, dgp.lib().dgp_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (name, M, N, split)
        # the binding's wrapper of the same entry point
        out2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        dgp.gemm_preshuffle_splitk_noalloc(a, Bs, split, out2, dA, dB, dmode(mode))
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), want.view(torch.int16)), (name, M, N, split)


def test_noalloc_refuses_sizes_past_the_scratch():
    M, N, K, split = 32, 16384, 7168, 14          # 28 MiB of partials > 16 MiB
    a = torch.zeros((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    Bs = torch.zeros((N, K), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.ones(1, device=DEV)
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    st = _call_noalloc(a, Bs, out, M, N, K, dgp.FP8_E4M3, dgp.SCALE_TENSOR, s, s, split)
    assert dgp.STATUS[st] == "DGP_ERR_WORKSPACE"
    assert "scratch" in dgp.lib().dgp_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0).item()
    # the largest accepted size: exactly the scratch (M = 32, N = 16384, split 8)
    M, split = 32, 8
    assert dgp.splitk_workspace_bytes(M, N, split) == dgp.NOALLOC_SCRATCH_BYTES
    w = synth.workload_inputs("fp8_decode", M=M, N=N)
    a = dev_codes(w["A"], "fp8")
    Bs = dgp.preshuffle_b(dev_codes(w["B"], "fp8"))
    dA, dB = dev_scales(w["sA"], "tensor"), dev_scales(w["sB"], "tensor")
    want = dgp.gemm_preshuffle_splitk(a, Bs, split, dA, dB, dgp.SCALE_TENSOR)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    assert _call_noalloc(a, Bs, out, M, N, 7168, dgp.FP8_E4M3, dgp.SCALE_TENSOR, dA, dB, split) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
