"""Parity at the full workload sizes, in the launch configuration the
benchmark times: the library's built-in kernel selection and every split
count it reports, on the benchmark's own seeded inputs.  The oracle computes
rows of C one by one (all N columns of each; every row where the oracle finishes in seconds); random data must be
within 1e-2 * max|C_ref| of the oracle's fp32 value at the same split count."""
import numpy as np
import pytest
import torch

import dense_gemm_packer_amd as dgp
import synth
from gpu_common import DEV, assert_close, dev_codes, dev_scales, dmode, host_bits, run_oracle

pytestmark = pytest.mark.gpu


def _scales(w, rows):
    """The workload's scales for its first `rows` rows of A (per-tensor: as is)."""
    if w["sA"] is None:
        return None, None
    sA = w["sA"] if w["scale_mode"] == "tensor" else w["sA"][:rows]
    return sA, w["sB"]


@pytest.mark.parametrize("name", ["bf16_large", "fp8_large"])
def test_large_workload_every_row(name):
    """The two 4096 x 4096 x 8192 GEMMs the benchmark headlines, all 4096
    rows of C against the oracle (about 4 s of oracle on 16 threads each)."""
    w = synth.workload_inputs(name)
    dt, mode, M = w["dtype"], w["scale_mode"], w["M"]
    A = dev_codes(w["A"], dt)
    Bs = dgp.preshuffle_b(dev_codes(w["B"], dt))
    sA, sB = _scales(w, M)
    C = dgp.gemm_preshuffle(A, Bs, dev_scales(sA, mode), dev_scales(sB, mode), dmode(mode))
    torch.cuda.synchronize()
    c32, _ = run_oracle(w["A"], w["B"], dt, mode, w["sA"], w["sB"])
    assert_close(host_bits(C), c32, what=name)


@pytest.mark.parametrize("name", ["fp8_blockscale", "fp8_mx128", "fp4_mx32"])
def test_large_workload_sampled_rows(name):
    """4096 x 4096 x 8192 blockscale, mxfp8 and mxfp4 (at the size of the
    fp8 GEMM, as the benchmark times them): rows on both sides of every
    256-row tile boundary the sample crosses, plus evenly spaced rows."""
    w = synth.workload_inputs(name, M=4096, N=4096, K=8192)
    dt, mode, M = w["dtype"], w["scale_mode"], w["M"]
    A = dev_codes(w["A"], dt)
    Bs = dgp.preshuffle_b(dev_codes(w["B"], dt))
    sA, sB = _scales(w, M)
    C = dgp.gemm_preshuffle(A, Bs, dev_scales(sA, mode), dev_scales(sB, mode), dmode(mode))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.linspace(0, M - 1, 24).astype(np.int64),
                                     np.array([255, 256, 2047, 2048, M - 1])]))
    c32, _ = run_oracle(w["A"], w["B"], dt, mode, w["sA"], w["sB"], rows=rows)
    assert_close(host_bits(C)[rows], c32, what=name)


@pytest.mark.parametrize("M", [4096, 16])
def test_blockscale_full_size_fused_accumulate_bit_exact(M):
    """The blockscale shapes the benchmark times (4096 x 4096 x 8192 and the
    M = 16 decode at N = 16384, K = 7168) through the built-in selection, on
    exact-integer operands with random fp32 block scales: every scaled
    accumulate rounds, so sampled rows must match the oracle bit for bit
    (same fused multiply-add, same K order; the decode tile's wave slices
    against the oracle's split-K over as many ranges)."""
    N, K = (4096, 8192) if M == 4096 else (16384, 7168)
    A = synth.exact_ints((M, K), 91, "fp8")
    B = synth.exact_ints((N, K), 92, "fp8")
    sA = synth.random_block_scales((M, K // 128), 93)
    sB = synth.random_block_scales((N // 128, K // 128), 94)
    a = dev_codes(A, "fp8")
    Bs = dgp.preshuffle_b(dev_codes(B, "fp8"))
    C = dgp.gemm_preshuffle(a, Bs, dev_scales(sA, "block128"), dev_scales(sB, "block128"), dgp.SCALE_BLOCK128)
    torch.cuda.synchronize()
    cfg, _, _, _ = dgp.kernels()[dgp.select_kernel(M, N, K, dgp.FP8_E4M3, dgp.SCALE_BLOCK128)]
    ksplit = cfg.tile_m == 16 and (cfg.tile_n in (8, 16) or cfg.waves_m in (8, 16))
    if ksplit:   # the oracle's split-K over the waves' slices: equal whole 128-K blocks
        assert (K // 128) % cfg.waves_m == 0
    rows = np.arange(M) if M <= 16 else np.unique(np.concatenate([np.linspace(0, M - 1, 24).astype(np.int64),
                                                                     np.array([255, 256, 2047, 2048])]))
    _, c16 = run_oracle(A, B, "fp8", "block128", sA, sB, split_k=cfg.waves_m if ksplit else 1, rows=rows)
    assert np.array_equal(host_bits(C)[rows], c16)


DECODE = [("fp8_decode", 2048), ("fp8_decode", 16384), ("bf16_decode", 2048), ("bf16_decode", 16384),
          ("fp4_mx32", 2048), ("fp4_mx32", 16384), ("fp8_blockscale", 16384), ("fp8_mx128", 16384)]


@pytest.mark.parametrize("name,N", DECODE)
def test_decode_workload_every_split(name, N):
    """Decode sizes (K = 7168): M = 1 and 16 where the benchmark times both,
    every split count of the workload, every row of C."""
    w = synth.workload_inputs(name, M=16, N=N)
    dt, mode = w["dtype"], w["scale_mode"]
    Bs = dgp.preshuffle_b(dev_codes(w["B"], dt))
    Ms = (1, 16) if name in ("fp8_decode", "bf16_decode", "fp4_mx32") else (16,)
    for M in Ms:
        A = dev_codes(w["A"][:M], dt)
        sA, sB = _scales(w, M)
        dA, dB = dev_scales(sA, mode), dev_scales(sB, mode)
        rows = np.arange(M)
        for split in synth.WORKLOADS[name]["splits"]:
            C = dgp.gemm_preshuffle_splitk(A, Bs, split, dA, dB, dmode(mode))
            torch.cuda.synchronize()
            c32, _ = run_oracle(w["A"][:M], w["B"], dt, mode, sA, sB, split_k=split, rows=rows)
            assert_close(host_bits(C)[rows], c32, what=f"{name} M={M} N={N} split={split}")
