"""Special values through every compiled kernel, against the oracle.

Exact-integer inputs (every partial sum exact, so any summation order gives
the same fp32 value) with special element codes planted at chosen places:

* NaN codes (bf16 0x7FC0 / 0xFFC0, e4m3fn 0x7F / 0xFF) in A and in B: the
  whole row (column) of C is NaN;
* bf16 +inf / -inf in A and B: the row (column) is +-inf where the other
  factor is non-zero, NaN where it is zero, and NaN where infinities of both
  signs meet;
* sums that overflow bf16 while exact in fp32: (2 - 2^-8) * 2^127 rounds to
  +-inf, on the bf16 path through the products and on the fp8 paths through
  per-tensor, blockscale and E8M0 scales that are exact powers of two.

Each outcome (NaN, +-inf or the exact finite value) does not depend on the
order of the additions, so the GPU result must equal the oracle's bf16
result entry for entry: the same NaN positions and bit-identical
everything else.  Every kernel of the compiled table runs, selected through
its own configuration (split-output kernels with split_k = 2)."""
import numpy as np
import pytest

import dense_gemm_packer_amd as dgp
from gpu_common import run_gpu, run_oracle
from test_gpu_c_gemm import exact_inputs

pytestmark = pytest.mark.gpu

MODES = {(dgp.BF16, dgp.SCALE_NONE): ("bf16", "none"), (dgp.FP8_E4M3, dgp.SCALE_TENSOR): ("fp8", "tensor"),
         (dgp.FP8_E4M3, dgp.SCALE_BLOCK128): ("fp8", "block128"), (dgp.FP8_E4M3, dgp.SCALE_MX128): ("fp8", "mx128")}


def kernels_of(dtype, mode):
    for cfg, dt, sm, split_out in dgp.kernels():
        if MODES.get((dt, sm)) == (dtype, mode):
            yield cfg, split_out


def shape_of(cfg, mode):
    if cfg.tile_m == 16:
        M, N = 37, 384
    else:
        M, N = 2 * cfg.tile_m + 44, 2 * cfg.tile_n + 128
    if mode == "block128" and N % 128:
        N += 128 - N % 128
    return M, N


def same_result(got, want, what):
    g = (got.astype(np.uint32) << 16).view(np.float32)
    w = (want.astype(np.uint32) << 16).view(np.float32)
    nan_g, nan_w = np.isnan(g), np.isnan(w)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ ({nan_g.sum()} vs {nan_w.sum()})"
    assert np.array_equal(got[~nan_w], want[~nan_w]), f"{what}: non-NaN entries differ"


def plant_specials(dtype, A, B, seed):
    """NaN and (bf16) infinity codes at fixed rows/columns and K positions."""
    rng = np.random.default_rng(seed)
    M, K = A.shape
    N = B.shape[0]
    ks = rng.choice(K, size=6, replace=False)
    if dtype == "bf16":
        A[1, ks[0]] = 0x7FC0          # NaN
        B[5, ks[1]] = 0xFFC0          # -NaN
        A[M - 2, ks[2]] = 0x7F80      # +inf
        B[N - 3, ks[3]] = 0xFF80      # -inf
        A[M - 2, ks[4]] = 0xFF80      # -inf in the same row: +inf and -inf meet where both factors are non-zero
        B[7, ks[5]] = 0x7F80
    else:
        A[1, ks[0]] = 0x7F            # e4m3fn NaN (no infinities in the format)
        B[5, ks[1]] = 0xFF
        A[M - 2, ks[2]] = 0xFF
        B[N - 3, ks[3]] = 0x7F
    return A, B


@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"), ("fp8", "mx128")])
def test_nan_and_inf_codes_every_kernel(dtype, mode):
    count = 0
    for cfg, split_out in kernels_of(dtype, mode):
        M, N = shape_of(cfg, mode)
        K = 512 if dtype == "bf16" else 1024
        split = 2 if split_out else 1
        A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 41)
        A, B = plant_specials(dtype, A.copy(), B.copy(), 43)
        got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
        _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
        what = f"{dtype} {mode} tile {cfg.tile_m}x{cfg.tile_n} wm{cfg.waves_m} s{cfg.schedule} l{cfg.a_layout} split {split}"
        c32w = (c16.astype(np.uint32) << 16).view(np.float32)
        assert np.isnan(c32w[1]).all() and np.isnan(c32w[:, 5]).all()   # the planted NaNs reach the oracle
        same_result(got, c16, what)
        count += 1
    assert count > 0


def overflow_inputs(dtype, mode, M, N, K, seed):
    """Exact-integer inputs plus row 2 (+) and row 3 (-) against column 9
    summing to (2 - 2^-8) * 2^127 in magnitude: exact in fp32, +-inf in bf16."""
    A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, seed)
    A, B = A.copy(), B.copy()
    ks = np.arange(9) * (K // 9)
    A[2, :] = 0
    A[3, :] = 0
    B[9, :] = 0
    if dtype == "bf16":
        # A = +-2^63, B = 2^64 .. 2^56: products 2^127 .. 2^119
        A[2, ks] = 0x5F00                                  # 2^63
        A[3, ks] = 0xDF00                                  # -2^63
        B[9, ks] = [(127 + 64 - i) << 7 for i in range(9)]  # 2^(64-i)
        return A, B, sA, sB
    # e4m3: A = +-16, B = 2^8 .. 2^0: products 2^12 .. 2^4, sum (2 - 2^-8) * 2^12;
    # the scales bring it to (2 - 2^-8) * 2^127 exactly
    A[2, ks] = 0x58                                        # 16 = 2^4
    A[3, ks] = 0xD8
    B[9, ks] = [(7 + 8 - i) << 3 for i in range(9)]        # 2^(8-i)
    if mode == "tensor":
        sA, sB = np.array([2.0 ** 60], np.float32), np.array([2.0 ** 55], np.float32)
    elif mode == "block128":
        sA = np.full((M, K // 128), 2.0 ** 57, np.float32)
        sB = np.full((N // 128, K // 128), 2.0 ** 58, np.float32)
    else:   # mx128: E8M0 bytes 127 + e
        sA = np.full((M, K // 128), 127 + 57, np.uint8)
        sB = np.full((N, K // 128), 127 + 58, np.uint8)
    return A, B, sA, sB


@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"), ("fp8", "mx128")])
def test_bf16_overflow_every_kernel(dtype, mode):
    for cfg, split_out in kernels_of(dtype, mode):
        M, N = shape_of(cfg, mode)
        K = 1152 if dtype == "fp8" else 576            # 9 K blocks of 128 (fp8) / 9 x 64 (bf16)
        split = (3 if dtype == "fp8" else 9) if split_out else 1   # K ranges of whole 128-byte steps
        A, B, sA, sB = overflow_inputs(dtype, mode, M, N, K, 47)
        got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
        c32, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
        assert c16[2, 9] == 0x7F80 and c16[3, 9] == 0xFF80          # +-inf in bf16 ...
        assert np.isfinite(c32[2, 9]) and c32[2, 9] > 0            # ... from a finite fp32 sum
        same_result(got, c16, f"{dtype} {mode} tile {cfg.tile_m}x{cfg.tile_n} wm{cfg.waves_m} s{cfg.schedule} split {split}")
