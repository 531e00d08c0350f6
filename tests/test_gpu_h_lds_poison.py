"""Parity on the LDS-poison debug build (libdgp_lds_poison.so).

The debug build fills each kernel's LDS with 0xFF bytes before its first
global -> LDS copy and overwrites every copy's destination with 0xFF until
the copy lands (include/dgp_diag.h, dgp_lds_poison).  A kernel that reads
LDS no copy filled -- a tile only partly loaded, a scale stage a copy skipped
-- or reads a stage before the wait for its copy then produces NaN (bf16,
e4m3, E8M0, fp32 bytes) or -6 (E2M1) where the release build may produce a
plausible value from stale LDS.  The cases are exact-integer inputs, so every
result is compared bit for bit with the oracle: every compiled kernel on a
ragged multi-tile grid, k-tile counts around the ring depths, the streaming
kernel's multi-panel K loop, and the built-in decode choices at every split."""
import numpy as np
import pytest

import dense_gemm_packer_amd as dgp
from gpu_common import run_gpu, run_oracle
from test_gpu_c_gemm import exact_inputs

pytestmark = pytest.mark.gpu

NAMES = {dgp.BF16: "bf16", dgp.FP8_E4M3: "fp8", dgp.FP4_E2M1: "fp4"}
MODES = {0: "none", 1: "tensor", 2: "block128", 3: "mx128", 4: "mx32"}


def test_every_compiled_kernel_bit_exact_on_poisoned_lds():
    count = 0
    with dgp.lds_poison_build() as P:
        assert P.dgp_lds_poison() == 1
        for cfg, dt, sm, split_out in dgp.kernels():
            dtype, mode = NAMES[dt], MODES[sm]
            if cfg.tile_m <= 16:
                M, N = (37 if cfg.tile_m == 16 else 3), 384
            else:
                M, N = 2 * cfg.tile_m + 44, 2 * cfg.tile_n + 128
            K = 1024 if dtype in ("fp8", "fp4") else 512
            split = 2 if split_out else 1
            what = (f"{dtype} {mode} tile {cfg.tile_m}x{cfg.tile_n} wm{cfg.waves_m} d{cfg.prefetch} "
                    f"s{cfg.schedule} l{cfg.a_layout} c{cfg.a_copy} split {split}")
            print(what, flush=True)
            A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 71)
            got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
            _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
            assert np.array_equal(got, c16), what
            count += 1
    assert count == len(dgp.kernels())


@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
def test_large_m_k_tile_counts_on_poisoned_lds(dtype, mode):
    """1, 2, 3, 4, 5 and 7 k-tiles: rings shorter than, equal to and wrapping
    past their stage count, so every stage is filled, read and refilled."""
    per_byte = {"bf16": 0.5, "fp8": 1, "fp4": 2}[dtype]
    with dgp.lds_poison_build():
        for cfg, dt, sm, so in dgp.kernels():
            if cfg.tile_m <= 16 or so or (NAMES[dt], MODES[sm]) != (dtype, mode):
                continue
            for tiles in (1, 2, 3, 4, 5, 7):
                K = int(tiles * 128 * per_byte)
                N = 640 if mode == "block128" else 528
                A, B, sA, sB = exact_inputs(dtype, mode, 300, N, K, 17)
                got = run_gpu(A, B, dtype, mode, sA, sB, config=cfg)
                _, c16 = run_oracle(A, B, dtype, mode, sA, sB)
                assert np.array_equal(got, c16), (tiles, cfg.tile_m, cfg.tile_n, cfg.schedule, cfg.a_layout)


@pytest.mark.parametrize("dtype,mode", [("fp8", "tensor"), ("fp8", "block128"), ("fp8", "mx128"),
                                        ("fp4", "mx32"), ("bf16", "none")])
def test_stream_panels_on_poisoned_lds(dtype, mode):
    """The streaming tile over several LDS panels of A per split: each panel
    after the first is copied into LDS the previous one occupied."""
    K = {"bf16": 12288, "fp8": 24576, "fp4": 40960}[dtype]
    with dgp.lds_poison_build():
        for split in (1, 2):
            A, B, sA, sB = exact_inputs(dtype, mode, 20, 256, K, 29)
            got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=dgp.Config(16, 64, 0, 0, 1, 0, 0))
            _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
            assert np.array_equal(got, c16), split


@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
@pytest.mark.parametrize("M", [1, 16])
def test_builtin_decode_choices_on_poisoned_lds(dtype, mode, M):
    """The built-in decode selection at splits 1, 2 and 4, N = 2048, K = 4096."""
    with dgp.lds_poison_build():
        A, B, sA, sB = exact_inputs(dtype, mode, M, 2048, 4096, 37)
        for split in (1, 2, 4):
            got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split)
            _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
            assert np.array_equal(got, c16), split
