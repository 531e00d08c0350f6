"""Seeded random shapes through the built-in kernel selection: every element
type and scale mode, decode-sized and large M, N any multiple of 16 the mode
allows, K any valid length, every valid split count up to 8.  Exact-integer
inputs, so C must equal the oracle's bit for bit whatever the kernel, tile
or split the library picks."""
import numpy as np
import pytest

import synth
from gpu_common import run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MODES = [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"), ("fp8", "mx128"), ("fp4", "mx32")]
K_UNIT = {"bf16": 64, "fp8": 128, "fp4": 256}   # elements per 128 row bytes


def exact(dtype, mode, M, N, K, seed):
    A = synth.exact_ints((M, K), seed, dtype)
    B = synth.exact_ints((N, K), seed + 1, dtype)
    if mode == "none":
        return A, B, None, None
    if mode == "tensor":
        return A, B, np.array([0.125], np.float32), np.array([1.0], np.float32)
    if mode == "mx128":
        return A, B, synth.exact_e8m0_scales((M, K // 128), seed + 2), synth.exact_e8m0_scales((N, K // 128), seed + 3)
    if mode == "mx32":
        return A, B, synth.exact_e8m0_scales((M, K // 32), seed + 2), synth.exact_e8m0_scales((N, K // 32), seed + 3)
    return A, B, synth.exact_block_scales((M, K // 128), seed + 2), synth.exact_block_scales((N // 128, K // 128), seed + 3)


def valid_splits(dtype, mode, K):
    row_bytes = K * {"bf16": 2, "fp8": 1, "fp4": 0.5}[dtype]
    out = []
    for s in range(1, 9):
        if K % s or (row_bytes / s) % 128:
            continue
        if mode in ("block128", "mx128") and (K // s) % 128:
            continue
        out.append(s)
    return out


def draw(rng):
    dtype, mode = MODES[rng.integers(len(MODES))]
    decode = rng.random() < 0.6
    M = int(rng.integers(1, 33)) if decode else int(rng.integers(33, 400))
    # decode-sized M reaches all three decode tile bands (N * split_k up to ~76000)
    nmax = 600 if decode else 70
    N = 128 * int(rng.integers(1, nmax // 8 + 1)) if mode == "block128" else 16 * int(rng.integers(1, nmax))
    K = K_UNIT[dtype] * int(rng.integers(1, 17))
    splits = valid_splits(dtype, mode, K)
    split = splits[int(rng.integers(len(splits)))]
    return dtype, mode, M, N, K, split


@pytest.mark.parametrize("block", range(4))
def test_random_shapes_bit_exact(block):
    rng = np.random.Generator(np.random.PCG64(9100 + block))
    for case in range(15):
        dtype, mode, M, N, K, split = draw(rng)
        seed = 9100 + 100 * block + 2 * case
        A, B, sA, sB = exact(dtype, mode, M, N, K, seed)
        got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split)
        _, want = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
        assert np.array_equal(got, want), (dtype, mode, M, N, K, split)
