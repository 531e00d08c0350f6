"""GEMM parity on the device against the oracle, element by element.

Shapes span several tiles and ragged tails (M and N not multiples of the
tile), every compiled kernel configuration is forced at least once, and the
degenerate cases (M = 1, K = 0, empty) are covered.  The bar: exact-integer
inputs are bit-exact; random inputs satisfy max|C - C_ref| <= 1e-2*max|C_ref|
with C_ref the oracle's fp32 value before rounding."""
import numpy as np
import pytest
import torch

import dense_gemm_packer_amd as dgp
import oracle
import synth
from gpu_common import (DEV, assert_close, dev_codes, dev_f32, dev_scales, dmode, host_bits, run_gpu,
                        run_oracle)

pytestmark = pytest.mark.gpu

TILED = [(256, 256, 1, 8), (256, 256, 2, 8), (128, 256, 1, 8), (128, 128, 2, 4)]


def rand_inputs(dtype, mode, M, N, K, seed):
    if dtype == "fp4":
        A, sA = synth.fp4_mx32(M, K, seed, seed + 2)
        B, sB = synth.fp4_mx32(N, K, seed + 1, seed + 3)
        return A, B, sA, sB
    if dtype == "bf16":
        return synth.bf16_uniform((M, K), seed), synth.bf16_uniform((N, K), seed + 1), None, None
    if mode == "tensor":
        A, sA = synth.fp8_per_tensor((M, K), seed)
        B, sB = synth.fp8_per_tensor((N, K), seed + 1)
        return A, B, sA, sB
    if mode == "mx128":
        A, sA = synth.fp8_mx128(M, K, seed, seed + 2)
        B, sB = synth.fp8_mx128(N, K, seed + 1, seed + 3)
        return A, B, sA, sB
    A, sA = synth.fp8_blockscale_a(M, K, seed, seed + 2)
    B, sB = synth.fp8_blockscale_b(N, K, seed + 1, seed + 3)
    return A, B, sA, sB


def exact_inputs(dtype, mode, M, N, K, seed):
    A = synth.exact_ints((M, K), seed, dtype)
    B = synth.exact_ints((N, K), seed + 1, dtype)
    if mode == "none":
        return A, B, None, None
    if mode == "tensor":
        return A, B, np.array([0.125], np.float32), np.array([1.0], np.float32)
    if mode == "mx128":
        return (A, B, synth.exact_e8m0_scales((M, K // 128), seed + 2),
                synth.exact_e8m0_scales((N, K // 128), seed + 3))
    if mode == "mx32":
        return (A, B, synth.exact_e8m0_scales((M, K // 32), seed + 2),
                synth.exact_e8m0_scales((N, K // 32), seed + 3))
    return (A, B, synth.exact_block_scales((M, K // 128), seed + 2),
            synth.exact_block_scales((N // 128, K // 128), seed + 3))


CASES = [  # dtype, mode, M, N, K
    ("bf16", "none", 128, 256, 256),
    ("bf16", "none", 300, 272, 512),
    ("bf16", "none", 1, 64, 128),
    ("bf16", "none", 16, 528, 1024),
    ("bf16", "none", 40, 144, 384),
    ("bf16", "none", 1030, 1040, 640),
    ("fp8", "tensor", 128, 256, 256),
    ("fp8", "tensor", 300, 272, 1024),
    ("fp8", "tensor", 1, 2048, 896),
    ("fp8", "tensor", 16, 528, 1024),
    ("fp8", "tensor", 1030, 1040, 1280),
    ("fp8", "block128", 16, 256, 1024),
    ("fp8", "block128", 1, 384, 512),
    ("fp8", "block128", 33, 128, 768),
    ("fp8", "block128", 300, 384, 640),
    ("fp8", "block128", 1030, 1152, 1280),
    ("fp8", "mx128", 16, 256, 1024),
    ("fp8", "mx128", 1, 2048, 896),
    ("fp8", "mx128", 37, 144, 768),
    ("fp8", "mx128", 300, 272, 512),
    ("fp8", "mx128", 1030, 1040, 1280),
    ("fp4", "mx32", 16, 256, 1024),
    ("fp4", "mx32", 1, 2048, 768),
    ("fp4", "mx32", 37, 144, 512),
    ("fp4", "mx32", 300, 272, 256),
    ("fp4", "mx32", 1030, 1040, 1280),
]


@pytest.mark.parametrize("dtype,mode,M,N,K", CASES)
def test_random_within_tolerance(dtype, mode, M, N, K):
    A, B, sA, sB = rand_inputs(dtype, mode, M, N, K, 7 + M)
    got = run_gpu(A, B, dtype, mode, sA, sB)
    c32, _ = run_oracle(A, B, dtype, mode, sA, sB)
    assert_close(got, c32, what=f"{dtype} {mode} {M}x{N}x{K}")


@pytest.mark.parametrize("dtype,mode,M,N,K", CASES)
def test_exact_integers_bit_exact(dtype, mode, M, N, K):
    A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 11 + N)
    got = run_gpu(A, B, dtype, mode, sA, sB)
    _, c16 = run_oracle(A, B, dtype, mode, sA, sB)
    assert np.array_equal(got, c16)


def test_every_compiled_kernel():
    """Each kernel of the compiled table, selected exactly through its config,
    on inputs ragged in M and N: exact integers bit-exact, random data within
    tolerance.  Split-output kernels run with split_k = 2."""
    names = {0: "none", 1: "tensor", 2: "block128", 3: "mx128", 4: "mx32"}
    for cfg, dt, sm, split_out in dgp.kernels():
        dtype = {dgp.BF16: "bf16", dgp.FP8_E4M3: "fp8", dgp.FP4_E2M1: "fp4"}[dt]
        mode = names[sm]
        if cfg.tile_m == 16:
            M, N = 37, 384
        else:
            M, N = 2 * cfg.tile_m + 44, 2 * cfg.tile_n + 128
        K = 1024 if dtype in ("fp8", "fp4") else 512
        split = 2 if split_out else 1
        what = f"{dtype} {mode} tile {cfg.tile_m}x{cfg.tile_n}x{cfg.tile_k} wm{cfg.waves_m} d{cfg.prefetch} s{split}"
        A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 5)
        got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
        _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
        assert np.array_equal(got, c16), what
        A, B, sA, sB = rand_inputs(dtype, mode, M, N, K, 6)
        got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
        c32, _ = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
        assert_close(got, c32, what=what)


def test_blockscale_fused_accumulate_bit_exact():
    """Exact-integer operands with random fp32 block scales: every 128-K
    partial is exact and each scaled accumulate rounds, so only the same
    fused multiply-add in the same order reproduces the oracle bit for bit.
    Kernels that walk K in order (large tiles, streaming tiles) match the
    oracle at their split; a K-split tile at split 1 sums its waves' slices
    (one 128-K block each at K = 1024) in wave order, which is the oracle's
    split-K over as many ranges as waves."""
    count = 0
    for cfg, dt, sm, split_out in dgp.kernels():
        if sm != dgp.SCALE_BLOCK128:
            continue
        if cfg.tile_m == 16:
            M, N = 37, 384
        else:
            M, N = 2 * cfg.tile_m + 44, 2 * cfg.tile_n + 128
        K = 1024
        ksplit = cfg.tile_m == 16 and (cfg.tile_n in (8, 16) or cfg.waves_m in (8, 16))
        if ksplit and split_out:
            continue   # partials of partials: no single oracle order
        split = 2 if split_out else 1
        what = f"tile {cfg.tile_m}x{cfg.tile_n} wm{cfg.waves_m} d{cfg.prefetch} s{cfg.schedule} split {split}"
        print(what, flush=True)
        A = synth.exact_ints((M, K), 81, "fp8")
        B = synth.exact_ints((N, K), 82, "fp8")
        sA = synth.random_block_scales((M, K // 128), 83)
        sB = synth.random_block_scales((N // 128, K // 128), 84)
        got = run_gpu(A, B, "fp8", "block128", sA, sB, split_k=split, config=cfg)
        _, c16 = run_oracle(A, B, "fp8", "block128", sA, sB, split_k=cfg.waves_m if ksplit else split)
        assert np.array_equal(got, c16), what
        count += 1
    assert count >= 8


@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
def test_k_tile_counts_not_multiple_of_prefetch_depth(dtype, mode):
    """ntiles % depth != 0 exercises the steps after the unrolled main loop
    (1, 2, 3, 5, 7 k-tiles of 128 bytes)."""
    per_byte = {"bf16": 0.5, "fp8": 1, "fp4": 2}[dtype]   # elements per row byte
    dcode = {"bf16": dgp.BF16, "fp8": dgp.FP8_E4M3, "fp4": dgp.FP4_E2M1}[dtype]
    scode = {"none": dgp.SCALE_NONE, "tensor": dgp.SCALE_TENSOR, "block128": dgp.SCALE_BLOCK128,
             "mx128": dgp.SCALE_MX128, "mx32": dgp.SCALE_MX32}[mode]
    for tiles in (1, 2, 3, 5, 7):
        k = int(tiles * 128 * per_byte)
        for cfg in [c for c, dt, sm, so in dgp.kernels() if c.tile_m > 16 and dt == dcode and sm == scode
                    and not so]:
            N = 640 if mode == "block128" else 528   # blockscale: whole 128-column blocks
            A, B, sA, sB = exact_inputs(dtype, mode, 300, N, k, 13)
            got = run_gpu(A, B, dtype, mode, sA, sB, config=cfg)
            _, c16 = run_oracle(A, B, dtype, mode, sA, sB)
            assert np.array_equal(got, c16), (k, cfg.tile_m, cfg.tile_n, cfg.waves_m, cfg.prefetch, cfg.schedule)


# Ordered load rings: the one-row VALU kernel (every compiled form) and the
# K-split tiles that use the ordered ring (16 columns; fp8 half strips):
# (config, dtype, mode, K bytes per step, waves, ring depth).
RING_CASES = [
    (dgp.Config(tile_m=1, tile_n=16, waves_m=4, prefetch=8), "bf16", "none", 64, 4, 8),
    (dgp.Config(tile_m=1, tile_n=8, waves_m=8, prefetch=4), "bf16", "none", 128, 8, 4),
    (dgp.Config(tile_m=1, tile_n=16, waves_m=8, prefetch=8), "fp8", "tensor", 64, 8, 8),
    (dgp.Config(tile_m=1, tile_n=8, waves_m=4, prefetch=8), "fp8", "tensor", 128, 4, 8),
    (dgp.Config(tile_m=16, tile_n=16, waves_m=8, prefetch=4), "bf16", "none", 64, 8, 4),
    (dgp.Config(tile_m=16, tile_n=16, waves_m=8, prefetch=4), "fp8", "tensor", 128, 8, 4),
    (dgp.Config(tile_m=16, tile_n=8, waves_m=8, prefetch=4), "fp8", "block128", 128, 8, 4),
    (dgp.Config(tile_m=16, tile_n=16, waves_m=8, prefetch=4), "fp8", "mx128", 128, 8, 4),
]


@pytest.mark.parametrize("case", range(len(RING_CASES)))
def test_ring_slice_lengths(case):
    """Every slice length a wave can get, 0 .. 3 x the ring depth steps (empty
    slices, each of the 2 x depth straight-line tails, one and two
    main-loop iterations before a tail), with equal and unequal slices
    across the waves; exact-integer inputs, bit-exact."""
    cfg, dtype, mode, step_bytes, nw, depth = RING_CASES[case]
    eb = 2 if dtype == "bf16" else 1
    M, N = (3 if cfg.tile_m == 1 else 19), 256
    seen = set()
    for n in range(0, 3 * depth + 1):
        for extra in (0, nw // 2, nw - 1):
            steps = nw * n + extra
            kb = steps * step_bytes
            if kb == 0 or kb % 128 or (kb // eb) % 128 and mode in ("block128", "mx128") or kb in seen:
                continue
            seen.add(kb)
            K = kb // eb
            A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 29)
            got = run_gpu(A, B, dtype, mode, sA, sB, config=cfg)
            _, c16 = run_oracle(A, B, dtype, mode, sA, sB)
            assert np.array_equal(got, c16), (dtype, mode, cfg.tile_m, cfg.tile_n, K)
    assert len(seen) > 2 * depth


@pytest.mark.parametrize("tile_n,waves", [(64, 0), (32, 0), (16, 0), (8, 0), (32, 8), (64, 8)])
@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
@pytest.mark.parametrize("M", [1, 16, 20])
@pytest.mark.parametrize("split_k", [1, 2, 4, 8])
def test_stream_splitk(dtype, mode, M, split_k, tile_n, waves):
    """Decode kernels: the 16x64 and 16x32 streaming tiles, the 16x16 K-split
    tile, its half-strip form (16x8) and its 2- and 4-strip forms (16x32,
    16x64 with 8 waves)."""
    N, K = 384, 2048
    cfg = dgp.Config(16, tile_n, 0, 0, 1, 0, 0, waves)
    A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 3)
    got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split_k, config=cfg)
    _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split_k)
    assert np.array_equal(got, c16)
    A, B, sA, sB = rand_inputs(dtype, mode, M, N, K, 4)
    got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split_k, config=cfg)
    c32, _ = run_oracle(A, B, dtype, mode, sA, sB, split_k=split_k)
    assert_close(got, c32)


@pytest.mark.parametrize("tile_n", [16, 8, 32, 64])
@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
def test_ksplit_uneven_and_empty_slices(dtype, mode, tile_n):
    """K-split kernel (half, one, two and four strips): step counts not
    divisible by the 8 waves and fewer steps than waves (some waves own no
    K), with splits.  (bf16 and fp4 steps are 64 bytes and K rows must be
    whole 128 bytes, so their counts are even.)"""
    cfg = dgp.Config(16, tile_n, 0, 0, 1, 0, 0, 8)
    step = {"bf16": 32, "fp8": 128, "fp4": 128}[dtype]    # K elements per MFMA step
    cases = (((18, 1), (26, 1), (2, 1), (6, 1), (36, 2), (20, 2)) if dtype != "fp8" else
             ((9, 1), (13, 1), (1, 1), (3, 1), (5, 1), (18, 2), (10, 2)))
    for steps, split in cases:
        K = steps * step
        if mode in ("block128", "mx128") and (K // split) % 128:
            continue
        A, B, sA, sB = exact_inputs(dtype, mode, 5, 256, K, 31)
        got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
        _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
        assert np.array_equal(got, c16), (steps, split)


@pytest.mark.parametrize("tile_n", [16, 8, 32, 64])
def test_mx128_ksplit_long_k_ragged_n(tile_n):
    """mxfp8 K-split tiles on long K ranges (K = 8192, split 1; K = 16384,
    split 2) with N = 80, which leaves the last tile's strips past N: every
    element bit-exact.  A NaN byte (E8M0 255) in the last K block of one B
    row poisons exactly that column of C."""
    cfg = dgp.Config(16, tile_n, 0, 0, 1, 0, 0, 8)
    for M, N, K, split in ((16, 80, 8192, 1), (5, 80, 16384, 2)):
        A, B, sA, sB = exact_inputs("fp8", "mx128", M, N, K, 53)
        got = run_gpu(A, B, "fp8", "mx128", sA, sB, split_k=split, config=cfg)
        _, c16 = run_oracle(A, B, "fp8", "mx128", sA, sB, split_k=split)
        assert np.array_equal(got, c16), (M, N, K, split)
    sB2 = sB.copy()
    sB2[70, 127] = 255
    f = (run_gpu(A, B, "fp8", "mx128", sA, sB2, split_k=2, config=cfg).astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(f[:, 70])) and np.all(np.isfinite(np.delete(f, 70, axis=1)))


@pytest.mark.parametrize("tile_n", [16, 8, 32, 64])
@pytest.mark.parametrize("M", [16, 7])
def test_mx32_scale_groups_past_array_end(M, tile_n):
    """mxfp4 K-split tiles load each row's E8M0 bytes four steps at a time,
    one group ahead; when a wave's slice is not a multiple of 4 steps, the
    last wave's group runs past the end of both scale arrays.  The final
    scale bytes of the last row of A (M = 16: the tile's last row, M = 7: a
    ragged tile) and of the last row of B must still be read: every element
    of C, and so its last row and column, is bit-exact."""
    cfg = dgp.Config(16, tile_n, 0, 0, 1, 0, 0, 8)
    for steps, split, N in ((14, 1, 48), (22, 1, 64), (10, 1, 16), (28, 2, 48), (6, 1, 80)):
        K = steps * 128
        A, B, sA, sB = exact_inputs("fp4", "mx32", M, N, K, 41 + steps)
        got = run_gpu(A, B, "fp4", "mx32", sA, sB, split_k=split, config=cfg)
        _, c16 = run_oracle(A, B, "fp4", "mx32", sA, sB, split_k=split)
        assert np.array_equal(got, c16), (steps, split, N)


@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
@pytest.mark.parametrize("M,split_k", [(1, 1), (16, 1), (20, 2)])
def test_half_strip_writes_every_column(dtype, mode, M, split_k):
    """Half-strip K-split tile: the two workgroups of a strip each store
    only their 8 columns; together they cover C.  C starts as NaN, so a
    column that neither stores stays NaN and fails the bit-exact check."""
    N, K = 256, 1024
    A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 17)
    a = dev_codes(A, dtype)
    Bs_dev = dgp.preshuffle_b(dev_codes(B, dtype))
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dgp.gemm_preshuffle_splitk(a, Bs_dev, split_k, dev_scales(sA, mode), dev_scales(sB, mode), dmode(mode),
                               out=out, config=dgp.Config(16, 8, 0, 0, 1, 0, 0))
    torch.cuda.synchronize()
    _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split_k)
    assert np.array_equal(host_bits(out), c16)


@pytest.mark.parametrize("tile_n,waves", [(64, 4), (32, 2), (16, 8), (8, 8), (32, 8), (64, 8)])
@pytest.mark.parametrize("dtype,mode", [("bf16", "none"), ("fp8", "tensor"), ("fp8", "block128"),
                                        ("fp8", "mx128"), ("fp4", "mx32")])
def test_decode_tiles_ragged_width(dtype, mode, tile_n, waves):
    """Every 16-row tile on widths that are not a whole number of tiles: the
    last workgroup owns strips past N (loaded as zero, never stored).  C
    starts as NaN, so a column left unwritten fails the bit-exact check."""
    for N, M, split_k in ((400, 20, 1), (336, 5, 2), (144, 1, 1)):
        if mode == "block128" and N % 128:
            N = 640 if N > 256 else 128 * (N // 128 + 1)   # blockscale: whole 128-column blocks
        K = 1024
        A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 23)
        a = dev_codes(A, dtype)
        Bs_dev = dgp.preshuffle_b(dev_codes(B, dtype))
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        dgp.gemm_preshuffle_splitk(a, Bs_dev, split_k, dev_scales(sA, mode), dev_scales(sB, mode), dmode(mode),
                                   out=out, config=dgp.Config(16, tile_n, 0, 0, 1, 0, 0, waves))
        torch.cuda.synchronize()
        _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split_k)
        assert np.array_equal(host_bits(out), c16), (N, M, split_k)


@pytest.mark.parametrize("dtype,mode", [("fp8", "tensor"), ("fp4", "mx32")])
@pytest.mark.parametrize("split_k", [1, 2])
def test_stream_multi_panel(dtype, mode, split_k):
    """K range larger than one LDS panel of A (several panels per split; the
    fp4 panel, which also stages its scales, is 4096 bytes = 8192 values)."""
    M, N, K = 20, 272, 24576 if dtype == "fp8" else 40960
    A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 9)
    got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split_k, config=dgp.Config(16, 64, 0, 0, 1, 0, 0))
    _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split_k)
    assert np.array_equal(got, c16)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_one_hot_rows_bit_exact(dtype):
    M, N, K = 64, 320, 1024
    B = synth.bf16_uniform((N, K), 1) if dtype == "bf16" else synth.fp8_per_tensor((N, K), 1)[0]
    ks = np.random.Generator(np.random.PCG64(2)).integers(0, K, size=M)
    A = np.zeros((M, K), dtype=np.uint16 if dtype == "bf16" else np.uint8)
    A[np.arange(M), ks] = 0x3F80 if dtype == "bf16" else 0x38
    mode = "none" if dtype == "bf16" else "tensor"
    sA = None if dtype == "bf16" else np.array([0.5], np.float32)
    sB = None if dtype == "bf16" else np.array([0.25], np.float32)
    for cfg in (None, dgp.Config(16, 64, 0, 0, 1, 0, 0), dgp.Config(128, 128, 128, 1, 4, 0, 0)):
        got = run_gpu(A, B, dtype, mode, sA, sB, config=cfg) if cfg else run_gpu(A, B, dtype, mode, sA, sB)
        _, c16 = run_oracle(A, B, dtype, mode, sA, sB)
        assert np.array_equal(got, c16)
    if dtype == "bf16":
        assert np.array_equal(got, B[:, ks].T)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_longest_rows_one_hot(dtype):
    """The longest rows the library accepts (K * element bytes = 8 MiB): A
    rows one-hot at distinct k near the end of K reach the largest buffer
    offsets of the tiled, streaming, K-split and split-K paths.  One-hot rows
    turn the long contraction into a single product per output, so the
    oracle computes the expected C from the extracted B columns alone."""
    eb = 2 if dtype == "bf16" else 1
    K = (8 << 20) // eb
    M, N = 272, 272
    gen = torch.Generator(device=DEV).manual_seed(77)
    if dtype == "bf16":
        B = (torch.rand((N, K), generator=gen, device=DEV, dtype=torch.float32) - 0.5).to(torch.bfloat16)
        one = 0x3F80
    else:
        codes = torch.randint(0, 256, (N, K), generator=gen, device=DEV, dtype=torch.int32)
        codes = torch.where((codes & 0x7F) == 0x7F, torch.zeros_like(codes), codes)   # no NaN codes
        B = codes.to(torch.uint8).view(torch.float8_e4m3fn)
        del codes
        one = 0x38
    ks = K - 1 - 13 * np.arange(M)
    A = torch.zeros((M, K), dtype=B.dtype, device=DEV)
    A.view(torch.int16 if dtype == "bf16" else torch.uint8)[torch.arange(M, device=DEV),
                                                             torch.from_numpy(ks).to(DEV)] = one
    Bs = dgp.preshuffle_b(B)
    # expected: the oracle on A' = [I 0] and B' = the picked columns, padded to 384
    cols = B.view(torch.int16 if dtype == "bf16" else torch.uint8)[:, torch.from_numpy(ks).to(DEV)].cpu().numpy()
    del B
    Kp = 384
    Ap = np.zeros((M, Kp), dtype=np.uint16 if dtype == "bf16" else np.uint8)
    Ap[np.arange(M), np.arange(M)] = one
    Bp = np.zeros((N, Kp), dtype=Ap.dtype)
    Bp[:, :M] = cols.view(Ap.dtype)
    mode = "none" if dtype == "bf16" else "tensor"
    s1 = None if dtype == "bf16" else np.array([1.0], np.float32)
    _, want = run_oracle(Ap, Bp, dtype, mode, s1, s1)
    sd = None if dtype == "bf16" else torch.ones(1, device=DEV)
    runs = [(M, None, 1), (M, dgp.Config(128, 128, 128, 1, 4, 0, 4, 2, 2), 2),
            (20, dgp.Config(16, 64, 0, 0, 1, 0, 0), 1), (20, dgp.Config(16, 64, 0, 0, 1, 0, 0), 2),
            (20, dgp.Config(16, 16, 0, 0, 1, 0, 0), 1), (1, None, 4)]
    for rows, cfg, split in runs:
        C = dgp.gemm_preshuffle_splitk(A[:rows], Bs, split, sd, sd, config=cfg)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(C), want[:rows]), (rows, cfg, split)


def test_identity_b_returns_a():
    M, K = 300, 512
    A = synth.bf16_uniform((M, K), 3)
    B = np.zeros((K, K), np.uint16)
    B[np.arange(K), np.arange(K)] = 0x3F80
    for cfg in (None, dgp.Config(256, 256, 128, 1, 8, 0, 8, 1, 2), dgp.Config(256, 256, 128, 1, 8, 0, 8, 2, 2)):
        got = run_gpu(A, B, "bf16", "none", config=cfg) if cfg else run_gpu(A, B, "bf16", "none")
        assert np.array_equal(got, A)


@pytest.mark.parametrize("tile", TILED)
def test_xcd_remap_is_bit_identical(tile):
    M, N, K = 1100, 1072, 512
    A, B, _, _ = rand_inputs("bf16", "none", M, N, K, 8)
    outs = []
    for remap, group in ((0, 1), (1, 1), (1, 4), (1, 8)):
        outs.append(run_gpu(A, B, "bf16", "none",
                            config=dgp.Config(tile[0], tile[1], 128, remap, group, 0, tile[3], tile[2], 2)))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


SCHED_CFG = {2: (1, 2), 3: (2, 1)}   # schedule -> (waves_m, prefetch) of its 256x256 kernel


@pytest.mark.parametrize("sched", [2, 3])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_schedules_ragged_splitk_and_remap(dtype, sched):
    """The ping-pong and both-in-LDS schedules on a ragged multi-tile grid:
    exact integers bit-exact for split_k 1 and 3 (3 splits of 5 k-tiles each)
    under every tile map; random data within tolerance."""
    wm, pf = SCHED_CFG[sched]
    mode = "none" if dtype == "bf16" else "tensor"
    M, N = 3 * 256 + 17, 2 * 256 + 48
    K = 15 * 128 // (2 if dtype == "bf16" else 1)
    A, B, sA, sB = exact_inputs(dtype, mode, M, N, K, 21)
    outs = []
    for split in (1, 3):
        for remap, group in ((0, 1), (1, 1), (1, 8)):
            cfg = dgp.Config(256, 256, 128, remap, group, 0, 0, wm, pf, sched)
            got = run_gpu(A, B, dtype, mode, sA, sB, split_k=split, config=cfg)
            _, c16 = run_oracle(A, B, dtype, mode, sA, sB, split_k=split)
            assert np.array_equal(got, c16), (split, remap, group)
    A, B, sA, sB = rand_inputs(dtype, mode, M, N, K, 22)
    got = run_gpu(A, B, dtype, mode, sA, sB, config=dgp.Config(256, 256, 128, 1, 8, 0, 0, wm, pf, sched))
    c32, _ = run_oracle(A, B, dtype, mode, sA, sB)
    assert_close(got, c32)


@pytest.mark.parametrize("M", [1, 16, 20])
@pytest.mark.parametrize("split_k", [1, 2, 4, 7])
def test_mxfp4_decode(M, split_k):
    """mxfp4 through the K-split and the streaming kernel: exact integers
    bit-exact, random microscaled data within tolerance, at the decode
    K = 7168; split 7 gives 8 steps of 64 bytes per split, split 4 14
    (uneven over the K-split kernel's 8 waves)."""
    N, K = 384, 7168
    A, B, sA, sB = exact_inputs("fp4", "mx32", M, N, K, 51)
    _, c16 = run_oracle(A, B, "fp4", "mx32", sA, sB, split_k=split_k)
    for tile_n in (16, 32, 64):
        got = run_gpu(A, B, "fp4", "mx32", sA, sB, split_k=split_k, config=dgp.Config(16, tile_n, 0, 0, 1, 0, 0))
        assert np.array_equal(got, c16), tile_n
    A, B, sA, sB = rand_inputs("fp4", "mx32", M, N, K, 52)
    c32, _ = run_oracle(A, B, "fp4", "mx32", sA, sB, split_k=split_k)
    for cfg in (None, dgp.Config(16, 64, 0, 0, 1, 0, 0)):
        got = run_gpu(A, B, "fp4", "mx32", sA, sB, split_k=split_k, config=cfg)
        assert_close(got, c32)


@pytest.mark.parametrize("tile_n", [64, 32, 16])
def test_mxfp4_scale_indexing_and_packer(tile_n):
    """Doubling one column's 32-block B scales doubles exactly that column,
    doubling one A row's doubles exactly that row, and raising one 32-block
    scale of one column changes only that column; the packer round-trips fp4
    weights bit-exactly (bytes are bytes)."""
    M, N, K = 3, 64, 512
    cfg = dgp.Config(16, tile_n, 0, 0, 1, 0, 0)
    A, B, eA, eB = exact_inputs("fp4", "mx32", M, N, K, 61)
    eA[:] = 127
    eB[:] = 127
    base = run_gpu(A, B, "fp4", "mx32", eA, eB, config=cfg)
    f = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    eB2 = eB.copy()
    eB2[21, :] = 128
    got = run_gpu(A, B, "fp4", "mx32", eA, eB2, config=cfg)
    assert np.array_equal(f(got)[:, 21], 2 * f(base)[:, 21])
    assert np.array_equal(np.delete(got, 21, axis=1), np.delete(base, 21, axis=1))
    eA2 = eA.copy()
    eA2[1, :] = 128
    got = run_gpu(A, B, "fp4", "mx32", eA2, eB, config=cfg)
    assert np.array_equal(f(got)[1], 2 * f(base)[1])
    assert np.array_equal(got[[0, 2]], base[[0, 2]])
    eB3 = eB.copy()
    eB3[37, 5] = 130
    got = run_gpu(A, B, "fp4", "mx32", eA, eB3, config=cfg)
    _, c16 = run_oracle(A, B, "fp4", "mx32", eA, eB3)
    assert np.array_equal(got, c16)
    assert np.array_equal(np.delete(got, 37, axis=1), np.delete(base, 37, axis=1))
    Bd = dev_codes(B, "fp4")
    Bs = dgp.preshuffle_b(Bd)
    assert np.array_equal(Bs.view(torch.uint8).cpu().numpy(), oracle.preshuffle_b(B))
    assert torch.equal(dgp.unshuffle_b(Bs).view(torch.uint8), Bd.view(torch.uint8))


@pytest.mark.parametrize("tile_n", [64, 32, 16])
def test_mx128_scale_indexing(tile_n):
    """mxfp8 scales reach the right operands: doubling one column's B scale
    row doubles exactly that column of C, and a NaN A scale poisons exactly
    its row (E8M0 255)."""
    M, N, K = 5, 128, 512
    cfg = dgp.Config(16, tile_n, 0, 0, 1, 0, 0)
    A, B, eA, eB = exact_inputs("fp8", "mx128", M, N, K, 41)
    eA[:] = 127
    eB[:] = 127
    base = run_gpu(A, B, "fp8", "mx128", eA, eB, config=cfg)
    eB2 = eB.copy()
    eB2[37, :] = 128
    got = run_gpu(A, B, "fp8", "mx128", eA, eB2, config=cfg)
    _, want = run_oracle(A, B, "fp8", "mx128", eA, eB2)
    assert np.array_equal(got, want)
    f = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(got)[:, 37], 2 * f(base)[:, 37])
    assert np.array_equal(np.delete(got, 37, axis=1), np.delete(base, 37, axis=1))
    eA2 = eA.copy()
    eA2[3, 2] = 255
    got = f(run_gpu(A, B, "fp8", "mx128", eA2, eB, config=cfg))
    assert np.all(np.isnan(got[3])) and np.all(np.isfinite(np.delete(got, 3, axis=0)))


def test_negative_control_corrupted_weight_diverges():
    M, N, K = 64, 256, 512
    A, B, _, _ = rand_inputs("bf16", "none", M, N, K, 12)
    Bs = dgp.preshuffle_b(dev_codes(B, "bf16"))
    raw = Bs.view(torch.uint8).view(-1)
    raw[12345] ^= 0x40
    got = run_gpu(A, B, "bf16", "none", Bs_dev=Bs)
    c32, c16 = run_oracle(A, B, "bf16", "none")
    assert not np.array_equal(got, c16)
    # and a double preshuffle (the hazard of shuffling an already-preshuffled B) corrupts C
    Bss = dgp.preshuffle_b(dgp.preshuffle_b(dev_codes(B, "bf16")))
    got = run_gpu(A, B, "bf16", "none", Bs_dev=Bss)
    err = np.max(np.abs((got.astype(np.uint32) << 16).view(np.float32) - c32))
    assert err > 1e-2 * np.max(np.abs(c32))


def test_k_zero_gives_zeros_and_empty_is_noop():
    A = torch.zeros((5, 0), dtype=torch.bfloat16, device=DEV)
    Bs = torch.zeros((32, 0), dtype=torch.bfloat16, device=DEV)
    out = torch.full((5, 32), 7.0, dtype=torch.bfloat16, device=DEV)
    dgp.gemm_preshuffle(A, Bs, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    A = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    Bs = torch.zeros((32, 128), dtype=torch.bfloat16, device=DEV)
    assert dgp.gemm_preshuffle(A, Bs).shape == (0, 32)


def test_binding_rejects_mismatched_operands_before_launch():
    """An output, weight or scale tensor smaller than the call assumes is
    refused by the binding (ValueError) and nothing runs: the output keeps
    its contents."""
    A = torch.ones((16, 1024), dtype=torch.bfloat16, device=DEV)
    Bs = torch.ones((256, 1024), dtype=torch.bfloat16, device=DEV)
    out = torch.full((16, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        dgp.gemm_preshuffle(A, Bs, out=out)
    with pytest.raises(ValueError):
        dgp.gemm_preshuffle_splitk(A, Bs, 2, out=out)
    with pytest.raises(ValueError):
        dgp.gemm_preshuffle(A, torch.ones((256, 512), dtype=torch.bfloat16, device=DEV))
    A8 = torch.zeros((16, 1024), dtype=torch.float8_e4m3fn, device=DEV)
    B8 = torch.zeros((256, 1024), dtype=torch.float8_e4m3fn, device=DEV)
    out2 = torch.full((16, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):   # blockscale sB must be [N/128][K/128]
        dgp.gemm_preshuffle(A8, B8, torch.ones((16, 8), device=DEV), torch.ones((1, 8), device=DEV),
                            dgp.SCALE_BLOCK128, out=out2)
    with pytest.raises(ValueError):
        dgp.preshuffle_b(B8, out=torch.empty((128, 1024), dtype=torch.float8_e4m3fn, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0).item() and torch.all(out2 == 7.0).item()


def test_side_stream_allocations():
    """A call on a stream other than the current one allocates its output
    and split-K workspace on that stream; the result equals the
    current-stream result bit for bit."""
    M, N, K = 16, 2048, 7168
    A, B, sA, sB = exact_inputs("fp8", "tensor", M, N, K, 29)
    a = dev_codes(A, "fp8")
    Bs_dev = dgp.preshuffle_b(dev_codes(B, "fp8"))
    dA, dB = dev_scales(sA, "tensor"), dev_scales(sB, "tensor")
    want = dgp.gemm_preshuffle_splitk(a, Bs_dev, 4, dA, dB, dgp.SCALE_TENSOR)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = [dgp.gemm_preshuffle_splitk(a, Bs_dev, 4, dA, dB, dgp.SCALE_TENSOR, stream=s) for _ in range(4)]
    with torch.cuda.stream(s):   # work queued behind the calls on their stream
        junk = [torch.full((M * N * 4,), 3.0, device=DEV) for _ in range(4)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    for o in outs:
        assert torch.equal(o.view(torch.int16), want.view(torch.int16))


def test_binding_rejects_bad_arguments():
    A = torch.zeros((16, 128), dtype=torch.float8_e4m3fn, device=DEV)
    Bs = torch.zeros((128, 128), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.ones(1, device=DEV)
    with pytest.raises(dgp.DgpError) as e:
        dgp.gemm_preshuffle_splitk(A, Bs, 3, s, s)
    assert e.value.name == "DGP_ERR_SPLITK"
    with pytest.raises(dgp.DgpError) as e:
        dgp.gemm_preshuffle(A, Bs, s, s, config=dgp.Config(100, 64, 128, 1, 4, 0, 0))
    assert e.value.name == "DGP_ERR_CONFIG"
    with pytest.raises(dgp.DgpError) as e:
        dgp.gemm_preshuffle(A, Bs, s, s, config=dgp.Config(128, 128, 128, 1, 4, -1, 2))
    assert e.value.name == "DGP_ERR_CONFIG"
