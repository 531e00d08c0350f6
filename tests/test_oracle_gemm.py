"""Pins for the oracle GEMM (per-tensor, blockscale, split-K).

The oracle is checked against things other than itself: exact rational
arithmetic on tiny shapes, numpy's float64 matmul of independently decoded
inputs (torch conversions) under the standard forward error bound of
recursive fp32 summation (Higham, Accuracy and Stability of Numerical
Algorithms, 2nd ed., section 3.1: |fl(sum) - sum| <= gamma_n * sum|terms|,
gamma_n = n*u/(1-n*u), u = 2^-24), exact-integer inputs where every order of
summation is exact, one-hot and identity operands, and split-K sums.
Shapes are non-square (M != N != K) so that a transposed operand fails.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def dec_torch(codes, dtype):
    """Independent decode through torch's storage types."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(codes).copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def odt(orc, dtype):
    return orc.BF16 if dtype == "bf16" else orc.FP8_E4M3


def rand_codes(shape, seed, dtype):
    if dtype == "bf16":
        return synth.bf16_uniform(shape, seed)
    codes, _ = synth.fp8_per_tensor(shape, seed)
    return codes


# ------------------------------------------------------- exact brute force

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (3, 32, 64), (5, 16, 128), (7, 48, 192)])
def test_tiny_against_exact_rationals(orc, dtype, M, N, K):
    A = rand_codes((M, K), 11 + M, dtype)
    B = rand_codes((N, K), 13 + N, dtype)
    a = dec_torch(A, dtype)
    b = dec_torch(B, dtype)
    c32, c16 = orc.gemm(A, B, odt(orc, dtype))
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(a[m, k])) * Fraction(float(b[n, k])) for k in range(K)),
                        Fraction(0))
            absum = sum(abs(float(a[m, k]) * float(b[n, k])) for k in range(K))
            err = abs(Fraction(float(c32[m, n])) - exact)
            assert err <= Fraction(gamma(K) * absum) + Fraction(1, 2**149), (m, n)
            assert c16[m, n] == orc.bf16_round(float(c32[m, n]))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_exact_integer_mode_is_exact(orc, dtype):
    M, N, K = 9, 32, 256
    A = synth.exact_ints((M, K), 1, dtype)
    B = synth.exact_ints((N, K), 2, dtype)
    a = dec_torch(A, dtype).astype(np.int64)
    b = dec_torch(B, dtype).astype(np.int64)
    exact = a @ b.T
    s = np.float32(0.125)
    mode = orc.SCALE_TENSOR if dtype == "fp8" else orc.SCALE_NONE
    sA = np.array([s]) if dtype == "fp8" else None
    sB = np.array([1.0]) if dtype == "fp8" else None
    c32, c16 = orc.gemm(A, B, odt(orc, dtype), mode, sA, sB)
    want = exact.astype(np.float64) * (0.125 if dtype == "fp8" else 1.0)
    assert np.array_equal(c32.astype(np.float64), want)
    ref16 = torch.from_numpy(want.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(c16.view(np.int16), ref16)


# ------------------------------------------------- numpy float64 + bounds

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K", [(17, 48, 320), (64, 96, 1024)])
def test_random_against_fp64_matmul(orc, dtype, M, N, K):
    A = rand_codes((M, K), 21, dtype)
    B = rand_codes((N, K), 22, dtype)
    a, b = dec_torch(A, dtype), dec_torch(B, dtype)
    c64 = a @ b.T
    bound = gamma(K) * (np.abs(a) @ np.abs(b).T)
    c32, c16 = orc.gemm(A, B, odt(orc, dtype))
    assert np.all(np.abs(c32 - c64) <= bound + 1e-30)
    # the fp32 accumulation really is fp32 (not exact): some entry differs from fp64
    assert np.any(c32.astype(np.float64) != c64)


def test_per_tensor_scale_against_fp64(orc):
    M, N, K = 24, 80, 512
    A, sA = synth.fp8_per_tensor((M, K), 31)
    B, sB = synth.fp8_per_tensor((N, K), 32)
    a, b = dec_torch(A, "fp8"), dec_torch(B, "fp8")
    s = float(sA[0]) * float(sB[0])
    c64 = (a @ b.T) * s
    bound = (gamma(K) + 3 * U) * (np.abs(a) @ np.abs(b).T) * s
    c32, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_TENSOR, sA, sB)
    assert np.all(np.abs(c32 - c64) <= bound + 1e-30)
    # scales matter: a wrong scale would be far outside the bound
    c32_unscaled, _ = orc.gemm(A, B, orc.FP8_E4M3)
    assert np.max(np.abs(c32_unscaled - c64)) > 100 * np.max(bound)


def test_blockscale_against_fp64(orc):
    M, N, K = 6, 256, 512
    A, sA = synth.fp8_blockscale_a(M, K, 41, 42)
    B, sB = synth.fp8_blockscale_b(N, K, 43, 44)
    a, b = dec_torch(A, "fp8"), dec_torch(B, "fp8")
    KB = K // 128
    c64 = np.zeros((M, N))
    mag = np.zeros((M, N))
    for kb in range(KB):
        sl = slice(kb * 128, kb * 128 + 128)
        blk = a[:, sl] @ b[:, sl].T
        sc = sA[:, kb].astype(np.float64)[:, None] * np.repeat(sB[:, kb].astype(np.float64), 128)[None, :]
        c64 += blk * sc
        mag += (np.abs(a[:, sl]) @ np.abs(b[:, sl]).T) * sc
    bound = (gamma(K + KB) + 3 * U) * mag
    c32, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_BLOCK128, sA, sB)
    assert np.all(np.abs(c32 - c64) <= bound + 1e-30)
    # the check is sensitive to the scale indexing: pairing block kb's data
    # with another block's scales lands far outside the bound
    alt = np.zeros((M, N))
    for kb in range(KB):
        sl = slice(kb * 128, kb * 128 + 128)
        wk = KB - 1 - kb
        sc = sA[:, wk].astype(np.float64)[:, None] * np.repeat(sB[:, wk].astype(np.float64), 128)[None, :]
        alt += (a[:, sl] @ b[:, sl].T) * sc
    assert np.max(np.abs(alt - c64) - bound) > 0


def test_blockscale_uniform_scales_equal_per_tensor(orc):
    M, N, K = 5, 128, 384
    A = synth.exact_ints((M, K), 51, "fp8")
    B = synth.exact_ints((N, K), 52, "fp8")
    sA = np.full((M, K // 128), 0.5, np.float32)
    sB = np.full((N // 128, K // 128), 2.0, np.float32)
    c_blk, h_blk = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_BLOCK128, sA, sB)
    c_ten, h_ten = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_TENSOR, np.array([0.5]), np.array([2.0]))
    assert np.array_equal(c_blk, c_ten) and np.array_equal(h_blk, h_ten)


def test_blockscale_exact_against_integer_arithmetic(orc):
    """Exact-integer data and scales in {0.5,1,2}: the blockscale result is
    sum_kb (A_kb . B_kb) * sA[m][kb] * sB[n/128][kb] exactly."""
    M, N, K = 4, 256, 640
    A = synth.exact_ints((M, K), 61, "fp8")
    B = synth.exact_ints((N, K), 62, "fp8")
    sA = synth.exact_block_scales((M, K // 128), 63)
    sB = synth.exact_block_scales((N // 128, K // 128), 64)
    a = dec_torch(A, "fp8").astype(np.int64)
    b = dec_torch(B, "fp8").astype(np.int64)
    want = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // 128):
        sl = slice(kb * 128, kb * 128 + 128)
        for n in range(N):
            want[:, n] += (a[:, sl] @ b[n, sl]) * sA[:, kb] * sB[n // 128, kb]
    c32, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_BLOCK128, sA, sB)
    assert np.array_equal(c32.astype(np.float64), want)


def _round_f32(x: Fraction) -> np.float32:
    """x rounded to the nearest fp32, ties to even, by exact comparison of
    the neighbours of a first guess (normal range only)."""
    g = np.float32(float(x))
    cands = [np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(c.view(np.uint32)) & 1))
    return np.float32(best)


def test_blockscale_accumulates_with_one_rounding_per_block(orc):
    """Exact-integer operands make every 128-K partial p exact; random fp32
    scales make p*s inexact.  The oracle's sum is then, bit for bit, the
    sequence acc <- round(p*s + acc) over the blocks in K order (s = sA*sB
    rounded once), computed here in exact rational arithmetic, and it differs
    from the two-rounding sequence acc <- round(acc + round(p*s))."""
    M, N, K = 3, 256, 1280
    A = synth.exact_ints((M, K), 65, "fp8")
    B = synth.exact_ints((N, K), 66, "fp8")
    sA = synth.random_block_scales((M, K // 128), 67)
    sB = synth.random_block_scales((N // 128, K // 128), 68)
    a = dec_torch(A, "fp8").astype(np.int64)
    b = dec_torch(B, "fp8").astype(np.int64)
    c32, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_BLOCK128, sA, sB)
    two_roundings_differ = 0
    for m in range(M):
        for n in range(N):
            fused = np.float32(0.0)
            split = np.float32(0.0)
            for kb in range(K // 128):
                sl = slice(kb * 128, kb * 128 + 128)
                p = int(a[m, sl] @ b[n, sl])
                s = np.float32(sA[m, kb]) * np.float32(sB[n // 128, kb])
                fused = _round_f32(Fraction(p) * Fraction(float(s)) + Fraction(float(fused)))
                split = np.float32(split + np.float32(np.float32(p) * s))
            assert c32[m, n] == fused, (m, n)
            two_roundings_differ += int(split != fused)
    assert two_roundings_differ > 0


# ---------------------------------------------------- one-hot / identity

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_one_hot_rows_select_b_columns(orc, dtype):
    M, N, K = 12, 64, 192
    B = rand_codes((N, K), 71, dtype)
    ks = np.random.Generator(np.random.PCG64(72)).integers(0, K, size=M)
    one = 0x3F80 if dtype == "bf16" else 0x38
    A = np.zeros((M, K), dtype=np.uint16 if dtype == "bf16" else np.uint8)
    A[np.arange(M), ks] = one
    if dtype == "fp8":
        c32, c16 = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_TENSOR, np.array([0.25]), np.array([0.5]))
        want = dec_torch(B, "fp8")[:, ks].T * 0.125
        assert np.array_equal(c32.astype(np.float64), want)
    else:
        c32, c16 = orc.gemm(A, B, orc.BF16)
        assert np.array_equal(c16, B[:, ks].T)


def test_identity_b_returns_a(orc):
    M, K = 20, 128
    A = synth.bf16_uniform((M, K), 81)
    B = np.zeros((K, K), dtype=np.uint16)
    B[np.arange(K), np.arange(K)] = 0x3F80
    c32, c16 = orc.gemm(A, B, orc.BF16)
    assert np.array_equal(c16, A)


# ------------------------------------------------------------- split-K

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_splitk_exact_equals_unsplit(orc, dtype):
    M, N, K = 16, 128, 1024
    A = synth.exact_ints((M, K), 91, dtype)
    B = synth.exact_ints((N, K), 92, dtype)
    mode = orc.SCALE_TENSOR if dtype == "fp8" else orc.SCALE_NONE
    sA = np.array([0.125]) if dtype == "fp8" else None
    sB = np.array([1.0]) if dtype == "fp8" else None
    c1, h1 = orc.gemm(A, B, odt(orc, dtype), mode, sA, sB)
    for S in (2, 4, 8):
        cS, hS, parts = orc.gemm(A, B, odt(orc, dtype), mode, sA, sB, split_k=S, want_partials=True)
        assert np.array_equal(cS, c1) and np.array_equal(hS, h1)
        assert np.array_equal(parts.sum(axis=0, dtype=np.float64), c1.astype(np.float64))


def test_splitk_partials_are_slices_and_reduce_in_order(orc):
    M, N, K = 3, 48, 768
    A, sA = synth.fp8_per_tensor((M, K), 101)
    B, sB = synth.fp8_per_tensor((N, K), 102)
    S = 4
    cS, hS, parts = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_TENSOR, sA, sB, split_k=S,
                             want_partials=True)
    ch = K // S
    for s in range(S):
        ps, _ = orc.gemm(np.ascontiguousarray(A[:, s * ch:(s + 1) * ch]),
                         np.ascontiguousarray(B[:, s * ch:(s + 1) * ch]),
                         orc.FP8_E4M3, orc.SCALE_TENSOR, sA, sB)
        assert np.array_equal(parts[s], ps)
    tot = parts[0].copy()
    for s in range(1, S):
        tot = (tot + parts[s]).astype(np.float32)
    assert np.array_equal(cS, tot)
    lib = orc.lib()
    assert all(hS.reshape(-1)[i] == lib.oracle_bf16_round(float(cS.reshape(-1)[i]))
               for i in range(0, cS.size, 7))


def test_splitk_blockscale_random_within_bound(orc):
    M, N, K = 4, 128, 1024
    A, sA = synth.fp8_blockscale_a(M, K, 111, 112)
    B, sB = synth.fp8_blockscale_b(N, K, 113, 114)
    c1, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_BLOCK128, sA, sB)
    for S in (2, 4, 8):
        cS, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_BLOCK128, sA, sB, split_k=S)
        assert np.max(np.abs(cS - c1)) <= 1e-5 * np.max(np.abs(c1))


# ---------------------------------------------------- rows / arguments

def test_row_subset_matches_full(orc):
    M, N, K = 33, 64, 256
    A = synth.bf16_uniform((M, K), 121)
    B = synth.bf16_uniform((N, K), 122)
    c32, c16 = orc.gemm(A, B, orc.BF16)
    rows = [32, 0, 17, 5]
    r32, r16 = orc.gemm(A, B, orc.BF16, rows=rows)
    assert np.array_equal(r32, c32[rows]) and np.array_equal(r16, c16[rows])


def test_invalid_arguments_rejected(orc):
    A = np.zeros((4, 256), np.uint8)
    B = np.zeros((128, 256), np.uint8)
    with pytest.raises(ValueError):
        orc.gemm(A, B, orc.FP8_E4M3, split_k=3)           # K % split_k
    with pytest.raises(ValueError):
        orc.gemm(A, np.zeros((64, 256), np.uint8), orc.FP8_E4M3, orc.SCALE_BLOCK128,
                 np.ones((4, 2)), np.ones((1, 2)))        # N % 128 for blockscale
    with pytest.raises(ValueError):
        orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_TENSOR)   # scales missing
    with pytest.raises(ValueError):
        orc.gemm(A, B, orc.FP8_E4M3, rows=[4])           # row out of range


# ---------------------------------------------------- mxfp8 (E8M0, 128-K blocks)

def test_e8m0_decode_exhaustive(orc):
    """Every E8M0 byte against its definition, 2^(e-127) with e = 255 NaN,
    computed with Python's exact ldexp."""
    import math
    for e in range(256):
        got = orc.e8m0_decode(e)
        if e == 255:
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, e - 127), e


def _mx_scale(e):
    return np.exp2(e.astype(np.float64) - 127)


def test_mx128_against_fp64(orc):
    """Random microscaled data: within the recursive-summation bound of the
    fp64 blockwise result sum_kb (A_kb . B_kb) * 2^(eA-127) * 2^(eB-127), and
    pairing the blocks with another block's scales lands outside it."""
    M, N, K = 6, 48, 640
    A, eA = synth.fp8_mx128(M, K, 141, 142)
    B, eB = synth.fp8_mx128(N, K, 143, 144)
    assert len(np.unique(eA)) > 3 and len(np.unique(eB)) > 3   # the scales do vary
    a, b = dec_torch(A, "fp8"), dec_torch(B, "fp8")
    KB = K // 128
    c64, mag, alt = np.zeros((M, N)), np.zeros((M, N)), np.zeros((M, N))
    for kb in range(KB):
        sl = slice(kb * 128, kb * 128 + 128)
        sc = _mx_scale(eA[:, kb])[:, None] * _mx_scale(eB[:, kb])[None, :]
        c64 += (a[:, sl] @ b[:, sl].T) * sc
        mag += (np.abs(a[:, sl]) @ np.abs(b[:, sl]).T) * sc
        wk = KB - 1 - kb
        alt += (a[:, sl] @ b[:, sl].T) * (_mx_scale(eA[:, wk])[:, None] * _mx_scale(eB[:, wk])[None, :])
    bound = (gamma(K + KB) + U) * mag
    c32, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB)
    assert np.all(np.abs(c32 - c64) <= bound + 1e-30)
    assert np.max(np.abs(alt - c64) - bound) > 0


def test_mx128_exact_against_integer_arithmetic(orc):
    """Exact-integer data, E8M0 scales in {126,127,128}: exact, and with every
    scale 127 (1.0) it equals the unscaled product."""
    M, N, K = 5, 40, 512
    A = synth.exact_ints((M, K), 151, "fp8")
    B = synth.exact_ints((N, K), 152, "fp8")
    eA = synth.exact_e8m0_scales((M, K // 128), 153)
    eB = synth.exact_e8m0_scales((N, K // 128), 154)
    a = dec_torch(A, "fp8").astype(np.int64)
    b = dec_torch(B, "fp8").astype(np.int64)
    want = np.zeros((M, N))
    for kb in range(K // 128):
        sl = slice(kb * 128, kb * 128 + 128)
        want += (a[:, sl] @ b[:, sl].T) * _mx_scale(eA[:, kb])[:, None] * _mx_scale(eB[:, kb])[None, :]
    c32, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB)
    assert np.array_equal(c32.astype(np.float64), want)
    ones_a = np.full_like(eA, 127)
    ones_b = np.full_like(eB, 127)
    c_mx, h_mx = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, ones_a, ones_b)
    c_pl, h_pl = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_TENSOR, np.array([1.0]), np.array([1.0]))
    assert np.array_equal(c_mx, c_pl) and np.array_equal(h_mx, h_pl)


def test_mx128_b_scale_is_per_output_column(orc):
    """B's scales index [n][kb]: doubling one row of B's scales (one output
    column) doubles exactly that column and nothing else."""
    M, N, K = 4, 32, 256
    A = synth.exact_ints((M, K), 161, "fp8")
    B = synth.exact_ints((N, K), 162, "fp8")
    eA = np.full((M, K // 128), 127, np.uint8)
    eB = np.full((N, K // 128), 127, np.uint8)
    base, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB)
    eB2 = eB.copy()
    eB2[7, :] = 128
    c, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB2)
    assert np.array_equal(c[:, 7], 2 * base[:, 7])
    assert np.array_equal(np.delete(c, 7, axis=1), np.delete(base, 7, axis=1))


def test_mx128_nan_scale_poisons_its_row(orc):
    M, N, K = 3, 16, 256
    A = synth.exact_ints((M, K), 171, "fp8")
    B = synth.exact_ints((N, K), 172, "fp8")
    eA = np.full((M, K // 128), 127, np.uint8)
    eB = np.full((N, K // 128), 127, np.uint8)
    eA[1, 1] = 255
    c, _ = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB)
    assert np.all(np.isnan(c[1])) and np.all(np.isfinite(c[[0, 2]]))


def test_mx128_splitk_exact_equals_unsplit(orc):
    M, N, K = 3, 24, 1024
    A = synth.exact_ints((M, K), 181, "fp8")
    B = synth.exact_ints((N, K), 182, "fp8")
    eA = synth.exact_e8m0_scales((M, K // 128), 183)
    eB = synth.exact_e8m0_scales((N, K // 128), 184)
    c1, h1 = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB)
    for S in (2, 4, 8):
        cS, hS, parts = orc.gemm(A, B, orc.FP8_E4M3, orc.SCALE_MX128, eA, eB, split_k=S, want_partials=True)
        assert np.array_equal(cS, c1) and np.array_equal(hS, h1)
        assert parts.shape == (S, M, N)


def test_mx128_invalid_arguments_rejected(orc):
    A8 = np.zeros((2, 256), np.uint8)
    e = np.full((2, 2), 127, np.uint8)
    with pytest.raises(ValueError):   # bf16 has no MX mode here
        orc.gemm(np.zeros((2, 256), np.uint16), np.zeros((2, 256), np.uint16), orc.BF16, orc.SCALE_MX128, e, e)
    with pytest.raises(ValueError):   # K not a whole number of 128-blocks
        orc.gemm(np.zeros((2, 192), np.uint8), np.zeros((2, 192), np.uint8), orc.FP8_E4M3, orc.SCALE_MX128, e, e)
    with pytest.raises(ValueError):   # split ranges must be whole blocks
        orc.gemm(A8, np.zeros((2, 256), np.uint8), orc.FP8_E4M3, orc.SCALE_MX128, e, e, split_k=4)


# ---------------------------------------------------- mxfp4 (E2M1 pairs, 32-K blocks)

def _e2m1_table():
    """code -> value from the golden file (OCP MX specification values)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e2m1_ocp_values.txt")
    t = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            c, v = line.split()
            t[int(c, 16)] = float(v)
    assert len(t) == 16
    return t


def dec_fp4_table(packed):
    """Unpack [rows][K/2] bytes (element 2j low nibble) through the golden table."""
    t = _e2m1_table()
    lut = np.array([t[c] for c in range(16)], np.float64)
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.float64)
    out[..., 0::2] = lut[p & 0xF]
    out[..., 1::2] = lut[p >> 4]
    return out


def test_e2m1_decode_exhaustive_against_ocp_table(orc):
    t = _e2m1_table()
    for c in range(16):
        got = orc.e2m1_decode(c)
        assert got == t[c] and np.signbit(got) == np.signbit(t[c]), c


def test_fp4_nibble_order_one_hot(orc):
    """A one-hot A row at element k picks B[:, k]: pins that element k of a row
    lives in byte k/2.  (Which nibble of the byte holds the even element is a
    relabeling of K applied alike to A and B that never crosses a 32-element
    scale block, so it cannot change C; the library's convention -- even
    element in the low nibble -- is the packing in synth.pack_e2m1.)"""
    M, N, K = 8, 16, 64
    B = synth.exact_ints((N, K), 191, "fp4")
    b = dec_fp4_table(B)
    ks = [0, 1, 2, 33, 62, 63, 17, 40]
    codes = np.zeros((M, K), np.uint8)
    codes[np.arange(M), ks] = 0x2            # 1.0
    A = synth.pack_e2m1(codes)
    eA = np.full((M, K // 32), 127, np.uint8)
    eB = np.full((N, K // 32), 127, np.uint8)
    c32, _ = orc.gemm(A, B, orc.FP4_E2M1, orc.SCALE_MX32, eA, eB)
    assert np.array_equal(c32.astype(np.float64), b[:, ks].T)


def test_mx32_against_fp64(orc):
    M, N, K = 5, 40, 512
    A, eA = synth.fp4_mx32(M, K, 201, 202)
    B, eB = synth.fp4_mx32(N, K, 203, 204)
    assert len(np.unique(eA)) > 3
    a, b = dec_fp4_table(A), dec_fp4_table(B)
    KB = K // 32
    c64, mag, alt = np.zeros((M, N)), np.zeros((M, N)), np.zeros((M, N))
    for kb in range(KB):
        sl = slice(kb * 32, kb * 32 + 32)
        sc = _mx_scale(eA[:, kb])[:, None] * _mx_scale(eB[:, kb])[None, :]
        c64 += (a[:, sl] @ b[:, sl].T) * sc
        mag += (np.abs(a[:, sl]) @ np.abs(b[:, sl]).T) * sc
        wk = (kb + 1) % KB
        alt += (a[:, sl] @ b[:, sl].T) * (_mx_scale(eA[:, wk])[:, None] * _mx_scale(eB[:, wk])[None, :])
    bound = (gamma(K + KB) + U) * mag
    c32, _ = orc.gemm(A, B, orc.FP4_E2M1, orc.SCALE_MX32, eA, eB)
    assert np.all(np.abs(c32 - c64) <= bound + 1e-30)
    assert np.max(np.abs(alt - c64) - bound) > 0


def test_mx32_exact_integers_and_per_column_scale(orc):
    M, N, K = 4, 24, 256
    A = synth.exact_ints((M, K), 211, "fp4")
    B = synth.exact_ints((N, K), 212, "fp4")
    eA = synth.exact_e8m0_scales((M, K // 32), 213)
    eB = synth.exact_e8m0_scales((N, K // 32), 214)
    a, b = dec_fp4_table(A), dec_fp4_table(B)
    want = np.zeros((M, N))
    for kb in range(K // 32):
        sl = slice(kb * 32, kb * 32 + 32)
        want += (a[:, sl] @ b[:, sl].T) * _mx_scale(eA[:, kb])[:, None] * _mx_scale(eB[:, kb])[None, :]
    c32, _ = orc.gemm(A, B, orc.FP4_E2M1, orc.SCALE_MX32, eA, eB)
    assert np.array_equal(c32.astype(np.float64), want)
    eB2 = eB.copy()
    eB2[5] = np.minimum(eB2[5] + 1, 254)
    c2, _ = orc.gemm(A, B, orc.FP4_E2M1, orc.SCALE_MX32, eA, eB2)
    assert np.array_equal(c2[:, 5], 2 * c32[:, 5])
    assert np.array_equal(np.delete(c2, 5, axis=1), np.delete(c32, 5, axis=1))


def test_mx32_splitk_exact_equals_unsplit(orc):
    M, N, K = 3, 16, 512
    A = synth.exact_ints((M, K), 221, "fp4")
    B = synth.exact_ints((N, K), 222, "fp4")
    eA = synth.exact_e8m0_scales((M, K // 32), 223)
    eB = synth.exact_e8m0_scales((N, K // 32), 224)
    c1, h1 = orc.gemm(A, B, orc.FP4_E2M1, orc.SCALE_MX32, eA, eB)
    for S in (2, 4, 8):
        cS, hS = orc.gemm(A, B, orc.FP4_E2M1, orc.SCALE_MX32, eA, eB, split_k=S)
        assert np.array_equal(cS, c1) and np.array_equal(hS, h1)


def test_mx32_invalid_arguments_rejected(orc):
    A = np.zeros((2, 64), np.uint8)
    e = np.full((2, 4), 127, np.uint8)
    with pytest.raises(ValueError):   # e2m1 takes only its 32-block scales
        orc.gemm(A, A, orc.FP4_E2M1, orc.SCALE_MX128, e, e)
    with pytest.raises(ValueError):   # and the 32-block mode only e2m1
        orc.gemm(np.zeros((2, 128), np.uint8), np.zeros((2, 128), np.uint8), orc.FP8_E4M3, orc.SCALE_MX32, e, e)
    with pytest.raises(ValueError):   # split ranges must be whole 32-blocks
        orc.gemm(A, A, orc.FP4_E2M1, orc.SCALE_MX32, e, e, split_k=8)
