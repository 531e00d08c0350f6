"""Seeded synthetic inputs for the preshuffled-B GEMM workloads.

This module only draws random numbers and stores them in the input types
(bf16 bit patterns, OCP e4m3fn codes, fp32 scales) using torch's own CPU
conversions.  It holds none of the GEMM's arithmetic and is the one piece
shared by the oracle side and the GPU side of every test and of the bench.

Seeds follow ``seed = 1000*cfg + {0: A, 1: B, 2: scales}`` with numpy's PCG64.

Workloads (the five configurations the library is measured and tested on):

* ``bf16_small``   bf16 M=128, N=256, K=256; A, B ~ U(-1, 1).
* ``bf16_large``   bf16 M=N=4096, K=8192; A, B ~ N(0, 1)/sqrt(K).
* ``fp8_large``    e4m3 M=N=4096, K=8192; A, B ~ N(0, 1) quantised with the
                   per-tensor scale amax/448.
* ``fp8_decode``   e4m3 per-tensor, M in {1, 16}, N in {2048, 16384}, K=7168,
                   split_k in {1, 2, 4, 8}; data as ``fp8_large``.
* ``fp8_blockscale`` e4m3 M=16, N=16384, K=7168; N(0, 1) data quantised per
                   block (A: per row per 128-K block, B: per 128x128 block) with
                   scales U(0.5, 2) * amax_block / 448.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0

CFG_BF16_SMALL = 0
CFG_BF16_LARGE = 1
CFG_FP8_LARGE = 2
CFG_FP8_DECODE = 3
CFG_FP8_BLOCKSCALE = 4
CFG_FP8_MX128 = 5         # microscaling (mxfp8) decode, the first adjacent workload
CFG_BF16_DECODE = 6       # bf16 weights at decode M, the second adjacent workload
CFG_FP4_MX32 = 7          # mxfp4 decode, the fourth adjacent workload

WORKLOADS = {
    "bf16_small": dict(cfg=CFG_BF16_SMALL, dtype="bf16", M=128, N=256, K=256),
    "bf16_large": dict(cfg=CFG_BF16_LARGE, dtype="bf16", M=4096, N=4096, K=8192),
    "fp8_large": dict(cfg=CFG_FP8_LARGE, dtype="fp8", M=4096, N=4096, K=8192),
    "fp8_decode": dict(cfg=CFG_FP8_DECODE, dtype="fp8", Ms=(1, 16), Ns=(2048, 16384), K=7168,
                       splits=(1, 2, 4, 8)),
    "fp8_blockscale": dict(cfg=CFG_FP8_BLOCKSCALE, dtype="fp8", M=16, N=16384, K=7168,
                           splits=(1, 2, 4, 8)),
    "fp8_mx128": dict(cfg=CFG_FP8_MX128, dtype="fp8", M=16, N=16384, K=7168, splits=(1, 2, 4, 8)),
    "bf16_decode": dict(cfg=CFG_BF16_DECODE, dtype="bf16", Ms=(1, 16), Ns=(2048, 16384), K=7168,
                        splits=(1, 2, 4, 8)),
    # fp4 rows of K=7168 are 3584 bytes: split ranges must stay whole 128-byte multiples
    "fp4_mx32": dict(cfg=CFG_FP4_MX32, dtype="fp4", M=16, N=16384, K=7168, splits=(1, 2, 4, 7)),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def seed_of(cfg: int, which: int) -> int:
    """which: 0 = A, 1 = B, 2 = scales."""
    return 1000 * cfg + which


# ----------------------------------------------------------- storage types

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) via torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes (uint8) via torch's conversion.  Callers clamp
    to +-448 first; torch does not saturate."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


E2M1_MAX = 6.0
_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def to_e2m1_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E2M1 codes (uint8, one per element): round to nearest on the
    grid 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code, saturating at 6."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(E2M1_MAX))
    idx = np.searchsorted(_E2M1_MIDS, a, side="left")
    at_mid = (idx < len(_E2M1_MIDS)) & (a == _E2M1_MIDS[np.minimum(idx, len(_E2M1_MIDS) - 1)])
    code = idx + (at_mid & (idx % 2 == 1))
    return (code + 8 * (x < 0)).astype(np.uint8)


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """[rows][K] E2M1 codes -> [rows][K/2] bytes, element 2j in the low nibble."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def quantise_e4m3(x: np.ndarray, scale) -> np.ndarray:
    """codes = e4m3(clamp(x / scale, -448, 448)); scale broadcasts against x."""
    y = np.clip(np.asarray(x, dtype=np.float32) / np.asarray(scale, dtype=np.float32),
                -E4M3_MAX, E4M3_MAX)
    return to_e4m3_codes(y)


# ------------------------------------------------------------- generators

def bf16_uniform(shape, seed, lo=-1.0, hi=1.0) -> np.ndarray:
    return to_bf16_bits(rng(seed).uniform(lo, hi, size=shape).astype(np.float32))


def bf16_normal(shape, seed, std=1.0) -> np.ndarray:
    return to_bf16_bits((rng(seed).standard_normal(size=shape) * std).astype(np.float32))


def fp8_per_tensor(shape, seed):
    """N(0,1) data quantised with the per-tensor scale amax/448.

    Returns (codes uint8, scale float32 array of shape (1,))."""
    x = rng(seed).standard_normal(size=shape).astype(np.float32)
    amax = float(np.max(np.abs(x))) if x.size else 1.0
    s = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    return quantise_e4m3(x, s), np.array([s], dtype=np.float32)


def fp8_blockscale_a(M, K, seed_data, seed_scale):
    """A [M][K] quantised per row per 128-K block; sA [M][K/128]."""
    x = rng(seed_data).standard_normal(size=(M, K)).astype(np.float32)
    kb = K // 128
    amax = np.abs(x.reshape(M, kb, 128)).max(axis=2)
    u = rng(seed_scale).uniform(0.5, 2.0, size=(M, kb)).astype(np.float32)
    s = (u * amax / E4M3_MAX).astype(np.float32)
    s[s == 0] = 1.0
    codes = quantise_e4m3(x.reshape(M, kb, 128), s[:, :, None]).reshape(M, K)
    return codes, s


def fp8_blockscale_b(N, K, seed_data, seed_scale):
    """B [N][K] quantised per 128x128 block; sB [N/128][K/128]."""
    x = rng(seed_data).standard_normal(size=(N, K)).astype(np.float32)
    nb, kb = N // 128, K // 128
    blocks = x.reshape(nb, 128, kb, 128)
    amax = np.abs(blocks).max(axis=(1, 3))
    u = rng(seed_scale).uniform(0.5, 2.0, size=(nb, kb)).astype(np.float32)
    s = (u * amax / E4M3_MAX).astype(np.float32)
    s[s == 0] = 1.0
    codes = quantise_e4m3(blocks, s[:, None, :, None]).reshape(N, K)
    return codes, s


def fp8_mx128(R, K, seed_data, seed_mag):
    """Rows [R][K] in the microscaling format with 128-element blocks: codes
    (e4m3) and one E8M0 byte per row per block ([R][K/128] uint8).

    Data: N(0,1) times a per-block magnitude 2^u, u uniform in {-4..4}, so the
    block scales differ.  Scale rule of the OCP microscaling format: shared
    exponent floor(log2(amax)) - 8 (8 = largest e4m3 exponent), stored biased
    by 127; elements x / 2^(shared exponent), saturated to +-448."""
    kb = K // 128
    x = rng(seed_data).standard_normal(size=(R, kb, 128)).astype(np.float32)
    x *= np.exp2(rng(seed_mag).integers(-4, 5, size=(R, kb, 1))).astype(np.float32)
    amax = np.abs(x).max(axis=2)
    shared = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - 8
    e = np.clip(shared + 127, 0, 254).astype(np.uint8)
    scale = np.exp2(e.astype(np.float64) - 127).astype(np.float32)
    codes = quantise_e4m3(x, scale[:, :, None]).reshape(R, K)
    return codes, e


def fp4_mx32(R, K, seed_data, seed_mag):
    """Rows [R][K] in mxfp4: packed E2M1 bytes [R][K/2] and one E8M0 byte per
    row per 32-element block ([R][K/32]).  Data N(0,1) times a per-block
    magnitude 2^u, u uniform in {-4..4}; scale rule of the OCP microscaling
    format, shared exponent floor(log2(amax)) - 2 (2 = largest E2M1
    exponent), elements saturated to +-6."""
    kb = K // 32
    x = rng(seed_data).standard_normal(size=(R, kb, 32)).astype(np.float32)
    x *= np.exp2(rng(seed_mag).integers(-4, 5, size=(R, kb, 1))).astype(np.float32)
    amax = np.abs(x).max(axis=2)
    shared = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - 2
    e = np.clip(shared + 127, 0, 254).astype(np.uint8)
    scale = np.exp2(e.astype(np.float64) - 127).astype(np.float32)
    codes = to_e2m1_codes(x / scale[:, :, None]).reshape(R, K)
    return pack_e2m1(codes), e


def exact_e8m0_scales(shape, seed) -> np.ndarray:
    """E8M0 bytes from {126, 127, 128} (scales 0.5, 1, 2): exact in every product."""
    return rng(seed).choice(np.array([126, 127, 128], dtype=np.uint8), size=shape)


def exact_ints(shape, seed, dtype: str, lo=-4, hi=4) -> np.ndarray:
    """Uniform integers in [lo, hi], stored exactly as bf16 bits or e4m3 codes.

    Every product and partial sum of such inputs is an exact fp32 number, so
    any summation order gives the same bits."""
    v = rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)
    if dtype == "fp4":    # packed pairs: shape[-1] elements -> shape[-1]/2 bytes
        return pack_e2m1(to_e2m1_codes(v))
    return to_bf16_bits(v) if dtype == "bf16" else to_e4m3_codes(v)


def exact_block_scales(shape, seed) -> np.ndarray:
    """Scales drawn from {0.5, 1, 2}: exact in every product."""
    return rng(seed).choice(np.array([0.5, 1.0, 2.0], dtype=np.float32), size=shape)


def random_block_scales(shape, seed) -> np.ndarray:
    """fp32 scales uniform in [0.5, 2): with exact-integer operands every
    128-K partial sum is exact, and scaling it rounds."""
    return rng(seed).uniform(0.5, 2.0, size=shape).astype(np.float32)


def workload_inputs(name: str, M=None, N=None, K=None):
    """Inputs of a named workload: dict(A, B, sA, sB, dtype, scale_mode, M, N, K).

    ``dtype`` is "bf16" or "fp8"; ``scale_mode`` is "none", "tensor", "block128"
    or "mx128" (E8M0 byte scales, sA [M][K/128], sB [N][K/128]).
    M/N/K override the workload's sizes (used for the decode family)."""
    w = WORKLOADS[name]
    cfg = w["cfg"]
    M = M if M is not None else w.get("M")
    N = N if N is not None else w.get("N")
    K = K if K is not None else w.get("K")
    sa, sb, ss = seed_of(cfg, 0), seed_of(cfg, 1), seed_of(cfg, 2)
    if name == "bf16_small":
        return dict(A=bf16_uniform((M, K), sa), B=bf16_uniform((N, K), sb), sA=None, sB=None,
                    dtype="bf16", scale_mode="none", M=M, N=N, K=K)
    if name in ("bf16_large", "bf16_decode"):
        std = 1.0 / np.sqrt(K)
        return dict(A=bf16_normal((M, K), sa, std), B=bf16_normal((N, K), sb, std), sA=None,
                    sB=None, dtype="bf16", scale_mode="none", M=M, N=N, K=K)
    if name in ("fp8_large", "fp8_decode"):
        A, sA = fp8_per_tensor((M, K), sa)
        B, sB = fp8_per_tensor((N, K), sb)
        return dict(A=A, B=B, sA=sA, sB=sB, dtype="fp8", scale_mode="tensor", M=M, N=N, K=K)
    if name == "fp8_blockscale":
        A, sA = fp8_blockscale_a(M, K, sa, ss)
        B, sB = fp8_blockscale_b(N, K, sb, ss + 500)
        return dict(A=A, B=B, sA=sA, sB=sB, dtype="fp8", scale_mode="block128", M=M, N=N, K=K)
    if name == "fp4_mx32":
        A, sA = fp4_mx32(M, K, sa, ss)
        B, sB = fp4_mx32(N, K, sb, ss + 500)
        return dict(A=A, B=B, sA=sA, sB=sB, dtype="fp4", scale_mode="mx32", M=M, N=N, K=K)
    if name == "fp8_mx128":
        A, sA = fp8_mx128(M, K, sa, ss)
        B, sB = fp8_mx128(N, K, sb, ss + 500)
        return dict(A=A, B=B, sA=sA, sB=sB, dtype="fp8", scale_mode="mx128", M=M, N=N, K=K)
    raise KeyError(name)
