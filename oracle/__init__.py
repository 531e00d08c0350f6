"""CPU oracle for the preshuffled-B GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it and shares no code with it.

Thin ctypes wrappers over ``oracle.c``; see that file for what each function
computes and which passage of the pages it follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16 = 0
FP8_E4M3 = 1
FP4_E2M1 = 2
SCALE_NONE = 0
SCALE_TENSOR = 1
SCALE_BLOCK128 = 2
SCALE_MX128 = 3
SCALE_MX32 = 4

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_bf16_decode.restype = ctypes.c_float
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_decode.restype = ctypes.c_float
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_decode.restype = ctypes.c_float
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [ctypes.c_float]
        for name in ("oracle_preshuffle_b", "oracle_unshuffle_b"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        L.oracle_gemm_rows.restype = ctypes.c_int
        L.oracle_gemm_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int]
        L.oracle_default_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def elem_bytes(dtype):
    return 2 if dtype == BF16 else 1


def bf16_decode(h):
    return lib().oracle_bf16_decode(int(h))


def e4m3_decode(b):
    return lib().oracle_e4m3_decode(int(b))


def e2m1_decode(nibble):
    return lib().oracle_e2m1_decode(int(nibble))


def e8m0_decode(e):
    return lib().oracle_e8m0_decode(int(e))


def bf16_round(f):
    return lib().oracle_bf16_round(float(f))


def decode_array(codes, dtype):
    """Decode a numpy array of bf16 bit patterns (uint16) or e4m3 codes (uint8)."""
    flat = np.ascontiguousarray(codes).reshape(-1)
    f = lib().oracle_bf16_decode if dtype == BF16 else lib().oracle_e4m3_decode
    out = np.fromiter((f(int(v)) for v in flat), dtype=np.float32, count=flat.size)
    return out.reshape(np.shape(codes))


def preshuffle_b(B):
    """Preshuffle B ([N][K] of uint16 bf16 patterns or uint8 e4m3 codes).

    Returns an array of the same dtype and shape holding the permuted bytes.
    """
    B = np.ascontiguousarray(B)
    N = B.shape[0]
    kb = B.shape[1] * B.itemsize
    out = np.empty_like(B)
    rc = lib().oracle_preshuffle_b(_ptr(B), _ptr(out), N, kb)
    if rc != 0:
        raise ValueError("oracle_preshuffle_b: N must be a multiple of 16 and K*bytes a multiple of 64")
    return out


def unshuffle_b(Bs):
    Bs = np.ascontiguousarray(Bs)
    N = Bs.shape[0]
    kb = Bs.shape[1] * Bs.itemsize
    out = np.empty_like(Bs)
    rc = lib().oracle_unshuffle_b(_ptr(Bs), _ptr(out), N, kb)
    if rc != 0:
        raise ValueError("oracle_unshuffle_b: N must be a multiple of 16 and K*bytes a multiple of 64")
    return out


def gemm(A, B, dtype, scale_mode=SCALE_NONE, sA=None, sB=None, split_k=1, rows=None,
         want_partials=False, nthreads=0):
    """C = A * B^T on unshuffled B.

    Scales: per-tensor and blockscale take fp32 arrays; mxfp8 (SCALE_MX128)
    takes E8M0 bytes, sA [M][K/128] and sB [N][K/128]; mxfp4 (FP4_E2M1 with
    SCALE_MX32) takes A and B as packed bytes [rows][K/2] and E8M0 bytes
    sA [M][K/32], sB [N][K/32].

    Returns (c_f32, c_bf16[, partials]): the fp32 value before rounding, the
    bf16 bit patterns, and (optionally) the per-split fp32 partials
    [split_k][nrows][N].  ``rows`` selects rows of C (default: all).
    """
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    if dtype == FP4_E2M1:    # packed pairs: the arrays hold K/2 bytes per row
        K *= 2
    sdt = np.uint8 if scale_mode in (SCALE_MX128, SCALE_MX32) else np.float32   # E8M0 bytes or fp32
    sA_ = None if sA is None else np.ascontiguousarray(np.asarray(sA, dtype=sdt))
    sB_ = None if sB is None else np.ascontiguousarray(np.asarray(sB, dtype=sdt))
    rows_ = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nrows = M if rows_ is None else rows_.size
    c32 = np.empty((nrows, N), dtype=np.float32)
    c16 = np.empty((nrows, N), dtype=np.uint16)
    parts = np.empty((split_k, nrows, N), dtype=np.float32) if want_partials else None
    rc = lib().oracle_gemm_rows(_ptr(A), _ptr(B), M, N, K, dtype, scale_mode, _ptr(sA_), _ptr(sB_),
                                split_k, _ptr(rows_), nrows, _ptr(c32), _ptr(c16), _ptr(parts),
                                nthreads)
    if rc != 0:
        raise ValueError("oracle_gemm_rows rejected its arguments")
    if want_partials:
        return c32, c16, parts
    return c32, c16


def default_threads():
    return lib().oracle_default_threads()
