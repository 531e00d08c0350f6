"""Python binding of the gfx950 preshuffled-B GEMM library (libdgp.so).

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in include/dgp.h.  torch supplies device memory (outputs
are allocated as torch tensors when not given) and the stream (the current
torch stream unless one is passed).  There is no fallback: if the compiled
library is missing, every call raises.

Element types follow the torch dtype of the operands: torch.bfloat16 ->
DGP_BF16, torch.float8_e4m3fn -> DGP_FP8_E4M3, torch.float4_e2m1fn_x2 (two
E2M1 values per byte; a [rows][K/2] tensor holds K elements per row) ->
DGP_FP4_E2M1.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgp.so")
# The LDS-poison debug build of the same sources (see lds_poison_build).
LDS_POISON_LIB_PATH = os.path.join(_HERE, "libdgp_lds_poison.so")

BF16 = 0
FP8_E4M3 = 1
FP4_E2M1 = 2
SCALE_NONE = 0
SCALE_TENSOR = 1
SCALE_BLOCK128 = 2
SCALE_MX128 = 3
SCALE_MX32 = 4

STATUS = {0: "DGP_OK", 1: "DGP_ERR_NULL", 2: "DGP_ERR_SHAPE", 3: "DGP_ERR_ALIGN", 4: "DGP_ERR_DTYPE",
          5: "DGP_ERR_SCALE_MODE", 6: "DGP_ERR_SPLITK", 7: "DGP_ERR_WORKSPACE", 8: "DGP_ERR_CONFIG",
          9: "DGP_ERR_ARCH", 10: "DGP_ERR_HIP"}


class DgpError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.name}: {message}")


class Config(ctypes.Structure):
    """dgp_config: tile_m/tile_n/tile_k, xcd_remap, group_m, preload pair, waves_m, prefetch, schedule,
    a_layout, a_copy."""
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("xcd_remap", ctypes.c_int), ("group_m", ctypes.c_int),
                ("preload_vmem", ctypes.c_int), ("preload_dsrd", ctypes.c_int),
                ("waves_m", ctypes.c_int), ("prefetch", ctypes.c_int), ("schedule", ctypes.c_int),
                ("a_layout", ctypes.c_int), ("a_copy", ctypes.c_int)]


# Every symbol include/dgp.h and include/dgp_diag.h declare.
EXPORTS = ("dgp_preshuffle_b", "dgp_unshuffle_b", "dgp_gemm_preshuffle", "dgp_splitk_workspace_bytes",
           "dgp_gemm_preshuffle_splitk", "dgp_gemm_preshuffle_splitk_noalloc", "dgp_check_arch", "dgp_status_string", "dgp_last_error",
           "dgp_tile_of_workgroup", "dgp_tile_map", "dgp_kernel_count", "dgp_kernel_info", "dgp_select_kernel",
           "dgp_probe_mfma_layout", "dgp_probe_mfma_scaled", "dgp_probe_lds_dma", "dgp_probe_lds_dma_narrow", "dgp_probe_copy",
           "dgp_probe_stream_read", "dgp_probe_mfma_peak", "dgp_lds_poison")

_lib = None
_loaded = {}                 # path -> CDLL
_swap = threading.Lock()     # serialises lds_poison_build's switch of the active library
_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The active library: libdgp.so unless inside lds_poison_build().  Raises
    if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def lds_poison_build():
    """Run every call made inside the block on the LDS-poison debug build
    (libdgp_lds_poison.so, built beside libdgp.so by the same build step): the
    same entry points and kernels, with each kernel's LDS filled with 0xFF
    bytes before use and each global -> LDS copy's destination poisoned until
    the copy lands, so a read of LDS no copy filled shows up as NaN or a wrong
    value in a bit-exact comparison.  For tests; the switch is process-wide
    (one block at a time)."""
    global _lib
    with _swap:
        saved = lib()
        poison = _load(LDS_POISON_LIB_PATH)
        if poison.dgp_lds_poison() != 1:
            raise ImportError(f"{LDS_POISON_LIB_PATH} is not an LDS-poison build")
        _lib = poison
        try:
            yield poison
        finally:
            _lib = saved


def _load(path: str) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(or python dense_gemm_packer_amd/build.py)")
    L = ctypes.CDLL(path)
    sigs = {
        "dgp_preshuffle_b": [_vp, _vp, _i64, _i64, _int, _vp],
        "dgp_unshuffle_b": [_vp, _vp, _i64, _i64, _int, _vp],
        "dgp_gemm_preshuffle": [_vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp],
        "dgp_gemm_preshuffle_splitk": [_vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _int, _vp,
                                       _sz, _vp, _vp],
        "dgp_gemm_preshuffle_splitk_noalloc": [_vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _vp, _int,
                                               _vp, _vp],
        "dgp_check_arch": [ctypes.c_char_p],
        "dgp_tile_of_workgroup": [_i64, _i64, _i64, _i64, _int, _int, ctypes.POINTER(_i64)],
        "dgp_tile_map": [_i64, _i64, _i64, _int, _int, _vp, _i64],
        "dgp_kernel_count": [],
        "dgp_kernel_info": [_int, ctypes.POINTER(Config), ctypes.POINTER(_int), ctypes.POINTER(_int),
                            ctypes.POINTER(_int)],
        "dgp_select_kernel": [_i64, _i64, _i64, _int, _int, _int, ctypes.POINTER(Config), ctypes.POINTER(_int)],
        "dgp_probe_mfma_layout": [_int, _vp, _vp, _vp, _vp],
        "dgp_probe_lds_dma": [_vp, _vp, _vp, _vp],
        "dgp_probe_lds_dma_narrow": [_int, _vp, _vp, _vp, _vp],
        "dgp_probe_mfma_scaled": [_int, _vp, _vp, _vp, _vp, _vp, _vp],
        "dgp_probe_copy": [_vp, _vp, _i64, _vp],
        "dgp_probe_stream_read": [_vp, _i64, _int, _vp, _vp],
        "dgp_probe_mfma_peak": [_int, _int, _int, _vp, _vp, _vp],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = _int
    L.dgp_splitk_workspace_bytes.argtypes = [_i64, _i64, _int]
    L.dgp_splitk_workspace_bytes.restype = _sz
    L.dgp_status_string.argtypes = [_int]
    L.dgp_status_string.restype = ctypes.c_char_p
    L.dgp_last_error.argtypes = []
    L.dgp_last_error.restype = ctypes.c_char_p
    L.dgp_lds_poison.argtypes = []
    L.dgp_lds_poison.restype = _int
    _loaded[path] = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise DgpError(status, lib().dgp_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    if t.dtype == torch.float4_e2m1fn_x2:
        return FP4_E2M1
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16, float8_e4m3fn or float4_e2m1fn_x2)")


def k_elements(t: torch.Tensor) -> int:
    """Elements per row of a [rows][...] operand (fp4 stores two per byte)."""
    return t.shape[1] * (2 if t.dtype == torch.float4_e2m1fn_x2 else 1)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _same_device(ref: torch.Tensor, *named):
    for t, what in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{what} is on {t.device}, A on {ref.device}")


# Scale tensors per mode: (dtype, numel of sA, numel of sB) for an M x N x K
# call, or None where K or N breaks the mode's divisibility rule (the C ABI
# then rejects the call with its own status).
def scale_shapes(mode: int, M: int, N: int, K: int):
    if mode == SCALE_NONE:
        return None
    if mode == SCALE_TENSOR:
        return torch.float32, 1, 1
    if mode == SCALE_BLOCK128:
        if K % 128 or N % 128:
            return None
        return torch.float32, M * (K // 128), (N // 128) * (K // 128)
    if mode == SCALE_MX128:
        if K % 128:
            return None
        return torch.uint8, M * (K // 128), N * (K // 128)
    if mode == SCALE_MX32:
        if K % 32:
            return None
        return torch.uint8, M * (K // 32), N * (K // 32)
    return None


def check_gemm_operands(A: torch.Tensor, Bs: torch.Tensor, sA, sB, mode: int, out) -> None:
    """Shape and dtype checks the C ABI cannot make (it sees pointers only):
    a buffer smaller than the call assumes would be read or written past its
    end.  Raises ValueError; device-independent, so it runs before any
    launch."""
    if A.dim() != 2 or Bs.dim() != 2:
        raise ValueError(f"A and Bs must be 2-D (got {A.dim()}-D and {Bs.dim()}-D)")
    if Bs.dtype != A.dtype:
        raise ValueError(f"Bs is {Bs.dtype}, A is {A.dtype}: both operands take one element type")
    M, K, N = A.shape[0], k_elements(A), Bs.shape[0]
    if k_elements(Bs) != K:
        raise ValueError(f"Bs holds {k_elements(Bs)} elements per row, A {K}")
    if out is not None:
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N):
            raise ValueError(f"out must be a ({M}, {N}) bfloat16 tensor (got {tuple(out.shape)} {out.dtype})")
    want = scale_shapes(mode, M, N, K)
    if want is None:
        return
    dt, na, nb = want
    for t, n, what in ((sA, na, "sA"), (sB, nb, "sB")):
        if t is None:
            continue   # a missing scale is the C ABI's DGP_ERR_NULL
        if t.dtype != dt or t.numel() != n:
            raise ValueError(f"{what} must hold {n} {dt} values for this scale mode and shape "
                             f"(got {t.numel()} {t.dtype})")


def _alloc_stream(stream):
    """Context in which outputs and workspaces are allocated: the launch
    stream, so the caching allocator never hands their memory to other work
    while the kernels that use it are still queued there."""
    import contextlib
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _config(config):
    if config is None:
        return None
    if isinstance(config, Config):
        return ctypes.byref(config)
    return ctypes.byref(Config(**config))


# -------------------------------------------------------------- entry points

def preshuffle_b(B: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Bs = dgp_preshuffle_b(B); B is [N][K] bf16 or e4m3, on the device."""
    _dev(B, "B")
    if B.dim() != 2:
        raise ValueError(f"B must be 2-D (got {B.dim()}-D)")
    if out is None:
        with _alloc_stream(stream):
            out = torch.empty_like(B)
    _dev(out, "out")
    if out.dtype != B.dtype or out.shape != B.shape:
        raise ValueError(f"out must match B ({tuple(B.shape)} {B.dtype}), got {tuple(out.shape)} {out.dtype}")
    _same_device(B, (out, "out"))
    _check(lib().dgp_preshuffle_b(_ptr(B), _ptr(out), B.shape[0], k_elements(B), dtype_code(B),
                                  _stream_handle(stream)))
    return out


def unshuffle_b(Bs: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev(Bs, "Bs")
    if Bs.dim() != 2:
        raise ValueError(f"Bs must be 2-D (got {Bs.dim()}-D)")
    if out is None:
        with _alloc_stream(stream):
            out = torch.empty_like(Bs)
    _dev(out, "out")
    if out.dtype != Bs.dtype or out.shape != Bs.shape:
        raise ValueError(f"out must match Bs ({tuple(Bs.shape)} {Bs.dtype}), got {tuple(out.shape)} {out.dtype}")
    _same_device(Bs, (out, "out"))
    _check(lib().dgp_unshuffle_b(_ptr(Bs), _ptr(out), Bs.shape[0], k_elements(Bs), dtype_code(Bs),
                                 _stream_handle(stream)))
    return out


def _scale_mode(A, sA, sB, scale_mode):
    """The scale mode of a call: given, or inferred from the scales (none for
    bf16; mxfp4 for fp4; uint8 E8M0 scales -> mxfp8; one fp32 in each of sA
    and sB -> per-tensor; more in both -> blockscale).  A one-element sA with
    a larger sB is ambiguous (blockscale with M = 1 and K = 128 has a
    one-element sA too) and must name its mode."""
    if scale_mode is not None:
        return scale_mode
    if dtype_code(A) == BF16:
        return SCALE_NONE
    if dtype_code(A) == FP4_E2M1:
        return SCALE_MX32
    if sA is not None and sA.dtype == torch.uint8:
        return SCALE_MX128
    if sA is None or sB is None:
        return SCALE_TENSOR   # the C ABI rejects the missing scale
    if sA.numel() == 1 and sB.numel() == 1:
        return SCALE_TENSOR
    if sA.numel() > 1 and sB.numel() > 1:
        return SCALE_BLOCK128
    raise ValueError("ambiguous fp8 scales (one of sA, sB holds a single value, the other more): "
                     "pass scale_mode=SCALE_TENSOR or SCALE_BLOCK128")


def gemm_preshuffle(A: torch.Tensor, Bs: torch.Tensor, sA: torch.Tensor | None = None,
                    sB: torch.Tensor | None = None, scale_mode: int | None = None,
                    out: torch.Tensor | None = None, config=None, stream=None) -> torch.Tensor:
    """C = A * B^T (bf16 [M][N]) with Bs = preshuffle_b(B)."""
    _dev(A, "A"), _dev(Bs, "Bs")
    for s, name in ((sA, "sA"), (sB, "sB"), (out, "out")):
        if s is not None:
            _dev(s, name)
    _same_device(A, (Bs, "Bs"), (sA, "sA"), (sB, "sB"), (out, "out"))
    mode = _scale_mode(A, sA, sB, scale_mode)
    check_gemm_operands(A, Bs, sA, sB, mode, out)
    M, K = A.shape[0], k_elements(A)
    N = Bs.shape[0]
    if out is None:
        with _alloc_stream(stream):
            out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _check(lib().dgp_gemm_preshuffle(_ptr(A), _ptr(Bs), _ptr(out), M, N, K, dtype_code(A), mode,
                                     _ptr(sA), _ptr(sB), _config(config), _stream_handle(stream)))
    return out


def splitk_workspace_bytes(M: int, N: int, split_k: int) -> int:
    return int(lib().dgp_splitk_workspace_bytes(M, N, split_k))


def gemm_preshuffle_splitk(A: torch.Tensor, Bs: torch.Tensor, split_k: int,
                           sA: torch.Tensor | None = None, sB: torch.Tensor | None = None,
                           scale_mode: int | None = None, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, config=None,
                           stream=None) -> torch.Tensor:
    """Two-pass split-K C = A * B^T; workspace (fp32) is allocated if not given
    (on the launch stream; it is freed on return, and the caching allocator
    reuses it only for work queued behind this call on that stream)."""
    _dev(A, "A"), _dev(Bs, "Bs")
    for s, name in ((sA, "sA"), (sB, "sB"), (out, "out"), (workspace, "workspace")):
        if s is not None:
            _dev(s, name)
    _same_device(A, (Bs, "Bs"), (sA, "sA"), (sB, "sB"), (out, "out"), (workspace, "workspace"))
    if workspace is not None and workspace.dtype != torch.float32:
        raise ValueError(f"workspace must be float32 (got {workspace.dtype})")
    mode = _scale_mode(A, sA, sB, scale_mode)
    check_gemm_operands(A, Bs, sA, sB, mode, out)
    M, K = A.shape[0], k_elements(A)
    N = Bs.shape[0]
    need = splitk_workspace_bytes(M, N, split_k)
    with _alloc_stream(stream):
        if out is None:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
        if workspace is None and need > 0:
            workspace = torch.empty(need // 4, dtype=torch.float32, device=A.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dgp_gemm_preshuffle_splitk(_ptr(A), _ptr(Bs), _ptr(out), M, N, K, dtype_code(A), mode,
                                            _ptr(sA), _ptr(sB), split_k, _ptr(workspace), ws_bytes,
                                            _config(config), _stream_handle(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20   # DGP_NOALLOC_SCRATCH_BYTES


def gemm_preshuffle_splitk_noalloc(A: torch.Tensor, Bs: torch.Tensor, split_k: int, out: torch.Tensor,
                                   sA: torch.Tensor | None = None, sB: torch.Tensor | None = None,
                                   scale_mode: int | None = None, config=None, stream=None) -> torch.Tensor:
    """Two-pass split-K C = A * B^T whose fp32 partials go to the library's
    fixed per-GPU scratch (dgp_gemm_preshuffle_splitk_noalloc): nothing is
    allocated, the caller passes `out`.  Calls that overlap on one GPU race on
    that scratch."""
    _dev(A, "A"), _dev(Bs, "Bs"), _dev(out, "out")
    for s, name in ((sA, "sA"), (sB, "sB")):
        if s is not None:
            _dev(s, name)
    _same_device(A, (Bs, "Bs"), (sA, "sA"), (sB, "sB"), (out, "out"))
    mode = _scale_mode(A, sA, sB, scale_mode)
    check_gemm_operands(A, Bs, sA, sB, mode, out)
    M, K = A.shape[0], k_elements(A)
    N = Bs.shape[0]
    _check(lib().dgp_gemm_preshuffle_splitk_noalloc(_ptr(A), _ptr(Bs), _ptr(out), M, N, K, dtype_code(A), mode,
                                                    _ptr(sA), _ptr(sB), split_k, _config(config),
                                                    _stream_handle(stream)))
    return out


def check_arch(name: str) -> bool:
    return lib().dgp_check_arch(name.encode()) == 0


def status_string(status: int) -> str:
    return lib().dgp_status_string(status).decode()


# ---------------------------------------------------------------- diagnostics

def tile_of_workgroup(wg: int, tiles_m: int, tiles_n: int, splits: int, xcd_remap: int, group_m: int):
    out = (ctypes.c_int64 * 3)()
    _check(lib().dgp_tile_of_workgroup(wg, tiles_m, tiles_n, splits, xcd_remap, group_m, out))
    return int(out[0]), int(out[1]), int(out[2])


def tile_map(tiles_m: int, tiles_n: int, splits: int, xcd_remap: int, group_m: int):
    """(tile_m, tile_n, split) of every workgroup of the grid: an int64 numpy array [W][3]."""
    import numpy as np
    out = np.empty((tiles_m * tiles_n * splits, 3), dtype=np.int64)
    _check(lib().dgp_tile_map(tiles_m, tiles_n, splits, xcd_remap, group_m, out.ctypes.data, out.size))
    return out


def kernels():
    """Every compiled GEMM kernel: list of (Config, dtype, scale_mode, split_out)."""
    L = lib()
    out = []
    for i in range(L.dgp_kernel_count()):
        cfg, dt, sm, so = Config(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(L.dgp_kernel_info(i, ctypes.byref(cfg), ctypes.byref(dt), ctypes.byref(sm), ctypes.byref(so)))
        out.append((cfg, dt.value, sm.value, so.value))
    return out


def select_kernel(M: int, N: int, K: int, dtype: int, scale_mode: int, split_k: int = 1, config=None) -> int:
    """Table index of the GEMM kernel such a call would launch (-1: none)."""
    idx = ctypes.c_int()
    cfg = None if config is None else (config if isinstance(config, Config) else Config(**config))
    _check(lib().dgp_select_kernel(M, N, K, dtype, scale_mode, split_k,
                                   None if cfg is None else ctypes.byref(cfg), ctypes.byref(idx)))
    return idx.value


def describe_kernel(index: int) -> str:
    """One-line description of compiled kernel `index`."""
    cfg, dt, sm, so = kernels()[index]
    dts = {BF16: "bf16", FP8_E4M3: "fp8", FP4_E2M1: "fp4"}[dt]
    # the K-split tiles run 8 waves per workgroup (16 for a bf16 tile and three
    # mxfp4 tiles), the streaming tiles 2 or 4
    if cfg.tile_m == 16 and (cfg.tile_n in (8, 16) or cfg.waves_m in (8, 16)):
        half = ", half a strip" if cfg.tile_n == 8 else ""
        return (f"gemm_ksplit_kernel<{dts}, 16x{cfg.tile_n} tile{half}, K split over {cfg.waves_m} waves, "
                f"{cfg.prefetch}-step ring{', fp32 partials' if so else ''}>")
    if cfg.tile_m == 1:
        half = ", half a strip" if cfg.tile_n == 8 else ""
        return (f"gemm_wave_kernel<{dts}, 1x{cfg.tile_n} tile{half}, VALU dot products, K split over "
                f"{cfg.waves_m} waves, {cfg.prefetch}-step ring{', fp32 partials' if so else ''}>")
    if cfg.tile_m == 16:
        return (f"gemm_stream_kernel<{dts}, 16x{cfg.tile_n} tile, {cfg.waves_m} waves, "
                f"{cfg.prefetch}-step ring{', fp32 partials' if so else ''}>")
    sched = {1: f"interleaved, LDS read-ahead {cfg.preload_dsrd}", 2: "ping-pong",
             3: f"A and B in LDS, LDS read-ahead {cfg.preload_dsrd}",
             4: f"4 waves (1 per SIMD{', 2x2' if cfg.waves_m == 2 else ''}"
                f"{', up to 2 workgroups per CU' if cfg.tile_m == 128 else ''}), AGPR accumulators, "
                f"LDS read-ahead {cfg.preload_dsrd}, "
                f"{'interleaved' if cfg.preload_vmem else 'bunched'} issue"}[cfg.schedule]
    lay = {1: "A in operand blocks", 2: "A in swizzled rows"}.get(cfg.a_layout, "")
    sched = f"{sched}, {lay}" if cfg.schedule == 4 and lay else sched
    if cfg.a_copy == 2:
        sched += ", A copied through registers"
    kname = {1: "tiled", 2: "pingpong", 3: "lds", 4: "w4"}[cfg.schedule]
    return (f"gemm_{kname}_kernel<{dts}, {cfg.tile_m}x{cfg.tile_n} tile, "
            f"{cfg.tile_k}-byte k-tile, waves_m {cfg.waves_m}, prefetch {cfg.prefetch}, {sched}"
            f"{', fp32 partials' if so else ''}>")


def probe_mfma_layout(which: int, a: torch.Tensor, b: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty(64 * 4, dtype=torch.float32, device=a.device)
    _check(lib().dgp_probe_mfma_layout(which, _ptr(a), _ptr(b), _ptr(out), _stream_handle(stream)))
    return out.view(64, 4)


def probe_mfma_scaled(a: torch.Tensor, b: torch.Tensor, sa: torch.Tensor, sb: torch.Tensor,
                      which: int = 0, stream=None) -> torch.Tensor:
    out = torch.empty(64 * 4, dtype=torch.float32, device=a.device)
    _check(lib().dgp_probe_mfma_scaled(which, _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), _ptr(out),
                                       _stream_handle(stream)))
    return out.view(64, 4)


def probe_lds_dma(src: torch.Tensor, perm: torch.Tensor, stream=None) -> torch.Tensor:
    dst = torch.empty(1024, dtype=torch.uint8, device=src.device)
    _check(lib().dgp_probe_lds_dma(_ptr(src), _ptr(perm), _ptr(dst), _stream_handle(stream)))
    return dst


def probe_lds_dma_narrow(width: int, src: torch.Tensor, perm: torch.Tensor, stream=None) -> torch.Tensor:
    dst = torch.empty(1024, dtype=torch.uint8, device=src.device)
    _check(lib().dgp_probe_lds_dma_narrow(width, _ptr(src), _ptr(perm), _ptr(dst), _stream_handle(stream)))
    return dst


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    _check(lib().dgp_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream_handle(stream)))


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor, blocks: int = 1024, nbytes: int | None = None,
                      stream=None) -> None:
    """Read the first `nbytes` (default: all) bytes of src with `blocks`
    workgroups, each streaming one contiguous span."""
    total = src.numel() * src.element_size()
    nbytes = total if nbytes is None else nbytes
    if nbytes > total:
        raise ValueError(f"nbytes {nbytes} exceeds the buffer ({total} bytes)")
    _check(lib().dgp_probe_stream_read(_ptr(src), nbytes, blocks, _ptr(sink), _stream_handle(stream)))


# FLOP per matrix-core instruction of dgp_probe_mfma_peak (which = 0 bf16,
# 1 e4m3, 2 E2M1), and the operand buffer it reads (256 sets x 16 fragments
# x 64 lanes x 16|32|16 B).
MFMA_PEAK_FLOP = (16384, 65536, 65536)
MFMA_PEAK_OPERAND_BYTES = (256 * 16 * 64 * 16, 256 * 16 * 64 * 32, 256 * 16 * 64 * 16)


def probe_mfma_peak(which: int, rounds: int, blocks: int, operands: torch.Tensor, sink: torch.Tensor,
                    stream=None) -> int:
    """Launch the register-only MFMA loop on `operands`; returns the FLOP it performs."""
    _dev(operands, "operands")
    if which not in (0, 1, 2):
        raise ValueError("which must be 0, 1 or 2")
    if operands.numel() * operands.element_size() < MFMA_PEAK_OPERAND_BYTES[which]:
        raise ValueError(f"operands must hold {MFMA_PEAK_OPERAND_BYTES[which]} bytes")
    _check(lib().dgp_probe_mfma_peak(which, rounds, blocks, _ptr(operands), _ptr(sink), _stream_handle(stream)))
    return blocks * 4 * rounds * 64 * MFMA_PEAK_FLOP[which]
