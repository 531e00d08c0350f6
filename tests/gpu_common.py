"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the library through its C ABI (via the binding) and compare with the
oracle."""
import numpy as np
import torch

import dense_gemm_packer_amd as dgp
import oracle

DEV = "cuda:0"


def dev_codes(codes: np.ndarray, dtype: str) -> torch.Tensor:
    """bf16 bit patterns (uint16), e4m3 codes (uint8) or packed e2m1 pairs
    (uint8, [rows][K/2]) -> device tensor of the matching torch type."""
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16 if dtype == "bf16" else np.uint8).copy())
    t = t.view({"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "fp4": torch.float4_e2m1fn_x2}[dtype])
    return t.to(DEV)


def dev_f32(x) -> torch.Tensor | None:
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to(DEV)


def dev_scales(x, mode: str) -> torch.Tensor | None:
    """Scales to the device: E8M0 bytes for mx128, fp32 otherwise."""
    if x is None:
        return None
    if mode in ("mx128", "mx32"):
        return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.uint8))).to(DEV)
    return dev_f32(x)


def host_bits(c: torch.Tensor) -> np.ndarray:
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def odt(dtype: str) -> int:
    return {"bf16": oracle.BF16, "fp8": oracle.FP8_E4M3, "fp4": oracle.FP4_E2M1}[dtype]


def omode(mode: str) -> int:
    return {"none": oracle.SCALE_NONE, "tensor": oracle.SCALE_TENSOR, "block128": oracle.SCALE_BLOCK128,
            "mx128": oracle.SCALE_MX128, "mx32": oracle.SCALE_MX32}[mode]


def dmode(mode: str) -> int:
    return {"none": dgp.SCALE_NONE, "tensor": dgp.SCALE_TENSOR, "block128": dgp.SCALE_BLOCK128,
            "mx128": dgp.SCALE_MX128, "mx32": dgp.SCALE_MX32}[mode]


def run_gpu(A, B, dtype, mode, sA=None, sB=None, split_k=1, config=None, Bs_dev=None):
    """Preshuffle B and run the GEMM on the device; returns C as bf16 bits."""
    a = dev_codes(A, dtype)
    if Bs_dev is None:
        Bs_dev = dgp.preshuffle_b(dev_codes(B, dtype))
    if split_k == 1 and config is None:
        c = dgp.gemm_preshuffle(a, Bs_dev, dev_scales(sA, mode), dev_scales(sB, mode), dmode(mode))
    else:
        c = dgp.gemm_preshuffle_splitk(a, Bs_dev, split_k, dev_scales(sA, mode), dev_scales(sB, mode),
                                       dmode(mode), config=config)
    torch.cuda.synchronize()
    return host_bits(c)


def run_oracle(A, B, dtype, mode, sA=None, sB=None, split_k=1, rows=None):
    return oracle.gemm(A, B, odt(dtype), omode(mode), sA, sB, split_k=split_k, rows=rows)


def assert_close(c_gpu_bits, c_ref_f32, tol=1e-2, what=""):
    """max |C_gpu - C_ref| <= tol * max |C_ref| (bf16 output vs fp32 oracle)."""
    g = bf16_to_f32(c_gpu_bits).astype(np.float64)
    r = c_ref_f32.astype(np.float64)
    assert g.shape == r.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    bound = tol * max(np.max(np.abs(r)), 1e-30)
    err = np.max(np.abs(g - r)) if g.size else 0.0
    assert err <= bound, f"{what}: max err {err:.4g} > {bound:.4g}"
    return err / max(np.max(np.abs(r)), 1e-30)
