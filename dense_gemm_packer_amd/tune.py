"""Kernel sweep: time every compiled GEMM kernel that accepts a shape.

    python -m dense_gemm_packer_amd.tune [--shapes SPEC ...] [--iters N]

SPEC is dtype:MxNxK[:split] with dtype one of bf16, fp8 (per-tensor scales),
fp8b (blockscale), mx8 (mxfp8), mx4 (mxfp4); the default list is the
headline shapes and the decode shapes.  For each shape every kernel of the
compiled table with the shape's element type and scale mode is forced through
its reported configuration (`kernels()`), skipped if the library rejects the
shape for it, and timed in a HIP graph; decode-sized shapes (M <= 32) are
timed cold, rotating copies of B whose total exceeds twice the 256 MiB
last-level cache, large-M shapes warm.  The chip's clock ramps under load,
so the built-in choice runs for a warm-up first and every kernel is timed in
two passes, keeping the faster.  One JSON line per shape goes to stdout: the
timings and the kernel the built-in selection (`select_kernel` without a configuration) picks, so a
change of that table can be checked against measurement.  The inputs are
random bytes of the right type (timing does not depend on their values
beyond the matrix units' power draw, which the headline benchmark measures
on its real data).

The built-in per-shape selection in the C library is a static table of rules
(no runtime tuning); this tool is how its entries are chosen.
"""
from __future__ import annotations

import argparse
import json
import sys

import torch

from . import (BF16, FP4_E2M1, FP8_E4M3, SCALE_BLOCK128, SCALE_MX32, SCALE_MX128, SCALE_NONE,
               SCALE_TENSOR, DgpError, describe_kernel, gemm_preshuffle_splitk, kernels, preshuffle_b,
               select_kernel, splitk_workspace_bytes)

LLC_BYTES = 256 << 20
# The headline shapes, bf16 and per-tensor fp8 at 2048 x 4096 and 4096 x 6144
# (the 128-row large-M tile's range: one tile per CU, and two at once), then
# the decode grid (K = 7168): bf16 and per-tensor
# fp8 at M = 1, 4, 16, N = 2048 and 16384, 1, 2 and 4 splits; blockscale and
# mxfp8 at M = 1 and 16 with 1 and 4 splits; mxfp4 at M = 1 and 16 with 1
# and 2 splits.
DEFAULT_SHAPES = (["bf16:4096x4096x8192", "fp8:4096x4096x8192", "fp8b:4096x4096x8192", "mx8:4096x4096x8192",
                   "mx4:4096x4096x8192", "bf16:2048x4096x8192", "fp8:2048x4096x8192", "bf16:4096x6144x8192",
                   "fp8:4096x6144x8192"]
                  + [f"{k}:{m}x{n}x7168:{s}" for k in ("bf16", "fp8") for m in (1, 4, 16) for n in (2048, 16384)
                     for s in (1, 2, 4)]
                  + [f"{k}:{m}x{n}x7168:{s}" for k in ("fp8b", "mx8") for m in (1, 16) for n in (2048, 16384)
                     for s in (1, 4)]
                  + [f"mx4:{m}x{n}x7168:{s}" for m in (1, 16) for n in (2048, 16384) for s in (1, 2)])
MODES = {"bf16": (BF16, SCALE_NONE), "fp8": (FP8_E4M3, SCALE_TENSOR), "fp8b": (FP8_E4M3, SCALE_BLOCK128),
         "mx8": (FP8_E4M3, SCALE_MX128), "mx4": (FP4_E2M1, SCALE_MX32)}


def parse(spec: str):
    parts = spec.split(":")
    dt, sm = MODES[parts[0]]
    M, N, K = (int(x) for x in parts[1].split("x"))
    split = int(parts[2]) if len(parts) > 2 else 1
    return parts[0], dt, sm, M, N, K, split


def operands(kind, dt, sm, M, N, K, dev, gen):
    """Random operands of the shape: A, B (unshuffled), sA, sB."""
    def codes(rows, cols):
        if dt == BF16:   # finite bf16: random sign/mantissa, exponent near 1
            x = torch.randn(rows, cols, generator=gen, device="cpu") / 64
            return x.to(torch.bfloat16).to(dev)
        if dt == FP8_E4M3:
            x = torch.randn(rows, cols, generator=gen, device="cpu").clamp(-448, 448)
            return x.to(torch.float8_e4m3fn).to(dev)
        b = torch.randint(0, 256, (rows, cols // 2), generator=gen, dtype=torch.uint8)
        return b.view(torch.float4_e2m1fn_x2).to(dev)
    A, B = codes(M, K), codes(N, K)
    if sm == SCALE_NONE:
        return A, B, None, None
    if sm == SCALE_TENSOR:
        one = torch.ones(1, device=dev)
        return A, B, one, one
    if sm == SCALE_BLOCK128:
        return A, B, torch.ones(M, K // 128, device=dev), torch.ones(N // 128, K // 128, device=dev)
    blk = 128 if sm == SCALE_MX128 else 32
    e = lambda r: torch.full((r, K // blk), 127, dtype=torch.uint8, device=dev)
    return A, B, e(M), e(N)


def graph_us(fn, iters: int) -> float:
    """Mean GPU time per call of fn(i), i = 0..iters-1, captured in one graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (3 * iters)


def sweep(spec: str, iters: int, dev="cuda:0") -> dict:
    kind, dt, sm, M, N, K, split = parse(spec)
    gen = torch.Generator().manual_seed(1234)
    A, B, sA, sB = operands(kind, dt, sm, M, N, K, dev, gen)
    Bs = preshuffle_b(B)
    wbytes = Bs.numel() * Bs.element_size()
    copies = int(2 * LLC_BYTES // wbytes) + 2 if M <= 32 else 1
    Bss = [Bs] + [Bs.clone() for _ in range(copies - 1)]
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, splitk_workspace_bytes(M, N, split) // 4), dtype=torch.float32, device=dev)
    flops = 2.0 * M * N * K
    nbytes = (A.numel() * A.element_size() + wbytes + 2 * M * N)
    cands = []
    for idx, (cfg, kdt, ksm, kout) in enumerate(kernels()):
        if kdt != dt or ksm != sm or kout != (split > 1):
            continue
        try:
            select_kernel(M, N, K, dt, sm, split, cfg)
        except DgpError:
            continue
        cands.append((idx, cfg))
    run = lambda cfg: (lambda i: gemm_preshuffle_splitk(A, Bss[i % copies], split, sA, sB, sm, out=C,
                                                        workspace=ws if split > 1 else None, config=cfg))
    # warm-up: ~0.3 s of the built-in choice
    import time
    warm = run(None)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        for i in range(20):
            warm(i)
        torch.cuda.synchronize()
    best = {}
    for _ in range(2):
        for idx, cfg in cands:
            us = graph_us(run(cfg), max(iters, copies))
            best[idx] = min(us, best.get(idx, us))
    rows = [{"kernel": describe_kernel(idx), "index": idx, "us": round(us, 2),
             "TFLOP/s": round(flops / us / 1e6, 1), "GB/s": round(nbytes / us / 1e3, 1)}
            for idx, us in best.items()]
    rows.sort(key=lambda r: r["us"])
    chosen = select_kernel(M, N, K, dt, sm, split)
    ratio = (best[chosen] / min(best.values())) if rows and chosen in best else None
    return {"shape": spec, "M": M, "N": N, "K": K, "split_k": split, "cold": copies > 1,
            "builtin_choice": describe_kernel(chosen),
            "builtin_time_over_fastest": None if ratio is None else round(ratio, 3),
            "kernels": rows}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", nargs="*", default=DEFAULT_SHAPES)
    ap.add_argument("--iters", type=int, default=20)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        return 1
    for spec in args.shapes:
        print(json.dumps(sweep(spec, args.iters)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
