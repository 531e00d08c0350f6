"""Build the gfx950 HIP library libdgp.so in-tree (dense_gemm_packer_amd/libdgp.so).

Each source under csrc/ is compiled with hipcc for gfx950 only, in parallel,
then linked into one shared library.  Packed-fp32 VALU instructions are
disabled for all device code.  The same sources compiled with
DGP_LDS_POISON=1 give the LDS-poison debug build, libdgp_lds_poison.so
(every kernel's LDS filled with 0xFF before use, every global -> LDS copy's
destination poisoned until the copy lands), which the tests run beside the
release build.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdgp.so")
POISON_LIB = os.path.join(HERE, "libdgp_lds_poison.so")
SOURCES = ["dgp_api.cpp", "packer.hip", "gemm_tiled.hip", "gemm_lds.hip", "gemm_stream.hip", "reduce.hip", "probe.hip", "noalloc.hip", "gemm_w4.hip", "gemm_wave.hip"]
HEADERS = ["common.h", "launch.h", "gemm_common.h"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Keep MFMA accumulators in arch VGPRs (avoids accumulator copies at loop
# latches) everywhere except in the kernels that need the AGPRs for them.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC_SOURCES = {"gemm_lds.hip", "gemm_w4.hip"}


def flags(src):
    """hipcc flags for one source file."""
    return CFLAGS + ([] if src in AGPR_ACC_SOURCES else VGPR_FORM)


def _compile(job):
    src, poison = job
    obj = os.path.join(BUILD, ("lds_poison_" if poison else "") + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *flags(src), *(["-DDGP_LDS_POISON=1"] if poison else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(force: bool = True, jobs: int = 0) -> str:
    """Compile every source twice and link libdgp.so and libdgp_lds_poison.so;
    returns the release library's path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    hdrs = [os.path.join(CSRC, h) for h in HEADERS] + [
        os.path.join(HERE, "..", "include", h) for h in ("dgp.h", "dgp_diag.h")]
    if not force and os.path.exists(LIB) and os.path.exists(POISON_LIB):
        newest = max(os.path.getmtime(p) for p in srcs + hdrs)
        if min(os.path.getmtime(LIB), os.path.getmtime(POISON_LIB)) >= newest:
            return LIB
    os.makedirs(BUILD, exist_ok=True)
    # the slowest sources first, so the pool's tail is short
    order = sorted(SOURCES, key=lambda f: -os.path.getsize(os.path.join(CSRC, f)))
    todo = [(f, False) for f in order] + [(f, True) for f in order]
    jobs = jobs or min(len(todo), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = dict(zip(todo, ex.map(_compile, todo)))
    for _, msgs in results.values():
        if msgs.strip():
            print(msgs, file=sys.stderr)
    _link([results[(f, False)][0] for f in SOURCES], LIB)
    _link([results[(f, True)][0] for f in SOURCES], POISON_LIB)
    return LIB


def asm(src: str, out: str) -> None:
    """Write the gfx950 assembly of one source (for inspection)."""
    cmd = [HIPCC, *flags(src), "-x", "hip", "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    print(build())
