// Internal launch interface between the C-ABI layer (dgp_api.cpp) and the
// HIP kernels.  Not installed; callers use include/dgp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgp {

// Arguments shared by both GEMM kernel families.  All sizes are validated by
// the host layer before a launch; byte quantities fit in 32 bits there.
struct GemmArgs {
    const uint8_t *A;     // [M][K] elements, row-major
    const uint8_t *Bs;    // preshuffled B (dgp_preshuffle_b layout)
    void *C;              // [M][N] bf16 (direct epilogue)
    float *ws;            // [splits][M][N] fp32 (split-K partial epilogue)
    const void *sA;       // per-tensor: 1 fp32; blockscale: [M][K/128] fp32; mxfp8: [M][K/128] E8M0
    const void *sB;       // per-tensor: 1 fp32; blockscale: [N/128][K/128] fp32; mxfp8: [N][K/128] E8M0
    int M, N;
    int K;                // elements per row
    int Kb;               // bytes per row of A and B
    int Ks;               // bytes of K per split
    int tiles_m, tiles_n, splits;
    int remap, group_m;
};

// Kernel family selectors.
enum Family { kTiled = 0, kStream = 1, kWave = 2 };

// Wave schedules of the tiled family (dgp_config.schedule).
enum Schedule { kSchedInterleaved = 1, kSchedPingPong = 2, kSchedBothLds = 3, kSchedW4 = 4 };

// A's layout in LDS (tiled kernels; dgp_config.a_layout - 1): 1 KiB operand
// blocks (gemm_common.h), or row-major 128-byte rows with XOR-swizzled
// 16-byte chunks (gemm_w4.hip).
enum ALayout { kLayBlocks = 0, kLaySwizzled = 1 };

// A's global -> LDS copy (tiled kernels; dgp_config.a_copy - 1): the async
// buffer load that writes LDS directly, or a buffer load into registers and
// an LDS write (gemm_w4.hip keeps it as an ablation).
enum ACopy { kCopyAsync = 0, kCopyRegs = 1 };

// One compiled kernel configuration.
struct KernelSpec {
    int family;
    int dtype;      // 0 bf16, 1 fp8
    int scale;      // 0 none, 1 tensor, 2 block128, 3 mxfp8 (E8M0, 128-K blocks)
    int out;        // 0 bf16 direct, 1 fp32 partial
    int tm, tn;     // workgroup output tile
    int kt;         // K bytes per main-loop step (tiled) / per LDS panel (stream)
    int waves;      // waves per workgroup
    int p0, p1;     // family-specific: tiled = (wm, wn); stream = (strips per wave, depth)
    int pv, pd;     // scheduling hint pair (tiled)
    int depth;      // prefetch distance: k-tiles (tiled) / steps (stream)
    int sched;      // tiled: kSchedInterleaved, kSchedPingPong, kSchedBothLds or kSchedW4; stream, wave: 0
    void (*launch)(const GemmArgs &, dim3 grid, hipStream_t);
    int lay = 0;    // tiled: A's LDS layout, kLayBlocks or kLaySwizzled
    int copy = 0;   // tiled: A's global -> LDS path, kCopyAsync or kCopyRegs
};

// The compiled GEMM kernels: the tiled family (gemm_tiled.hip), its
// both-in-LDS schedule (gemm_lds.hip), its one-wave-per-SIMD schedule
// (gemm_w4.hip), the streaming family (gemm_stream.hip), the one-row VALU
// kernels (gemm_wave.hip), and all of them in one table in that order
// (dgp_api.cpp) -- the numbering dgp_kernel_info uses.
const KernelSpec *tiled_kernels(int *count);
const KernelSpec *lds_kernels(int *count);
const KernelSpec *w4_kernels(int *count);
const KernelSpec *stream_kernels(int *count);
const KernelSpec *wave_kernels(int *count);
const KernelSpec *kernel_table(int *count);

// Library-owned split-K workspace (noalloc.hip): the size of the fixed
// per-device array, and its device address on the current device (taken
// once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(float **out);

hipError_t launch_preshuffle(const void *src, void *dst, int64_t N, int64_t Kb, bool inverse,
                             hipStream_t stream);
hipError_t launch_splitk_reduce(const float *ws, void *C, int64_t M, int64_t N, int splits,
                                hipStream_t stream);

// Probes (probe.hip).
hipError_t launch_probe_mfma(int which, const void *a, const void *b, float *out, hipStream_t s);
hipError_t launch_probe_lds_dma(const void *src, const int32_t *perm, void *dst, hipStream_t s);
hipError_t launch_probe_lds_dma_narrow(int width, const void *src, const int32_t *perm, void *dst, hipStream_t s);
hipError_t launch_probe_mfma_scaled(int which, const void *a, const void *b, const void *sa, const void *sb,
                                    float *out, hipStream_t s);
hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s);
hipError_t launch_probe_stream_read(const void *src, int64_t bytes, int blocks, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_mfma_peak(int which, int rounds, int blocks, const void *ops, uint32_t *sink,
                                  hipStream_t s);

}  // namespace dgp
