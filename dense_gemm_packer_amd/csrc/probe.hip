// Probe kernels: check the hardware facts the GEMM relies on (matrix-core
// register layouts, where the async global->LDS copy puts each lane's bytes)
// and measure the walls the GEMM is judged against (a plain copy of known
// traffic for counter calibration, a streaming read for the HBM wall).
#include "common.h"
#include "launch.h"

namespace dgp {

__global__ __launch_bounds__(64) void probe_mfma_kernel(int which, const uint8_t *a, const uint8_t *b, float *out)
{
    const int l = threadIdx.x;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (which == 0) {
        const i32x4 x = *reinterpret_cast<const i32x4 *>(a + l * 16);
        const i32x4 y = *reinterpret_cast<const i32x4 *>(b + l * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                      __builtin_bit_cast(bf16x8, y), acc, 0, 0, 0);
    } else {
        const i32x8 x = *reinterpret_cast<const i32x8 *>(a + l * 32);
        const i32x8 y = *reinterpret_cast<const i32x8 *>(b + l * 32);
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, 0, 0, 0, 0, 0, 0);
    }
    *reinterpret_cast<f32x4 *>(out + l * 4) = acc;
}

__global__ __launch_bounds__(64) void probe_lds_dma_kernel(const uint8_t *src, const int32_t *perm, uint8_t *dst)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[1024];
    const int l = threadIdx.x;
    *reinterpret_cast<i32x4 *>(lds + l * 16) = i32x4{-1, -1, -1, -1};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const auto r = make_rsrc(src, 1024);
    const int q = perm[l];
    const uint32_t off = (uint32_t)((q >= 0 && q < 64) ? q : 0) * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off, 0, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    *reinterpret_cast<i32x4 *>(dst + l * 16) = *reinterpret_cast<const i32x4 *>(lds + l * 16);
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const i32x4 *__restrict__ src, i32x4 *__restrict__ dst, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per thread

// Streaming read: round i of workgroup b covers the 64 KiB chunk i*grid + b;
// thread t reads bytes chunk + u*8192 + 16*t for u < 8 (8 loads in flight per
// thread, 64 KiB per workgroup), non-temporal.
__global__ __launch_bounds__(kStreamThreads) void probe_stream_read_kernel(const uint8_t *__restrict__ src,
                                                                           int64_t bytes, uint32_t *__restrict__ sink)
{
    constexpr int64_t kChunk = (int64_t)kStreamThreads * 16 * kStreamUnroll;
    const int64_t chunks = bytes / kChunk;
    i32x4 x = {0, 0, 0, 0};
    for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const auto r = make_rsrc(src + c * kChunk, (uint32_t)kChunk);
        i32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = load16<kAuxNonTemporal>(r, (uint32_t)(u * kStreamThreads * 16 + threadIdx.x * 16));
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            x ^= v[u];
    }
    const uint32_t f = (uint32_t)(x.x ^ x.y ^ x.z ^ x.w);
    if (f == 0x9E3779B9u)   // practically never true; keeps the loads alive
        sink[blockIdx.x & 4095] = f;
}

hipError_t launch_probe_mfma(int which, const void *a, const void *b, float *out, hipStream_t s)
{
    probe_mfma_kernel<<<1, 64, 0, s>>>(which, (const uint8_t *)a, (const uint8_t *)b, out);
    return hipGetLastError();
}

hipError_t launch_probe_lds_dma(const void *src, const int32_t *perm, void *dst, hipStream_t s)
{
    probe_lds_dma_kernel<<<1, 64, 0, s>>>((const uint8_t *)src, perm, (uint8_t *)dst);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t s)
{
    const int64_t n = bytes / 16;
    if (n == 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    probe_copy_kernel<<<(unsigned)blocks, 256, 0, s>>>((const i32x4 *)src, (i32x4 *)dst, n);
    return hipGetLastError();
}

hipError_t launch_probe_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s)
{
    // Whole 64 KiB chunks are read; the tail (bytes % 64 KiB) is not.
    const int64_t chunks = bytes / ((int64_t)kStreamThreads * 16 * kStreamUnroll);
    if (chunks == 0)
        return hipSuccess;
    const int64_t blocks = chunks < 1024 ? chunks : 1024;
    probe_stream_read_kernel<<<(unsigned)blocks, kStreamThreads, 0, s>>>((const uint8_t *)src, bytes, sink);
    return hipGetLastError();
}

}  // namespace dgp
