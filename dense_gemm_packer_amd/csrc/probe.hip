// Probe kernels: check the hardware facts the GEMM relies on (matrix-core
// register layouts, where the async global->LDS copy puts each lane's bytes)
// and measure the walls the GEMM is compared with (a plain copy of known
// traffic for counter calibration, a streaming read for the HBM wall, a
// register-only matrix-core loop for the sustained MFMA rate).
#include <type_traits>

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

// One hardware-scaled MFMA: lane l supplies E8M0 scale byte sa[l] for its A
// fragment (src1 here, as in the GEMM) and sb[l] for its B fragment (src0),
// each in byte 0 of a 32-bit operand (op_sel 0).  FMT 0: e4m3 operands, 32
// bytes per lane; FMT 4: e2m1 operands, the first 16 bytes of each lane's
// 32-byte slot (32 fp4 values), the upper half unused.
template <int FMT>
__global__ __launch_bounds__(64) void probe_mfma_scaled_kernel(const uint8_t *a, const uint8_t *b,
                                                               const uint8_t *sa, const uint8_t *sb, float *out)
{
    const int l = threadIdx.x;
    i32x8 x = *reinterpret_cast<const i32x8 *>(a + l * 32);
    i32x8 y = *reinterpret_cast<const i32x8 *>(b + l * 32);
    if constexpr (FMT == 4) {
        x.s4 = x.s5 = x.s6 = x.s7 = 0;
        y.s4 = y.s5 = y.s6 = y.s7 = 0;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(y, x, acc, FMT, FMT, 0, (int)sb[l], 0, (int)sa[l]);
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

// The narrow forms of the same load (W = 1, 2 or 4 bytes per lane): LDS is
// filled with 0xFF first, so the dump shows both where each lane's bytes land
// and which LDS bytes the load leaves alone.
template <int W>
__global__ __launch_bounds__(64) void probe_lds_dma_narrow_kernel(const uint8_t *src, const int32_t *perm,
                                                                  uint8_t *dst)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[1024];
    const int l = threadIdx.x;
    *reinterpret_cast<i32x4 *>(lds + l * 16) = i32x4{-1, -1, -1, -1};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const auto r = make_rsrc(src, 64 * W);
    const int q = perm[l];
    const uint32_t off = (uint32_t)((q >= 0 && q < 64) ? q : 0) * W;
    auto *d = (__attribute__((address_space(3))) void *)lds;
    if constexpr (W == 1)   // the size operand must be a literal
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 1, off, 0, 0, 0);
    else if constexpr (W == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 2, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 4, off, 0, 0, 0);
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
constexpr int64_t kStreamRound = (int64_t)kStreamThreads * 16 * kStreamUnroll;   // 64 KiB

// Streaming read: workgroup b reads bytes [b*span, min((b+1)*span, bytes))
// front to back in rounds of 64 KiB; in a round thread t reads 16 bytes at
// u*8192 + 16*t for u < 8 (8 loads in flight per thread), non-temporal.  The
// last round of a span is clamped by the buffer resource, so any span that
// is a multiple of 16 bytes is read exactly.
__global__ __launch_bounds__(kStreamThreads) void probe_stream_read_kernel(const uint8_t *__restrict__ src,
                                                                           int64_t bytes, int64_t span,
                                                                           uint32_t *__restrict__ sink)
{
    const int64_t b0 = (int64_t)blockIdx.x * span;
    const int64_t b1 = b0 + span < bytes ? b0 + span : bytes;
    i32x4 x = {0, 0, 0, 0};
    for (int64_t off = b0; off < b1; off += kStreamRound) {
        const auto r = make_rsrc(src + off, (uint32_t)(b1 - off < kStreamRound ? b1 - off : kStreamRound));
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

constexpr int kPeakThreads = 256;   // 4 waves per workgroup
constexpr int kPeakSets = 256;      // operand sets in the caller's buffer

// Sustained matrix-core rate on given operands: each wave loads 8 A and 8 B
// fragments (operand set wave % kPeakSets of the caller's buffer) into
// registers, then issues rounds x 64 MFMAs over 8 independent accumulators,
// pairing every B fragment with every A fragment in turn, with no memory
// traffic in the loop.  The matrix units draw more power on operands that
// toggle, so the rate depends on the data: random operands hold a lower
// clock than constant ones.  which = 0: v_mfma_f32_16x16x32_bf16,
// 1: the e4m3 16x16x128 form, 2: the E2M1 16x16x128 form; both scaled forms
// take unit block scales (E8M0 127).
template <int WHICH, typename F>
__device__ inline void peak_mfma(f32x4 &acc, const F &b, const F &a, int unit)
{
    if constexpr (WHICH == 0)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    else if constexpr (WHICH == 1)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                     : "+a"(acc)
                     : "v"(b), "v"(a), "v"(unit));
    else
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(acc)
                     : "v"(b), "v"(a), "v"(unit));
}

template <int WHICH>
__global__ __launch_bounds__(kPeakThreads) void probe_mfma_peak_kernel(int rounds, const uint8_t *__restrict__ ops,
                                                                       uint32_t *sink)
{
    constexpr int kFB = WHICH == 1 ? 32 : 16;   // bytes per lane per fragment
    using F = typename std::conditional<WHICH == 1, i32x8, i32x4>::type;
    const int l = threadIdx.x & 63;
    const int set = (int)((blockIdx.x * (kPeakThreads / 64) + (threadIdx.x >> 6)) % kPeakSets);
    const uint8_t *base = ops + (size_t)set * 16 * 64 * kFB + l * kFB;
    F af[8], bf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        af[j] = *reinterpret_cast<const F *>(base + j * 64 * kFB);
        bf[j] = *reinterpret_cast<const F *>(base + (8 + j) * 64 * kFB);
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int unit = 127;   // E8M0 2^0
    // 2 wait states between the vector-ALU write of the scale register and
    // the first scaled MFMA that reads it (the asm ties the nop to it).
    asm volatile("s_nop 1" : "+v"(unit));
    // Each accumulator is pinned to its AGPRs by the asm operand, so the
    // loop holds nothing but the 64 MFMAs and its branch (the builtins let
    // the register allocator rotate accumulators and add copies).
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                peak_mfma<WHICH>(acc[j], bf[j], af[(j + s) & 7], unit);
            }
        }
    }
    float f = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        f += acc[j].x + acc[j].y + acc[j].z + acc[j].w;
    if (f == 1.2345e-7f)   // practically never true; keeps the products alive
        sink[blockIdx.x & 4095] = (uint32_t)l;
}

hipError_t launch_probe_mfma(int which, const void *a, const void *b, float *out, hipStream_t s)
{
    probe_mfma_kernel<<<1, 64, 0, s>>>(which, (const uint8_t *)a, (const uint8_t *)b, out);
    return hipGetLastError();
}

hipError_t launch_probe_mfma_scaled(int which, const void *a, const void *b, const void *sa, const void *sb,
                                    float *out, hipStream_t s)
{
    if (which == 0)
        probe_mfma_scaled_kernel<0><<<1, 64, 0, s>>>((const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sa,
                                                     (const uint8_t *)sb, out);
    else
        probe_mfma_scaled_kernel<4><<<1, 64, 0, s>>>((const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sa,
                                                     (const uint8_t *)sb, out);
    return hipGetLastError();
}

hipError_t launch_probe_lds_dma(const void *src, const int32_t *perm, void *dst, hipStream_t s)
{
    probe_lds_dma_kernel<<<1, 64, 0, s>>>((const uint8_t *)src, perm, (uint8_t *)dst);
    return hipGetLastError();
}

hipError_t launch_probe_lds_dma_narrow(int width, const void *src, const int32_t *perm, void *dst, hipStream_t s)
{
    const auto *in = (const uint8_t *)src;
    auto *out = (uint8_t *)dst;
    if (width == 1)
        probe_lds_dma_narrow_kernel<1><<<1, 64, 0, s>>>(in, perm, out);
    else if (width == 2)
        probe_lds_dma_narrow_kernel<2><<<1, 64, 0, s>>>(in, perm, out);
    else
        probe_lds_dma_narrow_kernel<4><<<1, 64, 0, s>>>(in, perm, out);
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

hipError_t launch_probe_mfma_peak(int which, int rounds, int blocks, const void *ops, uint32_t *sink,
                                  hipStream_t s)
{
    if (which == 0)
        probe_mfma_peak_kernel<0><<<blocks, kPeakThreads, 0, s>>>(rounds, (const uint8_t *)ops, sink);
    else if (which == 1)
        probe_mfma_peak_kernel<1><<<blocks, kPeakThreads, 0, s>>>(rounds, (const uint8_t *)ops, sink);
    else
        probe_mfma_peak_kernel<2><<<blocks, kPeakThreads, 0, s>>>(rounds, (const uint8_t *)ops, sink);
    return hipGetLastError();
}

hipError_t launch_probe_stream_read(const void *src, int64_t bytes, int blocks, uint32_t *sink, hipStream_t s)
{
    // Equal spans of whole 16-byte units; the last workgroups may get less
    // (or nothing, when the rounded span already covers the range).
    const int64_t units = bytes / 16;
    const int64_t span = (units + blocks - 1) / blocks * 16;
    const int64_t used = (bytes + span - 1) / span;
    probe_stream_read_kernel<<<(unsigned)used, kStreamThreads, 0, s>>>((const uint8_t *)src, bytes, span, sink);
    return hipGetLastError();
}

}  // namespace dgp
