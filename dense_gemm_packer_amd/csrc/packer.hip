// B preshuffle packer: a byte permutation of B into 1 KiB matrix-core
// operand blocks (layout defined in include/dgp.h, dgp_preshuffle_b).  The
// pages name the preshuffled layout (FlyDSL PR #1008 title and file table,
// aiter PR #5148 "bpreshuffle") but never write it out.
//
// One workgroup per 16-row strip of B.  Thread t of the workgroup moves the
// 16-byte destination chunks d = t, t + 256, ... of the strip; chunk d of a
// strip is lane d % 64 of block kb = d / 64, i.e. source row 16*nb + lane % 16,
// K-bytes 64*kb + 16*(lane / 16).  Destination writes are fully contiguous per
// workgroup; each source row is read in 64-byte runs that together cover the
// whole row.  HBM-bound: 2 * N * Kb bytes per call.
#include "common.h"
#include "launch.h"

namespace dgp {

constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 4;

template <bool kInverse>
__global__ __launch_bounds__(kPackThreads) void preshuffle_kernel(const uint8_t *__restrict__ src,
                                                                   uint8_t *__restrict__ dst,
                                                                   uint32_t Kb)
{
    // Strip nb occupies the same byte range [16*nb*Kb, 16*(nb+1)*Kb) in both
    // layouts, so only the offsets inside the strip differ.
    const int64_t strip = (int64_t)blockIdx.x * 16 * (int64_t)Kb;
    const uint8_t *in_base = src + strip;
    uint8_t *out_base = dst + strip;
    const uint32_t chunks = Kb;   // 16 rows * Kb bytes / 16 bytes per chunk

    for (uint32_t d0 = threadIdx.x; d0 < chunks; d0 += kPackThreads * kPackUnroll) {
        i32x4 v[kPackUnroll];
        uint32_t row_off[kPackUnroll];
#pragma unroll
        for (int u = 0; u < kPackUnroll; ++u) {
            uint32_t d = d0 + u * kPackThreads;
            uint32_t kb = d >> 6, lane = d & 63u;
            row_off[u] = (lane & 15u) * Kb + kb * 64u + (lane >> 4) * 16u;
            if (d < chunks) {
                uint32_t in_off = kInverse ? d * 16u : row_off[u];
                v[u] = *reinterpret_cast<const i32x4 *>(in_base + in_off);
            }
        }
#pragma unroll
        for (int u = 0; u < kPackUnroll; ++u) {
            uint32_t d = d0 + u * kPackThreads;
            if (d < chunks) {
                uint32_t out_off = kInverse ? row_off[u] : d * 16u;
                *reinterpret_cast<i32x4 *>(out_base + out_off) = v[u];
            }
        }
    }
}

hipError_t launch_preshuffle(const void *src, void *dst, int64_t N, int64_t Kb, bool inverse,
                             hipStream_t stream)
{
    if (N == 0 || Kb == 0)
        return hipSuccess;
    dim3 grid((unsigned)(N / 16)), block(kPackThreads);
    if (inverse)
        preshuffle_kernel<true><<<grid, block, 0, stream>>>((const uint8_t *)src, (uint8_t *)dst,
                                                            (uint32_t)Kb);
    else
        preshuffle_kernel<false><<<grid, block, 0, stream>>>((const uint8_t *)src, (uint8_t *)dst,
                                                             (uint32_t)Kb);
    return hipGetLastError();
}

}  // namespace dgp
