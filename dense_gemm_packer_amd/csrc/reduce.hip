// Split-K pass 2: C[m][n] = bf16(P_0 + P_1 + ... + P_{S-1}) over the fp32
// partials ws[s][M][N], summed in fp32 in split order and rounded to bf16
// once (aiter PR #5148, file table: an fp32 split-K reduction kernel that
// downcasts once at the final store).  Each thread owns four consecutive
// outputs: S 16-byte loads, issued up to 8 at a time so their latencies
// overlap, added in split order; one 8-byte store.  HBM-bound:
// S*M*N*4 + M*N*2 bytes.  Also a zero fill for K = 0 (C = A*B^T = 0).
#include "common.h"
#include "launch.h"

namespace dgp {

constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(const float *__restrict__ ws,
                                                                        uint8_t *__restrict__ C,
                                                                        int64_t groups, int64_t mn,
                                                                        int splits)
{
    const int64_t g = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
    if (g >= groups)
        return;
    constexpr int kBatch = 8;
    const float *p = ws + g * 4;
    // The sum starts from partial 0 itself (not 0 + P_0, which would turn a
    // -0 partial into +0).
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += kBatch) {
        f32x4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (s0 + u < splits)
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + (int64_t)(s0 + u) * mn));
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (s0 + u >= splits)
                break;
            if (s0 + u == 0) {
                t = v[0];
            } else {
                t.x = __fadd_rn(t.x, v[u].x);
                t.y = __fadd_rn(t.y, v[u].y);
                t.z = __fadd_rn(t.z, v[u].z);
                t.w = __fadd_rn(t.w, v[u].w);
            }
        }
    }
    u32x2 out;
    out.x = pack_bf16x2(t.x, t.y);
    out.y = pack_bf16x2(t.z, t.w);
    *reinterpret_cast<u32x2 *>(C + g * 8) = out;
}

__global__ __launch_bounds__(kReduceThreads) void zero_fill_kernel(uint8_t *__restrict__ C, int64_t groups)
{
    const int64_t g = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x;
    if (g < groups)
        *reinterpret_cast<u32x2 *>(C + g * 8) = u32x2{0u, 0u};
}

hipError_t launch_splitk_reduce(const float *ws, void *C, int64_t M, int64_t N, int splits,
                                hipStream_t stream)
{
    const int64_t mn = M * N;              // N % 16 == 0, so mn % 4 == 0
    const int64_t groups = mn / 4;
    if (groups == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((groups + kReduceThreads - 1) / kReduceThreads));
    if (splits == 0)
        zero_fill_kernel<<<grid, kReduceThreads, 0, stream>>>((uint8_t *)C, groups);
    else
        splitk_reduce_kernel<<<grid, kReduceThreads, 0, stream>>>(ws, (uint8_t *)C, groups, mn, splits);
    return hipGetLastError();
}

}  // namespace dgp
