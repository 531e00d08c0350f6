// One-row decode GEMM on the vector ALUs (the "Wave" policy of aiter PR
// #5148's file table: an exact-shape bf16 / per-tensor fp8 decode GEMM
// whose dot products run on the vector units, beside a matrix-core policy).
//
// gemm_wave_kernel -- a workgroup owns one row of C (M = 1 is the case it is
//    for; a larger M runs one workgroup per row and reads B once per row)
//    and TN = 16 columns (one strip of Bs) or TN = 8 (half a strip); its K
//    range is cut into NW contiguous slices, one per wave.  Each lane loads
//    16 bytes of B per step -- one column's run of 8 bf16 or 16 e4m3 values
//    -- and the matching 16 bytes of the A row, and multiplies them on the
//    VALU: bf16 widened to fp32 (a shift or a mask), e4m3 bytes converted
//    to fp32 in pairs, and fused multiply-added into two fp32 accumulators.  A ring of DEPTH steps of loads is kept in flight.
//    The lanes that hold one column are added by cross-lane exchange, the
//    NW wave partials in LDS in wave order (a fixed order: results are
//    reproducible), and wave 0 writes the row.
//
// The matrix-core kernels feed a 16-row operand per instruction, 15 rows of
// which are zero when M = 1; here each load carries only the one row's
// products, so a step costs a few VALU instructions instead of an MFMA.
// Both read every weight byte once and are bound by HBM.
//
// Load shape.  The preshuffled block (16 columns x 64 K-bytes, 1 KiB) holds
// at byte 16*l column l%16 at K-bytes 16*(l/16).  TN = 16: a step is one
// block, lane l loading byte 16*l (64 lanes x 16 bytes, whole 128-byte
// lines).  TN = 8: a step is two consecutive blocks and a lane loads half of
// one: lane l takes block (l/8)%2 at position 16*(l/16) + 8*half + l%8, so
// each instruction still moves eight whole 128-byte lines, all of this
// workgroup's columns.

#include "gemm_common.h"

namespace dgp {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// The two bf16 of a dword as fp32 (exact: a bf16 is the high half of an fp32).
__device__ inline float bf16_lo(int w) { return __builtin_bit_cast(float, (uint32_t)w << 16); }
__device__ inline float bf16_hi(int w) { return __builtin_bit_cast(float, (uint32_t)w & 0xFFFF0000u); }

// 8 bf16 products of one 16-byte run.  A product of two bf16 is exact in
// fp32, so each fused multiply-add rounds once, like an add of the product.
// (The two-term bf16 dot instruction, v_dot2c_f32_bf16 as the compiler emits
// it for gfx950, returned wrong sums here -- values of the size an fp16
// reading of the operands would give -- so it is not used.)
__device__ inline void dot_run(const i32x4 &a, const i32x4 &b, float &acc0, float &acc1,
                               std::integral_constant<int, kDtypeBf16>)
{
    acc0 = __builtin_fmaf(bf16_lo(a.x), bf16_lo(b.x), acc0);
    acc1 = __builtin_fmaf(bf16_hi(a.x), bf16_hi(b.x), acc1);
    acc0 = __builtin_fmaf(bf16_lo(a.y), bf16_lo(b.y), acc0);
    acc1 = __builtin_fmaf(bf16_hi(a.y), bf16_hi(b.y), acc1);
    acc0 = __builtin_fmaf(bf16_lo(a.z), bf16_lo(b.z), acc0);
    acc1 = __builtin_fmaf(bf16_hi(a.z), bf16_hi(b.z), acc1);
    acc0 = __builtin_fmaf(bf16_lo(a.w), bf16_lo(b.w), acc0);
    acc1 = __builtin_fmaf(bf16_hi(a.w), bf16_hi(b.w), acc1);
}

// 16 e4m3 products: each dword's four bytes converted in two pairs
__device__ inline void dot_word8(int a, int b, float &acc0, float &acc1)
{
    const f32x2 a01 = __builtin_amdgcn_cvt_pk_f32_fp8(a, false), b01 = __builtin_amdgcn_cvt_pk_f32_fp8(b, false);
    const f32x2 a23 = __builtin_amdgcn_cvt_pk_f32_fp8(a, true), b23 = __builtin_amdgcn_cvt_pk_f32_fp8(b, true);
    acc0 = __builtin_fmaf(a01.x, b01.x, acc0);
    acc1 = __builtin_fmaf(a01.y, b01.y, acc1);
    acc0 = __builtin_fmaf(a23.x, b23.x, acc0);
    acc1 = __builtin_fmaf(a23.y, b23.y, acc1);
}

__device__ inline void dot_run(const i32x4 &a, const i32x4 &b, float &acc0, float &acc1,
                               std::integral_constant<int, kDtypeFp8>)
{
    dot_word8(a.x, b.x, acc0, acc1);
    dot_word8(a.y, b.y, acc0, acc1);
    dot_word8(a.z, b.z, acc0, acc1);
    dot_word8(a.w, b.w, acc0, acc1);
}

}  // namespace

template <int DT, int SCALE, int OUT, int NW, int DEPTH, int TN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
gemm_wave_kernel(const GemmArgs p)
{
    static_assert(DT == kDtypeBf16 || DT == kDtypeFp8, "bf16 or e4m3");
    static_assert(SCALE == kScaleNone || SCALE == kScaleTensor, "unscaled or per-tensor");
    static_assert(TN == 8 || TN == 16, "half a strip or one strip");
    constexpr bool kHalf = TN == 8;
    constexpr uint32_t kStepBytes = kHalf ? 128u : 64u;   // K-bytes per step
    __shared__ float red[NW][TN];
    if constexpr (kLdsPoison) {   // debug build: the partial-sum array poisoned before its writes
        lds_poison_fill(red, (int)sizeof(red));
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const auto tc = tile_of_workgroup<int>((int)blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.remap, p.group_m);
    const int m = (int)tc.tm;
    const int strip = kHalf ? (int)tc.tn >> 1 : (int)tc.tn;
    const int half = kHalf ? (int)tc.tn & 1 : 0;
    const int split = (int)tc.s;
    const uint32_t Kb = (uint32_t)p.Kb;
    const uint32_t kbase = (uint32_t)split * (uint32_t)p.Ks;
    const int nsteps = p.Ks / (int)kStepBytes;
    const int per = nsteps / NW, extra = nsteps % NW;
    const int s0 = wave * per + (wave < extra ? wave : extra);
    const int s1 = s0 + per + (wave < extra ? 1 : 0);

    // This lane's 16 bytes in a step: block j of the step (TN = 8: the
    // lane's half-block; TN = 16: the one block), position pos in it; the A
    // bytes at the same K: K-byte 64*j + 16*(l/16) of the step.
    const uint32_t j = kHalf ? (uint32_t)(lane >> 3) & 1u : 0u;
    const uint32_t pos = kHalf ? (uint32_t)(lane >> 4) * 16u + (uint32_t)half * 8u + (uint32_t)(lane & 7)
                               : (uint32_t)lane;
    const uint32_t b_off = j * 1024u + pos * 16u;
    const uint32_t a_off = j * 64u + (uint32_t)(lane >> 4) * 16u;
    // The resources cover the strip (16 rows of Bs) and the row of A; the
    // grid holds only strips < N / 16 and rows < M.
    const auto rB = make_rsrc(p.Bs + (int64_t)strip * 16 * Kb, 16u * Kb);
    const auto rA = make_rsrc(p.A + (int64_t)m * Kb, Kb);

    // The slice's steps stream through a ring of DEPTH slots of in-flight
    // loads (ring_run: loads only for steps of the slice, exact waits while
    // the ring is refilled).
    i32x4 areg[DEPTH], breg[DEPTH];
    float acc0 = 0.f, acc1 = 0.f;
    ring_run<DEPTH>(
        s1 - s0,
        [&](int d, int i) {
            const uint32_t k = kbase + (uint32_t)(s0 + i) * kStepBytes;
            breg[d] = load16<kAuxNonTemporal>(rB, k * 16u + b_off);
            areg[d] = load16<kAuxNone>(rA, k + a_off);
        },
        [&](int d, int) { dot_run(areg[d], breg[d], acc0, acc1, std::integral_constant<int, DT>{}); });

    // Lanes holding one column: l % 16 (TN = 16) or l % 8 (TN = 8, whose
    // lanes l and l ^ 8 hold the two blocks of a step).  Each exchange adds a
    // pair in the same order on both lanes, so all of them end equal.
    float v = acc0 + acc1;
    if constexpr (kHalf)
        v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lane < TN)
        red[wave][lane] = v;
    __syncthreads();
    if (wave == 0 && lane < TN) {
        float s = red[0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            s += red[w][lane];
        const int n = strip * 16 + half * 8 + lane;
        if constexpr (OUT == kOutBf16) {
            if constexpr (SCALE == kScaleTensor)
                s = s * (static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0]);
            static_cast<__bf16 *>(p.C)[(int64_t)m * p.N + n] = (__bf16)s;
        } else {
            if constexpr (SCALE == kScaleTensor)
                s = s * (static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0]);
            p.ws[((int64_t)split * p.M + m) * p.N + n] = s;
        }
    }
}

template <int DT, int SCALE, int OUT, int NW, int DEPTH, int TN>
void launch_wave(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    gemm_wave_kernel<DT, SCALE, OUT, NW, DEPTH, TN><<<grid, NW * 64, 0, s>>>(a);
}

#define DGP_WAVE(DT, SC, OUT, NW, DEPTH, TN) \
    {kWave, DT, SC, OUT, 1, TN, 0, NW, 0, DEPTH, 0, 0, DEPTH, 0, &launch_wave<DT, SC, OUT, NW, DEPTH, TN>}
#define DGP_WAVE_BOTH_OUT(DT, SC, NW, DEPTH, TN) \
    DGP_WAVE(DT, SC, kOutBf16, NW, DEPTH, TN), DGP_WAVE(DT, SC, kOutPartial, NW, DEPTH, TN)
#define DGP_WAVE_SET(DT, SC, TN)                                                            \
    DGP_WAVE_BOTH_OUT(DT, SC, 4, 8, TN), DGP_WAVE_BOTH_OUT(DT, SC, 8, 4, TN),              \
        DGP_WAVE_BOTH_OUT(DT, SC, 8, 8, TN), DGP_WAVE_BOTH_OUT(DT, SC, 4, 4, TN)

static const KernelSpec kWaveKernels[] = {
    // one row, one strip / half a strip: waves per workgroup, ring depth
    DGP_WAVE_SET(kDtypeBf16, kScaleNone, 16),
    DGP_WAVE_SET(kDtypeBf16, kScaleNone, 8),
    DGP_WAVE_SET(kDtypeFp8, kScaleTensor, 16),
    DGP_WAVE_SET(kDtypeFp8, kScaleTensor, 8),
};

const KernelSpec *wave_kernels(int *count)
{
    *count = (int)(sizeof(kWaveKernels) / sizeof(kWaveKernels[0]));
    return kWaveKernels;
}

}  // namespace dgp
