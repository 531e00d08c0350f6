// Large-M GEMM kernel for C = A * B^T with B preshuffled (include/dgp.h) with
// both operands staged in LDS, and its table entries.  Operand layout and
// epilogue: gemm_common.h.
//
// gemm_lds_kernel -- per 128-byte k-tile, the A tile (TM rows) and the
// preshuffled B tile (TN/16 strips) go global -> LDS with the async buffer
// load into a two-stage ring, and the waves (WM x WN, each owning TM/WM rows
// x TN/WN columns) read both operands' fragments from LDS.  The preshuffled B
// needs no swizzle there: a 1 KiB block of Bs is copied unchanged (one fully
// coalesced 16-byte-per-lane load per wave) and already sits in operand
// order, so its fragment reads are conflict-free like A's.  Against
// gemm_tiled_kernel, every global load is an LDS-bound copy (none returns
// through the VGPRs), and a B fragment read once feeds TM/WM/16 MFMAs.
//
// Pipeline.  A k-tile is two phases of equal matrix-core work: bf16 phase p
// is MFMA k-step p over the wave's row tiles, fp8 phase p is the single
// 128-deep k-step over half of them.  The fragments of a phase live in
// register set p, so the reads for the next phase run under the MFMAs of the
// current one:
//
//   phase (t,0): MFMAs of (t,0)   | copies of tile t+1 into the free stage,
//                                 | fragment reads of (t,1)
//   phase (t,1): first half of its MFMAs,
//                wait for this wave's copies and reads, workgroup barrier,
//                second half       | fragment reads of (t+1,0) from the
//                                  | other stage
//
// The barrier certifies that tile t+1 has landed for every wave and that no
// wave still reads tile t's stage, which tile t+2's copies overwrite during
// phase (t+1,0).  One barrier per k-tile, placed where MFMAs already in
// registers cover it.  The last tile's "next" copy is a clamped repeat of
// tile t into the free stage, so every step has the same shape.
//
// Built without the VGPR-form MFMA option (see build.py): the accumulators
// may live in AGPRs, leaving the VGPRs to the two fragment sets.

#include "gemm_common.h"

namespace dgp {

template <int DT, int TM, int TN, int WM, int WN, int SCALE, int OUT>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu((WM * WN + 3) / 4, (WM * WN + 3) / 4)))
gemm_lds_kernel(const GemmArgs p)
{
    constexpr int KT = 128;
    using S = TiledShape<DT, TM, TN, WM, WN, KT>;
    using Frag = typename Op<DT>::Frag;
    constexpr bool kBf16 = DT == kDtypeBf16;
    constexpr int kABytes = TM * KT, kBBytes = TN * KT, kStage = kABytes + kBBytes;
    constexpr int kBBlocks = (TN / 16) * S::kCH;
    constexpr int kBDmaPerWave = kBBlocks / S::kWaves;
    constexpr int kDma = S::kDmaPerWave + kBDmaPerWave;      // copies per wave per k-tile
    constexpr int kRowsPh = kBf16 ? S::kMT : S::kMT / 2;       // row tiles per phase
    constexpr int kMfmaPh = kRowsPh * S::kNT;                  // MFMAs per phase
    constexpr int kReadsPh = (kRowsPh + S::kNT) * S::kStepCh;  // LDS reads per phase
    static_assert(S::kCH == 2 && (kBf16 ? S::kSteps == 2 : (S::kSteps == 1 && S::kMT % 2 == 0)),
                  "two phases per 128-byte k-tile");
    static_assert(kBBlocks % S::kWaves == 0, "B tile must split into whole copies per wave");
    static_assert(2 * kStage <= 160 * 1024, "two stages must fit in LDS");
    static_assert(kMfmaPh % 2 == 0 && kMfmaPh >= kDma, "phase too short for its copies");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStage];
    if constexpr (kLdsPoison) {   // debug build: all of LDS poisoned before the first copy
        lds_poison_fill(lds, (int)sizeof(lds));
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const auto tc = tile_of_workgroup<int>((int)blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.remap, p.group_m);
    const int m0 = (int)tc.tm * TM;
    const int n0 = (int)tc.tn * TN;
    const int split = (int)tc.s;
    const uint32_t Kb = (uint32_t)p.Kb;
    const uint32_t kbase = (uint32_t)split * (uint32_t)p.Ks;
    const int ntiles = p.Ks / KT;

    // A copies: instruction j fills A block j*waves + wave = (row group,
    // 64-byte chunk), lane l holding row 16*rg + l%16 at K-bytes 64*ch +
    // 16*(l/16); rows >= M load as zero.
    const auto rA = make_rsrc(p.A + (int64_t)m0 * Kb, clamp_bytes((int64_t)(p.M - m0) * Kb));
    uint32_t a_voff[S::kDmaPerWave];
#pragma unroll
    for (int j = 0; j < S::kDmaPerWave; ++j) {
        const int blk = j * S::kWaves + wave;
        a_voff[j] = (uint32_t)((blk / S::kCH) * 16 + (lane & 15)) * Kb +
                    (uint32_t)((blk % S::kCH) * 64 + (lane >> 4) * 16);
    }
    // B copies: instruction j copies block j*waves + wave = (strip sb of the
    // tile, chunk ch) of Bs unchanged; strips >= N/16 load as zero.
    const int strip0 = n0 / 16;
    const auto rB = make_rsrc(p.Bs + (int64_t)strip0 * 16 * Kb,
                              clamp_bytes((int64_t)(p.N / 16 - strip0) * 16 * Kb));
    uint32_t b_voff[kBDmaPerWave];
#pragma unroll
    for (int j = 0; j < kBDmaPerWave; ++j) {
        const int blk = j * S::kWaves + wave;
        b_voff[j] = (uint32_t)(blk / S::kCH) * 16u * Kb + (uint32_t)(blk % S::kCH) * 1024u + (uint32_t)lane * 16u;
    }

    float scale = 1.0f;
    if constexpr (SCALE == kScaleTensor)
        scale = static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0];

    f32x4 acc[S::kMT][S::kNT];
#pragma unroll
    for (int i = 0; i < S::kMT; ++i)
#pragma unroll
        for (int j = 0; j < S::kNT; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Frag af[2][kRowsPh], bf[2][S::kNT];   // fragment set = phase

    auto copy_tile = [&](uint32_t stage_off, int t) {
        const uint32_t koff = kbase + (uint32_t)(t < ntiles ? t : ntiles - 1) * KT;
#pragma unroll
        for (int j = 0; j < S::kDmaPerWave; ++j)
            lds_dma16(rA, lds + stage_off + (j * S::kWaves + wave) * 1024, a_voff[j], koff);
#pragma unroll
        for (int j = 0; j < kBDmaPerWave; ++j)
            lds_dma16(rB, lds + stage_off + kABytes + (j * S::kWaves + wave) * 1024, b_voff[j], koff * 16u);
    };
    // Row tile and k-step of fragment r of phase P.
    auto row_of = [](int P, int r) { return kBf16 ? r : P * kRowsPh + r; };
    auto step_of = [](int P) { return kBf16 ? P : 0; };
    auto read_phase = [&](auto pc, uint32_t stage_off) {
        constexpr int P = decltype(pc)::value;
        const uint8_t *abase = lds + stage_off + (wm * S::kMT * S::kCH) * 1024 + lane * 16;
        const uint8_t *bbase = lds + stage_off + kABytes + (wn * S::kNT * S::kCH) * 1024 + lane * 16;
        // B first: every MFMA of the phase's first row tile needs all of them.
#pragma unroll
        for (int nt = 0; nt < S::kNT; ++nt)
            bf[P][nt] = lds_frag<DT>(bbase + (nt * S::kCH + step_of(P) * S::kStepCh) * 1024);
#pragma unroll
        for (int r = 0; r < kRowsPh; ++r)
            af[P][r] = lds_frag<DT>(abase + (row_of(P, r) * S::kCH + step_of(P) * S::kStepCh) * 1024);
    };
    auto mfma_phase = [&](auto pc, auto loc, auto hic) {
        constexpr int P = decltype(pc)::value, LO = decltype(loc)::value, HI = decltype(hic)::value;
#pragma unroll
        for (int i = LO; i < HI; ++i) {
            const int r = i / S::kNT, nt = i % S::kNT;
            acc[row_of(P, r)][nt] = mfma_op(bf[P][nt], af[P][r], acc[row_of(P, r)][nt]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using IHalf = std::integral_constant<int, kMfmaPh / 2>;
    using IAll = std::integral_constant<int, kMfmaPh>;

    // Prologue: tile 0 into stage 0, visible to all waves; phase (0,0) read.
    copy_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    read_phase(I0{}, 0);

    for (int t = 0; t < ntiles; ++t) {
        const uint32_t cur = (uint32_t)(t & 1) * kStage, nxt = kStage - cur;
        // ---- phase (t,0): copies of tile t+1, reads of (t,1).
        copy_tile(nxt, t + 1);
        read_phase(I1{}, cur);
        mfma_phase(I0{}, I0{}, IAll{});
        // The copies one per MFMA first, then the reads spread over the rest.
#pragma unroll
        for (int j = 0; j < kDma; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        {
            constexpr int kLeft = kMfmaPh - kDma;
            constexpr int kPer = (kReadsPh + kLeft - 1) / kLeft;   // reads per MFMA, rounded up
#pragma unroll
            for (int j = 0; j < kLeft; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (j * kPer < kReadsPh)
                    __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- phase (t,1): half, barrier, half with the reads of (t+1,0).
        mfma_phase(I1{}, I0{}, IHalf{});
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        read_phase(I0{}, nxt);
        mfma_phase(I1{}, IHalf{}, IAll{});
        {
            constexpr int kLeft = kMfmaPh / 2;
            constexpr int kPer = (kReadsPh + kLeft - 1) / kLeft;
#pragma unroll
            for (int j = 0; j < kLeft; ++j) {
                if (j * kPer < kReadsPh)
                    __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
    for (int mt = 0; mt < S::kMT; ++mt) {
        const int m = m0 + (wm * S::kMT + mt) * 16 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < S::kNT; ++nt) {
            const int n = n0 + (wn * S::kNT + nt) * 16 + (lane >> 4) * 4;
            f32x4 v = acc[mt][nt];
            if constexpr (SCALE == kScaleTensor)
                v = v * scale;
            store_tile<OUT>(p, split, m, n, v);
        }
    }
}

template <int DT, int TM, int TN, int WM, int WN, int SCALE, int OUT>
void launch_lds(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    gemm_lds_kernel<DT, TM, TN, WM, WN, SCALE, OUT><<<grid, WM * WN * 64, 0, s>>>(a);
}

#define DGP_LDS(DT, TM, TN, WM, WN, SC, OUT)                                                  \
    {kTiled, DT, SC, OUT, TM, TN, 128, WM * WN, WM, WN, 0, 0, 1, kSchedBothLds,                \
     &launch_lds<DT, TM, TN, WM, WN, SC, OUT>}
#define DGP_LDS_BOTH_OUT(DT, TM, TN, WM, WN, SC)                                              \
    DGP_LDS(DT, TM, TN, WM, WN, SC, kOutBf16), DGP_LDS(DT, TM, TN, WM, WN, SC, kOutPartial)

static const KernelSpec kLdsKernels[] = {
    // (tm, tn, waves m x n, scale)
    DGP_LDS_BOTH_OUT(kDtypeBf16, 256, 256, 2, 4, kScaleNone),
    DGP_LDS_BOTH_OUT(kDtypeFp8, 256, 256, 2, 4, kScaleTensor),
};

const KernelSpec *lds_kernels(int *count)
{
    *count = (int)(sizeof(kLdsKernels) / sizeof(kLdsKernels[0]));
    return kLdsKernels;
}

}  // namespace dgp
