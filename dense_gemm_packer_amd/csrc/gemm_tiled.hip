// Large-M GEMM kernels for C = A * B^T with B preshuffled (include/dgp.h):
// the interleaved gemm_tiled_kernel and the ping-pong schedule of the
// 256 x 256 tile, and their table entries (the both-in-LDS schedule:
// gemm_lds.hip).
// Operand layout and epilogue: gemm_common.h.
//
// gemm_tiled_kernel -- large M (the compute-bound path of FlyDSL PR #1008,
//    "Performance": bf16 preshuffle GEMM, and the fp8 M=N=4096 K=8192 figure on
//    FlyDSL PR #974 "Validation").  A workgroup owns a TM x TN tile of C.  Per
//    k-tile of KT bytes the A tile goes global -> LDS with the async buffer
//    load (no VGPR round trip, FlyDSL PR #1008 "Summary"), double-buffered,
//    while each wave pulls its preshuffled B fragments straight into VGPRs;
//    A fragments are read from LDS per MFMA k-step, interleaved with the
//    MFMAs that consume them (the per-k-step reads restored on FlyDSL PR #974,
//    follow-up commit item 2).
//    fp8 blockscale (fp32 scales per 128-K block, aiter PR #5148) and mxfp8
//    (E8M0 bytes per 128-K block, the hardware-scaled MFMA) take one k-tile
//    per K block: the tile's scales ride in a small area after each A buffer,
//    copied with the same async load as A (one instruction per wave per
//    k-tile), so the wait and barrier that certify A certify them too.

#include "gemm_common.h"

namespace dgp {

// ================================================================ tiled


template <int DT, int TM, int TN, int WM, int WN, int KT, int DEPTH, int SCALE, int OUT, int PV, int PD>
__global__ void __attribute__((amdgpu_flat_work_group_size(WM * WN * 64, WM * WN * 64),
                               amdgpu_waves_per_eu((WM * WN + 3) / 4, (WM * WN + 3) / 4)))
gemm_tiled_kernel(const GemmArgs p)
{
    using S = TiledShape<DT, TM, TN, WM, WN, KT>;
    using Frag = typename Op<DT>::Frag;
    // Per-k-tile scales staged in LDS: fp32 (blockscale) or E8M0 bytes (mxfp8).
    // The scale area after an A buffer holds TM + TN dwords: dword d < TM is
    // A row (d % (TM/16))*16 + d / (TM/16) of the tile, dword TM + d is B
    // column (d % (TN/16))*16 + d / (TN/16); so a lane's scales for its row
    // tiles (column strips) are consecutive dwords.  An E8M0 byte lands in
    // the low byte of its dword (the narrow async load writes lane l at dword
    // l), which is the byte the scaled MFMA reads.
    // mxfp4: a 128-byte k-tile is 256 elements, 8 E8M0 bytes per row (one per
    // 32-element block), copied as 2 dwords per row: dword 2r + j of the
    // area is bytes 4j..4j+3 of tile row r, dword 2*TM + 2c + j the same for
    // column c -- the byte order of the [rows][K/32] scale arrays.
    constexpr bool kX4 = SCALE == kScaleMx32;
    constexpr bool kXS = SCALE == kScaleBlock || SCALE == kScaleMx || kX4;
    constexpr int kES = SCALE == kScaleMx ? 1 : 4;             // bytes per scale copy
    constexpr int kXDwords = kX4 ? 2 * (TM + TN) : kXS ? TM + TN : 0;
    constexpr int kXDma = kXDwords / (64 * S::kWaves);        // scale copies per wave per k-tile
    static_assert(!kXS || (KT == 128 && kXDwords % (64 * S::kWaves) == 0 && TM % 64 == 0 &&
                           (kX4 ? DT == kDtypeFp4 : DT == kDtypeFp8 && S::kMT % 4 == 0) &&
                           (S::kNT == 2 || S::kNT == 4)),
                  "staged scales: one 128-byte k-tile per scale stage, whole copies per wave");
    constexpr int kStageBytes = S::kBufBytes + kXDwords * 4;
    static_assert(DEPTH >= 1 && (DEPTH + 1) * kStageBytes <= 160 * 1024, "A ring must fit in LDS");
    // Prefetch distance DEPTH k-tiles: a ring of DEPTH+1 A buffers in LDS and
    // DEPTH sets of B registers.
    constexpr int kRing = DEPTH + 1;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * kStageBytes];
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

    // A: rows m0.. of A; rows >= M are past num_records and load as zero.
    const auto rA = make_rsrc(p.A + (int64_t)m0 * Kb, clamp_bytes((int64_t)(p.M - m0) * Kb));
    // Where the copy puts each lane's 16 bytes: instruction j of this wave
    // fills LDS block blk = j*waves + wave = (row group rg, 64-byte chunk ch),
    // lane l landing at byte 16*l with row 16*rg + l%16, K-bytes
    // 64*ch + 16*(l/16) -- the lane's global address selects the bytes.
    uint32_t dma_voff[S::kDmaPerWave];
#pragma unroll
    for (int j = 0; j < S::kDmaPerWave; ++j) {
        const int blk = j * S::kWaves + wave;
        const int rg = blk / S::kCH, ch = blk % S::kCH;
        dma_voff[j] = (uint32_t)(rg * 16 + (lane & 15)) * Kb + (uint32_t)(ch * 64 + (lane >> 4) * 16);
    }
    // B: this wave's strips; strips >= N/16 are past num_records and load as zero.
    const int strip0 = (n0 + wn * (TN / WN)) / 16;
    const auto rB = make_rsrc(p.Bs + (int64_t)strip0 * 16 * Kb,
                              clamp_bytes((int64_t)(p.N / 16 - strip0) * 16 * Kb));
    uint32_t b_voff[S::kNT];
#pragma unroll
    for (int nt = 0; nt < S::kNT; ++nt)
        b_voff[nt] = (uint32_t)nt * 16u * Kb + (uint32_t)lane * 16u;

    // Scale copies: instruction j of this wave fills dwords 64g .. 64g+63 of
    // the scale area (g = j*waves + wave); lane l supplies dword 64g + l.
    // Rows >= M and (blockscale) column blocks past N load as zero.
    [[maybe_unused]] __amdgpu_buffer_rsrc_t x_rsrc[kXDma > 0 ? kXDma : 1];
    [[maybe_unused]] uint32_t x_voff[kXDma > 0 ? kXDma : 1];
    if constexpr (kX4) {
        const uint32_t rowb = Kb / 16u;    // E8M0 bytes per row: one per 32 elements = 16 bytes
        const auto rXA = make_rsrc((const uint8_t *)p.sA + (int64_t)m0 * rowb,
                                   clamp_bytes((int64_t)(p.M - m0) * rowb));
        const auto rXB = make_rsrc((const uint8_t *)p.sB + (int64_t)n0 * rowb,
                                   clamp_bytes((int64_t)(p.N - n0) * rowb));
#pragma unroll
        for (int j = 0; j < kXDma; ++j) {
            const int g = j * S::kWaves + wave;
            const bool on_a = g * 64 < 2 * TM;
            const int d = (on_a ? g * 64 : g * 64 - 2 * TM) + lane;
            x_rsrc[j] = on_a ? rXA : rXB;
            x_voff[j] = (uint32_t)(d >> 1) * rowb + 4u * (uint32_t)(d & 1);
        }
    } else if constexpr (kXS) {
        const uint32_t kblk = Kb / 128u;   // 128-K blocks per row (fp8: one byte per element)
        const auto rXA = make_rsrc((const uint8_t *)p.sA + (int64_t)m0 * kblk * kES,
                                   clamp_bytes((int64_t)(p.M - m0) * kblk * kES));
        const int64_t bcol0 = SCALE == kScaleBlock ? n0 / 128 : n0;   // first sB row of the tile
        const int64_t brows = SCALE == kScaleBlock ? p.N / 128 : p.N;
        const auto rXB = make_rsrc((const uint8_t *)p.sB + bcol0 * kblk * kES,
                                   clamp_bytes((brows - bcol0) * kblk * kES));
#pragma unroll
        for (int j = 0; j < kXDma; ++j) {
            const int g = j * S::kWaves + wave;
            if (g * 64 < TM) {
                const int d = g * 64 + lane;
                const int row = (d % (TM / 16)) * 16 + d / (TM / 16);
                x_rsrc[j] = rXA;
                x_voff[j] = (uint32_t)row * kblk * kES;
            } else {
                const int d = g * 64 - TM + lane;
                const int col = (d % (TN / 16)) * 16 + d / (TN / 16);
                x_rsrc[j] = rXB;
                x_voff[j] = (uint32_t)(SCALE == kScaleBlock ? col / 128 : col) * kblk * kES;
            }
        }
    }

    f32x4 acc[S::kMT][S::kNT];
#pragma unroll
    for (int i = 0; i < S::kMT; ++i)
#pragma unroll
        for (int j = 0; j < S::kNT; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B registers: DEPTH sets.  The fragments of chunk c of k-tile t (set
    // t % DEPTH) are reloaded with chunk c of tile t+DEPTH as soon as the MFMAs
    // of chunk c have consumed them, so every B load has DEPTH whole k-tiles
    // of compute to land in.
    i32x4 breg[DEPTH][S::kNT][S::kCH];

    auto load_b = [&](auto setc, int ch, uint32_t koff) {
        constexpr int SET = decltype(setc)::value;
#pragma unroll
        for (int nt = 0; nt < S::kNT; ++nt)
            breg[SET][nt][ch] = load16<kAuxNone>(rB, b_voff[nt] + ch * 1024 + koff * 16u);
    };
    auto dma_a = [&](uint32_t buf_off, uint32_t koff) {
#pragma unroll
        for (int j = 0; j < S::kDmaPerWave; ++j)
            lds_dma16(rA, lds + buf_off + (j * S::kWaves + wave) * 1024, dma_voff[j], koff);
        if constexpr (kXS) {
#pragma unroll
            for (int j = 0; j < kXDma; ++j) {
                uint8_t *d = lds + buf_off + S::kBufBytes + (j * S::kWaves + wave) * 256;
                if constexpr (kX4)
                    lds_dma<4>(x_rsrc[j], d, x_voff[j], koff / 16u);
                else if constexpr (kES == 4)
                    lds_dma<4>(x_rsrc[j], d, x_voff[j], (koff / 128u) * 4u);
                else
                    lds_dma<1>(x_rsrc[j], d, x_voff[j], koff / 128u);
            }
        }
    };
    auto kofs = [&](int t) {   // first K byte of tile t, clamped to the last tile
        return kbase + (uint32_t)(t < ntiles ? t : ntiles - 1) * KT;
    };

    // Prologue: A and B of tiles 0..DEPTH-1, in the exact order the loop body
    // issues them (A copy, then B chunk by chunk), so the compiler's load
    // counters agree on the loop-entry and back-edge paths.
    auto prologue_tile = [&](auto setc) {
        constexpr int D = decltype(setc)::value;
        dma_a((uint32_t)D * kStageBytes, kofs(D));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ch = 0; ch < S::kCH; ++ch) {
            load_b(setc, ch, kofs(D));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    prologue_tile(std::integral_constant<int, 0>{});
    if constexpr (DEPTH > 1)
        prologue_tile(std::integral_constant<int, (DEPTH > 1 ? 1 : 0)>{});
    if constexpr (DEPTH > 2)
        prologue_tile(std::integral_constant<int, (DEPTH > 2 ? 2 : 0)>{});
    if constexpr (DEPTH > 3)
        prologue_tile(std::integral_constant<int, (DEPTH > 3 ? 3 : 0)>{});
    static_assert(DEPTH <= 4, "prologue and loop unrolled for DEPTH <= 4");

    // Loads issued after the A (and scale) copy of tile t, when step t
    // begins: the B loads of tile t, then DEPTH-1 more tiles of A copies,
    // scale copies and B loads.
    constexpr int kAfter = S::kBLoads + (DEPTH - 1) * (S::kDmaPerWave + kXDma + S::kBLoads);
    static_assert(kAfter <= 63, "vmcnt field is 6 bits");

    uint32_t cur = 0;                                   // LDS offset of tile t
    uint32_t nxt = (uint32_t)DEPTH * kStageBytes;       // LDS offset of tile t+DEPTH
    // Blockscale k-tile (one 128-K scale block per k-tile).  Each fragment's
    // MFMAs start from a zero accumulator; the fp32 partial is multiplied by
    // sA[row][kb] * sB[col / 128][kb] and added to the running sum in one
    // fused multiply-add (one rounding per block).  The order
    // is fixed by scheduling fences, one fragment at a time: issue the LDS
    // reads (A fragment and the row's A scale) of fragment f + PD, issue the
    // MFMAs of fragment f, then scale and add the partials of fragment f - 1,
    // whose MFMAs completed while those of f were issued (the scaling of
    // each column strip follows the MFMA of the same strip of fragment f).
    // So the LDS reads have PD fragments of work to land in and the VALU work
    // never waits on the MFMA that produced its operand.  All columns of a
    // wave lie in one 128-column block (its 16 * kNT columns divide 128), so
    // sB is one value per wave and k-tile.
    [[maybe_unused]] auto block_step = [&](auto setc, uint32_t knext) {
        if constexpr (SCALE == kScaleBlock) {
            constexpr int SET = decltype(setc)::value;
            static_assert(DT == kDtypeFp8 && S::kSteps == 1 && PD >= 1, "blockscale: one fp8 MFMA step per k-tile");
            static_assert(128 % (16 * S::kNT) == 0, "a wave's columns in one block");
            constexpr int kFr = S::kMT;
            constexpr int kRA = PD < kFr ? PD : kFr;
            constexpr int kR = kRA + 1;                        // fragment ring slots
            const uint8_t *abase = lds + cur + (wm * S::kMT * S::kCH) * 1024 + lane * 16;
            const uint8_t *xs = lds + cur + S::kBufBytes;
            const uint8_t *xap = xs + ((lane & 15) * (TM / 16) + wm * S::kMT) * 4;
            const float sb =
                *reinterpret_cast<const float *>(xs + TM * 4 + ((lane & 15) * (TN / 16) + wn * S::kNT) * 4);
            Frag ring[kR];
            float ra[kR];
            auto fetch = [&](int f) {
                ring[f % kR] = lds_frag<DT>(abase + f * S::kCH * 1024);
                ra[f % kR] = *reinterpret_cast<const float *>(xap + 4 * f);
            };
            __builtin_amdgcn_sched_barrier(0);   // sB first: the first product needs it
#pragma unroll
            for (int f = 0; f < kRA; ++f) {
                fetch(f);
                __builtin_amdgcn_sched_barrier(0);
            }
            f32x4 part[2][S::kNT];
            float sc[2];
#pragma unroll
            for (int f = 0; f < kFr; ++f) {
                if (f + kRA < kFr)
                    fetch(f + kRA);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < S::kNT; ++nt) {
                    part[f & 1][nt] = mfma_op(cat(breg[SET][nt][0], breg[SET][nt][1]), ring[f % kR],
                                              f32x4{0.f, 0.f, 0.f, 0.f});
                    if (nt == 0)
                        sc[f & 1] = __fmul_rn(ra[f % kR], sb);
                    if (f == kFr - 1 && nt == S::kNT - 1) {
#pragma unroll
                        for (int cc = 0; cc < S::kStepCh; ++cc)
                            load_b(setc, cc, knext);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (f > 0) {
                        f32x4 &a = acc[f - 1][nt];
                        const f32x4 &q = part[(f - 1) & 1][nt];
                        const float c = sc[(f - 1) & 1];
                        a.x = __builtin_fmaf(q.x, c, a.x);
                        a.y = __builtin_fmaf(q.y, c, a.y);
                        a.z = __builtin_fmaf(q.z, c, a.z);
                        a.w = __builtin_fmaf(q.w, c, a.w);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int nt = 0; nt < S::kNT; ++nt) {
                f32x4 &a = acc[kFr - 1][nt];
                const f32x4 &q = part[(kFr - 1) & 1][nt];
                const float c = sc[(kFr - 1) & 1];
                a.x = __builtin_fmaf(q.x, c, a.x);
                a.y = __builtin_fmaf(q.y, c, a.y);
                a.z = __builtin_fmaf(q.z, c, a.z);
                a.w = __builtin_fmaf(q.w, c, a.w);
            }
        }
    };

    // mxfp4 k-tile: two 128-element MFMA steps, 32 fragments (step-major,
    // as in the other modes).  Lane l's 16-byte fragment is one 32-element
    // block of its row, block 4*step + l/16 of the k-tile, whose E8M0 byte is
    // byte l/16 of the row's scale dword for that step.  Same fenced order as
    // the blockscale k-tile: LDS reads (fragment and scale dword) PD
    // fragments ahead, then the fragment's MFMAs.
    [[maybe_unused]] auto mx4_step = [&](auto setc, uint32_t knext) {
        if constexpr (SCALE == kScaleMx32) {
            constexpr int SET = decltype(setc)::value;
            static_assert(DT == kDtypeFp4 && S::kStepCh == 1 && PD >= 1, "mxfp4: one 64-byte chunk per MFMA step");
            constexpr int kFr = S::kSteps * S::kMT;
            constexpr int kRA = PD < kFr ? PD : kFr;
            constexpr int kR = kRA + 1;                        // fragment ring slots
            const int rit = lane & 15;
            const uint32_t sh = 8u * (uint32_t)(lane >> 4);
            const uint8_t *abase = lds + cur + (wm * S::kMT * S::kCH) * 1024 + lane * 16;
            const uint8_t *xs = lds + cur + S::kBufBytes;
            const uint8_t *xap = xs + ((wm * S::kMT * 16 + rit) * 2) * 4;
            const uint8_t *xbp = xs + 2 * TM * 4 + ((wn * S::kNT * 16 + rit) * 2) * 4;
            int eb[S::kNT][S::kSteps];
#pragma unroll
            for (int nt = 0; nt < S::kNT; ++nt)
#pragma unroll
                for (int st = 0; st < S::kSteps; ++st)
                    eb[nt][st] = (int)((*reinterpret_cast<const uint32_t *>(xbp + (nt * 32 + st) * 4) >> sh) & 0xFFu);
            Frag ring[kR];
            uint32_t ra[kR];
            auto fetch = [&](int f) {
                const int st = f / S::kMT, mt = f % S::kMT;
                ring[f % kR] = lds_frag<DT>(abase + (mt * S::kCH + st) * 1024);
                ra[f % kR] = *reinterpret_cast<const uint32_t *>(xap + (mt * 32 + st) * 4);
            };
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int f = 0; f < kRA; ++f) {
                fetch(f);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int f = 0; f < kFr; ++f) {
                const int st = f / S::kMT, mt = f % S::kMT;
                if (f + kRA < kFr)
                    fetch(f + kRA);
                __builtin_amdgcn_sched_barrier(0);
                const int ea = (int)((ra[f % kR] >> sh) & 0xFFu);
#pragma unroll
                for (int nt = 0; nt < S::kNT; ++nt)
                    acc[mt][nt] = mfma_mx4(breg[SET][nt][st], ring[f % kR], acc[mt][nt], eb[nt][st], ea);
                if (mt == S::kMT - 1)
                    load_b(setc, st, knext);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    auto step = [&](auto setc, int t) {
        // This wave's A copy of tile t has landed once at most kAfter loads are
        // outstanding, and every earlier LDS read has completed; the barrier
        // certifies both for all waves, so tile t is readable and the buffer
        // of tile t-1 is free for tile t+DEPTH.
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kAfter) : "memory");
        const uint32_t knext = kofs(t + DEPTH);
        dma_a(nxt, knext);

        constexpr int SET = decltype(setc)::value;
        if constexpr (SCALE == kScaleBlock) {
            block_step(setc, knext);
        } else if constexpr (SCALE == kScaleMx32) {
            mx4_step(setc, knext);
        } else {
            // mxfp8: this tile's E8M0 scales, the lane's row tiles (A) and column strips (B).
            [[maybe_unused]] i32x4 xa[kXS ? S::kMT / 4 : 1];
            [[maybe_unused]] int xb[kXS ? S::kNT : 1];
            if constexpr (kXS) {
                const uint8_t *xs = lds + cur + S::kBufBytes;
                const int rit = lane & 15;
#pragma unroll
                for (int q = 0; q < S::kMT / 4; ++q)
                    xa[q] = *reinterpret_cast<const i32x4 *>(xs + (rit * (TM / 16) + wm * S::kMT) * 4 + 16 * q);
                const uint8_t *xbp = xs + TM * 4 + (rit * (TN / 16) + wn * S::kNT) * 4;
                if constexpr (S::kNT == 2) {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(xbp);
                    xb[0] = (int)v.x;
                    xb[1] = (int)v.y;
                } else {
                    const i32x4 v = *reinterpret_cast<const i32x4 *>(xbp);
#pragma unroll
                    for (int nt = 0; nt < S::kNT; ++nt)
                        xb[nt] = v[nt];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            const uint8_t *abase = lds + cur + (wm * S::kMT * S::kCH) * 1024 + lane * 16;
            // A fragments in MFMA order: fragment f = (step f / kMT, row tile f % kMT).
            constexpr int kFr = S::kSteps * S::kMT;
            auto frag_at = [&](int f) {
                return lds_frag<DT>(abase + ((f % S::kMT) * S::kCH + (f / S::kMT) * S::kStepCh) * 1024);
            };
#pragma unroll
            for (int f = 0; f < kFr; ++f) {
                const int st = f / S::kMT, mt = f % S::kMT;
                const Frag a = frag_at(f);
#pragma unroll
                for (int nt = 0; nt < S::kNT; ++nt) {
                    Frag b;
                    if constexpr (DT == kDtypeBf16)
                        b = breg[SET][nt][st];
                    else
                        b = cat(breg[SET][nt][2 * st], breg[SET][nt][2 * st + 1]);
                    if constexpr (SCALE == kScaleMx) {
                        acc[mt][nt] = mfma_mx(b, a, acc[mt][nt], xb[nt], xa[mt / 4][mt % 4]);
                    } else {
                        acc[mt][nt] = mfma_op(b, a, acc[mt][nt]);
                    }
                }
                if (mt == S::kMT - 1) {
#pragma unroll
                    for (int cc = 0; cc < S::kStepCh; ++cc)
                        load_b(setc, st * S::kStepCh + cc, knext);
                }
            }
            if constexpr (PD > 0) {
                // Software-pipeline the A fragments: the LDS reads of PD fragments
                // first, then for every fragment its MFMAs followed by the reads of
                // the fragment PD places ahead -- each read gets PD fragments'
                // worth of MFMAs to land.  With PV > 0, one global load (B reload
                // or A copy) is placed after every PV MFMAs.
                constexpr int kRA = PD < kFr ? PD : kFr;
                constexpr int kRd = S::kStepCh;   // LDS reads per fragment
                __builtin_amdgcn_sched_group_barrier(0x100, kRA * kRd, 0);
#pragma unroll
                for (int f = 0; f < kFr; ++f) {
                    if constexpr (PV > 0) {
                        static_assert(PV <= S::kNT && S::kNT % PV == 0, "PV must divide the MFMAs per fragment");
#pragma unroll
                        for (int m = 0; m < S::kNT / PV; ++m) {
                            __builtin_amdgcn_sched_group_barrier(0x008, PV, 0);
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                        }
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x008, S::kNT, 0);
                    }
                    if (f + kRA < kFr)
                        __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
                }
            }
        }
        cur = cur + kStageBytes == kRing * kStageBytes ? 0 : cur + kStageBytes;
        nxt = nxt + kStageBytes == kRing * kStageBytes ? 0 : nxt + kStageBytes;
    };

    // Main loop, unrolled by DEPTH so that the B register set of every step is
    // a compile-time index; the remaining ntiles % DEPTH steps follow.
    int t = 0;
    for (; t + DEPTH <= ntiles; t += DEPTH) {
        step(std::integral_constant<int, 0>{}, t);
        if constexpr (DEPTH > 1)
            step(std::integral_constant<int, (DEPTH > 1 ? 1 : 0)>{}, t + 1);
        if constexpr (DEPTH > 2)
            step(std::integral_constant<int, (DEPTH > 2 ? 2 : 0)>{}, t + 2);
        if constexpr (DEPTH > 3)
            step(std::integral_constant<int, (DEPTH > 3 ? 3 : 0)>{}, t + 3);
    }
    if constexpr (DEPTH > 1)
        if (t < ntiles)
            step(std::integral_constant<int, 0>{}, t++);
    if constexpr (DEPTH > 2)
        if (t < ntiles)
            step(std::integral_constant<int, (DEPTH > 2 ? 1 : 0)>{}, t++);
    if constexpr (DEPTH > 3)
        if (t < ntiles)
            step(std::integral_constant<int, (DEPTH > 3 ? 2 : 0)>{}, t++);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue: scale once, round once.  The per-tensor scales are loaded
    // here, not before the loop: a scalar load still in flight at the loop
    // would make the compiler wait for every LDS read (lgkmcnt(0)) before the
    // first MFMA of each unrolled loop body.
    float scale = 1.0f;
    if constexpr (SCALE == kScaleTensor)
        scale = static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0];
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

// ============================================================ ping-pong

// gemm_pingpong_kernel -- the 256 x 256 tile of gemm_tiled_kernel (8 waves,
// each owning 256 rows x 32 columns, 128-byte k-tiles, a ring of three A
// buffers in LDS, preshuffled B straight into VGPRs) with a different
// schedule.  Every k-tile is cut into two phases of 512 matrix-core cycles
// per wave: bf16 phase p is MFMA k-step p over all 16 row tiles, fp8 phase p
// is the single 128-deep k-step over row tiles 8p..8p+7.  A phase is split
// into a memory part M -- issue this phase's share of the global loads, read
// the phase's 16 A fragments from LDS and wait for them -- and a compute part
// C that only issues MFMAs.  Waves 0-3 (one per SIMD) and waves 4-7 (the
// other wave of each SIMD) run half a phase apart, separated by workgroup
// barriers, so on every SIMD one wave issues an unbroken run of MFMAs while
// the other does its memory work: the memory instructions and their waits
// never sit in front of a ready MFMA.  Between two barriers group 0 is in
// M(t,p) while group 1 is in C of the phase before, and the other way round.
//
// Load pipeline per wave (program order, vmcnt counts in-order completion):
// the prologue issues A(0), then [B(0) half 0, A(1) half 0], [B(0) half 1,
// A(1) half 1]; M(t,p) issues [B(t+1) half p, A(t+2) half p] (2 + 2 loads;
// half p of B is the 64-byte chunk p, half p of A is copy instructions 2p,
// 2p+1).  At the end of M(t,0), vmcnt(6) means B(t) has landed; at the end of
// M(t,1), vmcnt(8) means this wave's A(t+1) copy has landed, and the barrier
// that follows (before any wave reads tile t+1) makes that hold for all
// waves.  A(t+2) goes to the buffer of tile t-1, whose last reader (group 1,
// M(t-1,1)) finished before the barrier that opens M(t,0).
template <int DT, int SCALE, int OUT>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
gemm_pingpong_kernel(const GemmArgs p)
{
    constexpr int TM = 256, TN = 256, WM = 1, WN = 8, KT = 128;
    using S = TiledShape<DT, TM, TN, WM, WN, KT>;
    using Frag = typename Op<DT>::Frag;
    static_assert(S::kCH == 2 && S::kNT == 2 && S::kMT == 16 && S::kDmaPerWave == 4, "fixed shape");
    constexpr int kRing = 3;
    constexpr int kFrP = DT == kDtypeBf16 ? 16 : 8;   // A fragments per phase: 16 LDS reads either way
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * S::kBufBytes];
    if constexpr (kLdsPoison) {   // debug build: all of LDS poisoned before the first copy
        lds_poison_fill(lds, (int)sizeof(lds));
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const auto tc = tile_of_workgroup<int>((int)blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.remap, p.group_m);
    const int m0 = (int)tc.tm * TM;
    const int n0 = (int)tc.tn * TN;
    const int split = (int)tc.s;
    const uint32_t Kb = (uint32_t)p.Kb;
    const uint32_t kbase = (uint32_t)split * (uint32_t)p.Ks;
    const int ntiles = p.Ks / KT;

    // A copy: instruction j of this wave fills LDS block blk = j*8 + wave
    // (row group blk/2, 64-byte chunk blk%2), as in gemm_tiled_kernel.
    const auto rA = make_rsrc(p.A + (int64_t)m0 * Kb, clamp_bytes((int64_t)(p.M - m0) * Kb));
    uint32_t dma_voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int blk = j * 8 + wave;
        dma_voff[j] = (uint32_t)((blk / 2) * 16 + (lane & 15)) * Kb + (uint32_t)((blk % 2) * 64 + (lane >> 4) * 16);
    }
    const int strip0 = (n0 + wave * 32) / 16;
    const auto rB = make_rsrc(p.Bs + (int64_t)strip0 * 16 * Kb,
                              clamp_bytes((int64_t)(p.N / 16 - strip0) * 16 * Kb));
    uint32_t b_voff[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
        b_voff[nt] = (uint32_t)nt * 16u * Kb + (uint32_t)lane * 16u;

    float scale = 1.0f;
    if constexpr (SCALE == kScaleTensor)
        scale = static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0];

    f32x4 acc[16][2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 breg[2][2][2];   // [set = tile % 2][strip][64-byte chunk]
    Frag fr[kFrP];

    auto kofs = [&](int t) { return kbase + (uint32_t)(t < ntiles ? t : ntiles - 1) * KT; };
    auto load_b_half = [&](auto setc, int h, uint32_t koff) {
        constexpr int SET = decltype(setc)::value;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            breg[SET][nt][h] = load16<kAuxNone>(rB, b_voff[nt] + h * 1024 + koff * 16u);
    };
    auto dma_half = [&](uint32_t buf_off, int h, uint32_t koff) {
#pragma unroll
        for (int j = 2 * h; j < 2 * h + 2; ++j)
            lds_dma16(rA, lds + buf_off + (j * 8 + wave) * 1024, dma_voff[j], koff);
    };
    auto read_frags = [&](uint32_t buf_off, int ph) {
        const uint8_t *abase = lds + buf_off + lane * 16;
#pragma unroll
        for (int f = 0; f < kFrP; ++f) {
            if constexpr (DT == kDtypeBf16)
                fr[f] = lds_frag<DT>(abase + (f * 2 + ph) * 1024);
            else
                fr[f] = lds_frag<DT>(abase + ((8 * ph + f) * 2) * 1024);
        }
    };
    auto compute = [&](auto setc, auto phc) {
        constexpr int SET = decltype(setc)::value, PH = decltype(phc)::value;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < kFrP; ++f) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                if constexpr (DT == kDtypeBf16)
                    acc[f][nt] = mfma_op(breg[SET][nt][PH], fr[f], acc[f][nt]);
                else
                    acc[8 * PH + f][nt] = mfma_op(cat(breg[SET][nt][0], breg[SET][nt][1]), fr[f],
                                                  acc[8 * PH + f][nt]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Prologue: A(0); then B(0) and A(1) in the per-phase order.
    dma_half(0, 0, kofs(0));
    dma_half(0, 1, kofs(0));
    __builtin_amdgcn_sched_barrier(0);
    load_b_half(std::integral_constant<int, 0>{}, 0, kofs(0));
    dma_half(S::kBufBytes, 0, kofs(1));
    __builtin_amdgcn_sched_barrier(0);
    load_b_half(std::integral_constant<int, 0>{}, 1, kofs(0));
    dma_half(S::kBufBytes, 1, kofs(1));
    __builtin_amdgcn_sched_barrier(0);
    // A(0) has landed for every wave.
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (wave >= 4)   // group 1 starts half a phase behind
        asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    uint32_t cur = 0;                          // LDS offset of tile t
    uint32_t nxt = 2u * S::kBufBytes;          // LDS offset of tile t+2
    auto tile_step = [&](auto setc, int t) {
        constexpr int SET = decltype(setc)::value;
        const std::integral_constant<int, SET ^ 1> nset{};
        const uint32_t kb1 = kofs(t + 1), ka2 = kofs(t + 2);
        // M(t,0)
        load_b_half(nset, 0, kb1);
        dma_half(nxt, 0, ka2);
        read_frags(cur, 0);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // C(t,0)
        compute(setc, std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // M(t,1)
        load_b_half(nset, 1, kb1);
        dma_half(nxt, 1, ka2);
        read_frags(cur, 1);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // C(t,1)
        compute(setc, std::integral_constant<int, 1>{});
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        cur = cur + S::kBufBytes == kRing * S::kBufBytes ? 0 : cur + S::kBufBytes;
        nxt = nxt + S::kBufBytes == kRing * S::kBufBytes ? 0 : nxt + S::kBufBytes;
    };

    int t = 0;
    for (; t + 2 <= ntiles; t += 2) {
        tile_step(std::integral_constant<int, 0>{}, t);
        tile_step(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < ntiles)
        tile_step(std::integral_constant<int, 0>{}, t);
    if (wave < 4)   // group 0 matches group 1's extra barrier
        asm volatile("s_barrier" ::: "memory");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
    for (int mt = 0; mt < 16; ++mt) {
        const int m = m0 + mt * 16 + (lane & 15);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = n0 + (wave * 2 + nt) * 16 + (lane >> 4) * 4;
            f32x4 v = acc[mt][nt];
            if constexpr (SCALE == kScaleTensor)
                v = v * scale;
            store_tile<OUT>(p, split, m, n, v);
        }
    }
}

template <int DT, int TM, int TN, int WM, int WN, int KT, int DEPTH, int SCALE, int OUT, int PV, int PD>
void launch_tiled(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    gemm_tiled_kernel<DT, TM, TN, WM, WN, KT, DEPTH, SCALE, OUT, PV, PD><<<grid, WM * WN * 64, 0, s>>>(a);
}

template <int DT, int SCALE, int OUT>
void launch_pingpong(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    gemm_pingpong_kernel<DT, SCALE, OUT><<<grid, 512, 0, s>>>(a);
}

#define DGP_TILED(DT, TM, TN, WM, WN, KT, DEPTH, SC, OUT, PV, PD)                            \
    {kTiled, DT, SC, OUT, TM, TN, KT, WM * WN, WM, WN, PV, PD, DEPTH, kSchedInterleaved,      \
     &launch_tiled<DT, TM, TN, WM, WN, KT, DEPTH, SC, OUT, PV, PD>}
#define DGP_PINGPONG(DT, SC, OUT)                                                             \
    {kTiled, DT, SC, OUT, 256, 256, 128, 8, 1, 8, 0, 0, 2, kSchedPingPong,                     \
     &launch_pingpong<DT, SC, OUT>}
#define DGP_TILED_BOTH_OUT(DT, TM, TN, WM, WN, KT, DEPTH, SC, PV, PD)                         \
    DGP_TILED(DT, TM, TN, WM, WN, KT, DEPTH, SC, kOutBf16, PV, PD),                           \
        DGP_TILED(DT, TM, TN, WM, WN, KT, DEPTH, SC, kOutPartial, PV, PD)
#define DGP_PINGPONG_BOTH_OUT(DT, SC) DGP_PINGPONG(DT, SC, kOutBf16), DGP_PINGPONG(DT, SC, kOutPartial)

static const KernelSpec kTiledKernels[] = {
    // large tiles, bf16 (tm, tn, waves m x n, k-tile bytes, prefetch depth, scale, preload pair);
    // within one tile the first entry is the tuned default
    DGP_TILED_BOTH_OUT(kDtypeBf16, 256, 256, 1, 8, 128, 2, kScaleNone, 0, 8),
    DGP_PINGPONG_BOTH_OUT(kDtypeBf16, kScaleNone),
    DGP_TILED_BOTH_OUT(kDtypeBf16, 256, 256, 2, 4, 128, 2, kScaleNone, 0, 8),
    DGP_TILED_BOTH_OUT(kDtypeBf16, 128, 256, 1, 4, 128, 2, kScaleNone, 0, 8),
    DGP_TILED_BOTH_OUT(kDtypeBf16, 128, 128, 2, 2, 128, 2, kScaleNone, 0, 4),
    // large tiles, fp8 per-tensor
    DGP_TILED_BOTH_OUT(kDtypeFp8, 256, 256, 1, 8, 128, 2, kScaleTensor, 0, 8),
    DGP_PINGPONG_BOTH_OUT(kDtypeFp8, kScaleTensor),
    DGP_TILED_BOTH_OUT(kDtypeFp8, 256, 256, 2, 4, 128, 2, kScaleTensor, 0, 8),
    DGP_TILED_BOTH_OUT(kDtypeFp8, 128, 256, 1, 4, 128, 2, kScaleTensor, 0, 8),
    DGP_TILED_BOTH_OUT(kDtypeFp8, 128, 128, 2, 2, 128, 2, kScaleTensor, 0, 4),
    // large tiles, fp8 blockscale and mxfp8 (scales staged per k-tile)
    // (LDS read-ahead 4 fragments: the staged scales leave no registers for
    // 8; measured equal to 2 and 6)
    DGP_TILED_BOTH_OUT(kDtypeFp8, 256, 256, 1, 8, 128, 2, kScaleBlock, 0, 4),
    DGP_TILED_BOTH_OUT(kDtypeFp8, 128, 128, 2, 2, 128, 2, kScaleBlock, 0, 4),
    DGP_TILED_BOTH_OUT(kDtypeFp8, 256, 256, 1, 8, 128, 2, kScaleMx, 0, 4),
    DGP_TILED_BOTH_OUT(kDtypeFp8, 128, 128, 2, 2, 128, 2, kScaleMx, 0, 4),
    // large tiles, mxfp4 (two 128-element steps and 8 scale bytes per row per k-tile)
    DGP_TILED_BOTH_OUT(kDtypeFp4, 256, 256, 1, 8, 128, 2, kScaleMx32, 0, 8),
    DGP_TILED_BOTH_OUT(kDtypeFp4, 128, 128, 2, 2, 128, 2, kScaleMx32, 0, 4),
};

const KernelSpec *tiled_kernels(int *count)
{
    *count = (int)(sizeof(kTiledKernels) / sizeof(kTiledKernels[0]));
    return kTiledKernels;
}

}  // namespace dgp
