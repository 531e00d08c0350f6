// gemm_w4_kernel -- the large-M tile with one wave per SIMD: 256 x 256 (bf16,
// per-tensor fp8, mxfp8 and mxfp4) and 128 x 256 (bf16 and per-tensor fp8;
// two waves per SIMD when two workgroups share a CU).
//
// Same operation, operand layouts and epilogue as gemm_tiled_kernel
// (gemm_tiled.hip, gemm_common.h): per k-tile of 128 bytes the A tile goes
// global -> LDS with the async buffer load (FlyDSL PR #1008 "Summary"), the
// preshuffled B fragments go straight to VGPRs, and A fragments are read from
// LDS per MFMA k-step (FlyDSL PR #974, follow-up commit item 2).  What
// differs is the split of the workgroup: 4 waves (1 x 4), each owning all 256
// rows and 64 columns of the tile, 256 fp32 accumulators per lane (128 rows and
// 128 accumulators in the 128-row form).  Against
// the 8-wave tile this halves the LDS read traffic (each wave reads the whole
// A tile once per k-tile, and there are half as many waves) while B still
// passes through the L1 exactly once.
//
// Registers.  The accumulators live in the 256 AGPRs and every MFMA is
// issued as inline assembly on its accumulator in place ("+a"), so the
// compiler never moves them between register files.  Because the compiler
// does not see these instructions as MFMAs, the code keeps to inputs whose
// hazards the hardware or s_waitcnt covers: operands come straight from LDS
// or buffer loads into the registers the MFMA reads, an accumulator is only
// reused 64 MFMAs later, and the epilogue waits out the last MFMAs with
// s_nop before reading the AGPRs.
//
// Schedule (one wave per SIMD: nothing else hides a stall, so the order is
// fixed with scheduling fences).  A k-tile is kFr fragments (A fragment f =
// row tile f % 16 of MFMA k-step f / 16), each with its 4 MFMAs (one per
// 16-column strip).  The LDS read of fragment f + 7 is issued after the
// first MFMA of fragment f, global loads after the second and third.  A ring of 4 LDS stages: the workgroup barrier that
// certifies tile t+1 sits 7 fragments before the end of tile t, right where
// the reads of tile t+1 begin, and the copy of tile t+3 (into the stage tile
// t-1 used) follows it.  Every global load has a fixed fragment position, so
// the wait before the barrier is a compile-time count (kVmAtBarrier).
#include "gemm_common.h"

namespace dgp {

namespace w4 {

constexpr int TN = 256, NW = 4, KT = 128;
constexpr int kCH = KT / 64;             // 64-byte chunks per k-tile
constexpr int kRing = 4;                 // LDS stages
constexpr int kRA = 7;                   // tuned LDS read-ahead (fragments ahead of their MFMAs)
// Where a k-tile's A copy is issued: right after the barrier that frees its
// stage, 3 k-tiles ahead (false), or early in the next k-tile, 2 ahead (true).
constexpr bool kDmaLate = false;
constexpr int kDmaAhead = kDmaLate ? 2 : 3;

// WM = waves along M: 1 = the 1 x 4 split (each wave all TM rows, 64
// columns), 2 = 2 x 2 (each wave TM/2 rows, 128 columns).  TM = tile rows:
// 256, or 128 (two workgroups per CU, two waves per SIMD).
template <int DT, int RA, int WM = 1, int TM = 256>
struct Plan {
    static constexpr int kBuf = TM * KT;                  // bytes per LDS stage
    static constexpr int kDma = (TM / 16) * kCH / NW;     // async copies per wave per k-tile
    static_assert((TM * KT) % (NW * 64 * 16) == 0, "A tile must split into whole 16-byte loads");
    static constexpr int kMT = TM / 16 / WM;              // 16-row tiles per wave
    static constexpr int kNT = 4 * WM;                    // 16-column strips per wave
    static constexpr int kStepCh = Op<DT>::kBlocks;       // 64-byte chunks per MFMA step
    static constexpr int kSteps = kCH / kStepCh;          // MFMA k-steps per k-tile
    static constexpr int kFr = kSteps * kMT;              // A fragments per k-tile
    static constexpr int kBar = kFr - RA;                 // barrier position
    static_assert(RA >= 1 && kFr % (RA + 1) == 0, "the fragment ring must wrap at the k-tile boundary");
    // Global loads at fixed fragment positions.  Copy j of tile t+kDmaAhead:
    // after the barrier, spread over the last RA fragments, or (kDmaLate)
    // spread over the fragments before the barrier.
    static constexpr int dma_pos(int j) { return kDmaLate ? (j * kBar) / kDma : kBar + (j * RA) / kDma; }
    // The copy through registers (ablation): the loads sit where the async
    // copies would, their LDS writes RA fragments earlier in the next k-tile
    // (before that k-tile's barrier, which waits for them).
    static constexpr int write_pos(int j) { return dma_pos(j) - RA; }
    // B reloads: the chunks of a step are reloaded for tile t+kDB right after
    // that step's last MFMA -- one load per fragment, starting at the next
    // fragment; the last step's reloads wrap into the next k-tile.
    static constexpr int kBLoads = kNT * kCH;
    static constexpr int bload_pos(int i)   // i = step-major index (step, chunk of step, strip)
    {
        return ((i / (kNT * kStepCh)) * kMT + kMT + i % (kNT * kStepCh)) % kFr;
    }
    static constexpr bool bload_wraps(int i) { return (i / (kNT * kStepCh)) == kSteps - 1; }
    // Loads issued after the last copy of tile t+1 (in tile t+1-kDmaAhead)
    // up to the barrier of tile t+1 (tile t, fragment kBar).  Within a
    // fragment position the B reloads precede the copies.
    static constexpr int vm_at_barrier()
    {
        int n = 0;
        for (int i = 0; i < kBLoads; ++i)   // the copies' tile, after its last copy
            n += bload_pos(i) > dma_pos(kDma - 1) ? 1 : 0;
        n += (kDmaAhead - 2) * (kDma + kBLoads);   // whole k-tiles in between
        for (int i = 0; i < kBLoads; ++i)   // tile t before the barrier
            n += bload_pos(i) < kBar ? 1 : 0;
        for (int j = 0; j < kDma; ++j)
            n += dma_pos(j) < kBar ? 1 : 0;
        return n;
    }
    static_assert(kBar >= kMT || kSteps == 1, "");
};

}  // namespace w4

// acc += B-fragment x A-fragment, in place on AGPRs: bf16 K32 ...
__device__ inline void mfma_acc(f32x4 &acc, const i32x4 &b, const i32x4 &a)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// ... and e4m3 K128 (unscaled form: both operands OCP e4m3).
__device__ inline void mfma_acc(f32x4 &acc, const i32x8 &b, const i32x8 &a)
{
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// ... and the hardware-scaled e4m3 K128 form (mxfp8): eb scales the B
// fragment (first operand: lane l's byte for its column), ea the A fragment
// (its row), both E8M0 in the low byte (op_sel byte 0).
__device__ inline void mfma_acc_mx(f32x4 &acc, const i32x8 &b, const i32x8 &a, int eb, int ea)
{
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(acc)
                 : "v"(b), "v"(a), "v"(eb), "v"(ea));
}

// ... and the hardware-scaled E2M1 K128 form (mxfp4: 16 bytes = 32 values per
// lane, one 32-value block, cbsz = blgp = 4).
__device__ inline void mfma_acc_mx4(f32x4 &acc, const i32x4 &b, const i32x4 &a, int eb, int ea)
{
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                 : "+a"(acc)
                 : "v"(b), "v"(a), "v"(eb), "v"(ea));
}

// DB: B register sets = k-tiles of B loads in flight (2..4).
// RA: A fragments read from LDS ahead of the MFMAs that consume them.
// ILV: 1 = a fragment's 4 MFMAs with one slot of other work between each
// two (the LDS read, the B reloads, the A copies); 0 = all of that work
// first, then the 4 MFMAs.
// SYNC: 0 = A copied global -> LDS by the async buffer load; 1 = through
// registers (buffer load into VGPRs, ds_write a k-tile later): the copy
// path FlyDSL PR #1008 replaced, kept to measure against.
// SWZ: A's LDS layout.  0 = the operand-block order of gemm_common.h (one
// copy instruction = 16 rows x 64 bytes); 1 = row-major 128-byte rows with
// the 16-byte chunks XOR-swizzled (one copy instruction = 8 whole rows, i.e.
// 8 whole 128-byte lines): chunk c of tile row r is stored at chunk
// c ^ ((r >> 1) & 7) of its row, so the 16 rows one fragment read touches
// (rows 16mt + i, one chunk each) fall on 16 distinct 16-byte bank groups
// -- the row-major tile with an XOR swizzle known to writer and reader of
// FlyDSL PR #1008 "Changes" item 2.
//
// mxfp8 (SCALE = kScaleMx): a 128-byte k-tile is one 128-K scale block, so
// each k-tile carries one E8M0 byte per A row (sA [M][K/128]) and per column
// (sB [N][K/128]).  They are staged per stage of the LDS ring beside the A
// tile by two 1-byte async copies per wave (one dword per lane, the byte
// zero-extended), issued with the tile's first A copy so the barrier that
// certifies the tile certifies them.  The staging order lets a lane read its
// scales in 16-byte pieces: A row 16mt + i at dword 16i + mt (a lane reads the
// 4 row tiles of a quad at once, one read per 4 fragments, 4 fragments of
// ring), column 64w + 16s + i at dword 256 + 4(16w + i) + s (one read per
// k-tile, right after the barrier, for the next tile).
//
// mxfp4 (SCALE = kScaleMx32): a 128-byte k-tile is 256 values = 8 blocks of
// 32, two MFMA k-steps whose lane l holds block 4s + l/16 of its row.  Each
// row and column has 2 scale dwords per k-tile (bytes 4s..4s+3 = the blocks
// of step s), staged by 4-byte async copies (2 for rows, 2 for columns per
// wave): row 16mt + i, dword s at dword 2(16i + mt) + s, so a lane reads a
// quad of row tiles' 8 dwords in two 16-byte reads, and column 64w + 16c + i
// at dword 512 + 2(4(16w + i) + c) + s; a lane's byte is taken with one
// bit-field extract per fragment.
template <int DT, int SCALE, int OUT, int DB, int SWZ, int RA, int ILV, int SYNC, int WM, int TM>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(256 / TM, 256 / TM)))
gemm_w4_kernel(const GemmArgs p)
{
    static_assert(DB >= 2 && DB <= 4, "B sets");
    constexpr int kDB = DB;
    using namespace w4;
    static_assert(!SYNC || (SWZ && !kDmaLate), "the register copy: swizzled rows, copies after the barrier");
    constexpr bool kMx = SCALE == kScaleMx;
    constexpr bool kMx4 = SCALE == kScaleMx32;
    static_assert(!kMx || (DT == kDtypeFp8 && SWZ && !SYNC && !kDmaLate), "mxfp8: fp8, swizzled rows, async copies");
    static_assert(!kMx4 || (DT == kDtypeFp4 && SWZ && !SYNC && !kDmaLate), "mxfp4: fp4, swizzled rows, async copies");
    constexpr int kRA = RA;
    static_assert(WM == 1 || WM == 2, "waves along M: 1 (1 x 4) or 2 (2 x 2)");
    static_assert(WM == 1 || !(kMx || kMx4), "the MX scale staging assumes the 1 x 4 split");
    static_assert(TM == 256 || (TM == 128 && !(kMx || kMx4)), "tile rows: 256, or 128 without MX scales");
    using P = Plan<DT, RA, WM, TM>;
    constexpr int kBuf = P::kBuf, kDma = P::kDma;
    constexpr int kMT = P::kMT, kNT = P::kNT;
    using Frag = typename Op<DT>::Frag;
    constexpr int kFr = P::kFr, kBar = P::kBar, kStepCh = P::kStepCh;
    static_assert(!kMx || (kFr == kMT && kMT % 4 == 0 && kRA < kFr - 4), "mxfp8: one k-step per k-tile, quad ring");
    static_assert(!kMx4 || (kFr == 2 * kMT && kRA < kMT - 4), "mxfp4: two k-steps per k-tile, quad ring");
    static_assert(!kMx4 || kFr % 2 == 0, "mxfp4: the row-scale slot of fragment f is f % 2 across k-tiles");
    // The barrier's count: the scale copies of the k-tiles in between are
    // 2 (mxfp8) or 4 (mxfp4) more loads per k-tile (those of the barrier's
    // own tile precede its last A copy).
    constexpr int kXCopies = kMx ? 2 : kMx4 ? 4 : 0;
    constexpr int kVm = P::vm_at_barrier() + kXCopies * (kDmaAhead - 2);
    static_assert(kVm <= 63, "vmcnt field is 6 bits");
    // One LDS object (the A ring, then for mxfp8 the scale stages): the
    // compiler's wait insertion keeps the async copies and the LDS reads of
    // one object apart by their order, where a second object made it wait
    // for every copy in flight before each read.
    constexpr int kXStage = kMx ? 2048 : kMx4 ? 4096 : 0;   // scale bytes per stage
    constexpr int kXBytes = kRing * kXStage;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * kBuf + kXBytes];
    if constexpr (kLdsPoison) {   // debug build: all of LDS poisoned before the first copy
        lds_poison_fill(lds, (int)sizeof(lds));
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // This wave's place in the tile: rows wm*TM/WM.., columns wn*64*WM..
    const int wm = WM == 1 ? 0 : wave / 2, wn = WM == 1 ? wave : wave % 2;
    const auto tc = tile_of_workgroup<int>((int)blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.remap, p.group_m);
    const int m0 = (int)tc.tm * TM;
    const int n0 = (int)tc.tn * TN;
    const int split = (int)tc.s;
    const uint32_t Kb = (uint32_t)p.Kb;
    const uint32_t kbase = (uint32_t)split * (uint32_t)p.Ks;
    const int ntiles = p.Ks / KT;

    // A copy: instruction j of this wave fills LDS block j*NW + wave = (row
    // group rg, 64-byte chunk ch); lane l's global address selects row
    // 16*rg + l%16, K-bytes 64*ch + 16*(l/16) (the operand-block order of
    // gemm_common.h).  Rows >= M are past the range and load as zero.
    const auto rA = make_rsrc(p.A + (int64_t)m0 * Kb, clamp_bytes((int64_t)(p.M - m0) * Kb));
    uint32_t dma_voff[kDma];
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
        const int blk = j * NW + wave;
        if constexpr (SWZ) {
            // instruction j fills rows 8*blk .. 8*blk+7 (1 KiB, linear): lane l
            // lands at row 8*blk + l/8, stored chunk l%8, so it fetches logical
            // chunk (l%8) ^ swizzle(row)
            const int r = 8 * blk + (lane >> 3);
            dma_voff[j] = (uint32_t)r * Kb + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
        } else {
            dma_voff[j] = (uint32_t)((blk / kCH) * 16 + (lane & 15)) * Kb +
                          (uint32_t)((blk % kCH) * 64 + (lane >> 4) * 16);
        }
    }
    // A fragment reads (SWZ): lane l reads row 16mt + l%16; logical chunk
    // 4s + l/16 of step s sits at stored chunk (4s) ^ v with v = (l/16) ^
    // ((l%16) >> 1 & 7), i.e. at lane offset a_off[0] (s = 0) or a_off[1]
    // (s = 1; fp8: the upper 64 bytes of its one step).
    [[maybe_unused]] uint32_t a_off[2];
    if constexpr (SWZ) {
        const uint32_t v = (uint32_t)((lane >> 4) ^ ((lane & 15) >> 1));
        a_off[0] = (uint32_t)(lane & 15) * 128u + 16u * v;
        a_off[1] = (uint32_t)(lane & 15) * 128u + 16u * (v ^ 4u);
    }
    // mxfp8 scale staging: copy lane e = 64*wave + lane fetches A row
    // 16*(e%16) + e/16 and column 64*wave + 16*(lane%4) + lane/4 of this
    // k-tile's scale block; rows >= M and columns >= N are past the ranges and
    // stage 0 (2^-127, finite), which only ever scales zero data.
    // (mxfp4: rows of the scale arrays are K/32 bytes, and a k-tile's dwords
    // start at byte koff / 16 of a row, koff in K-bytes of two values each.)
    [[maybe_unused]] const int kblk = kMx4 ? p.K / 32 : p.K / 128;
    constexpr bool kX = kMx || kMx4;
    [[maybe_unused]] const auto rXa = make_rsrc(kX ? static_cast<const uint8_t *>(p.sA) + (int64_t)m0 * kblk : nullptr,
                                                kX ? clamp_bytes((int64_t)(p.M - m0) * kblk) : 0);
    [[maybe_unused]] const auto rXb = make_rsrc(kX ? static_cast<const uint8_t *>(p.sB) + (int64_t)n0 * kblk : nullptr,
                                                kX ? clamp_bytes((int64_t)(p.N - n0) * kblk) : 0);
    [[maybe_unused]] const uint32_t xa_voff =
        (uint32_t)(16 * ((wave * 64 + lane) % 16) + (wave * 64 + lane) / 16) * (uint32_t)kblk;
    [[maybe_unused]] const uint32_t xb_voff = (uint32_t)(64 * wave + 16 * (lane & 3) + (lane >> 2)) * (uint32_t)kblk;
    // mxfp4 copy j (0, 1) of this wave: dword e = 128*wave + 64*j + lane of the
    // row region (row 16*((e/2)%16) + e/32, dword e%2) and dword e' = 64*j +
    // lane of this wave's part of the column region (column 64*wave +
    // 16*((e'/2)%4) + (e'/8)%16, dword e'%2).
    [[maybe_unused]] uint32_t xa4_voff[2], xb4_voff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = 128 * wave + 64 * j + lane, e2 = 64 * j + lane;
        xa4_voff[j] = (uint32_t)(16 * ((e / 2) % 16) + e / 32) * (uint32_t)kblk + 4u * (uint32_t)(e % 2);
        xb4_voff[j] = (uint32_t)(64 * wave + 16 * ((e2 / 2) % 4) + (e2 / 8) % 16) * (uint32_t)kblk +
                      4u * (uint32_t)(e2 % 2);
    }
    auto xstage = [&](int t) -> uint32_t * {
        return reinterpret_cast<uint32_t *>(lds + kRing * kBuf + (kX ? (t & (kRing - 1)) * kXStage : 0));
    };
    auto dma_scales = [&](int t, uint32_t koff) {
        if constexpr (kMx) {
            lds_dma<1>(rXa, xstage(t) + wave * 64, xa_voff, koff / 128u);
            lds_dma<1>(rXb, xstage(t) + 256 + wave * 64, xb_voff, koff / 128u);
        } else if constexpr (kMx4) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lds_dma<4>(rXa, xstage(t) + 128 * wave + 64 * j, xa4_voff[j], koff / 16u);
                lds_dma<4>(rXb, xstage(t) + 512 + 128 * wave + 64 * j, xb4_voff[j], koff / 16u);
            }
        }
    };
    [[maybe_unused]] i32x4 xq[4];              // mxfp8: A scales of row tiles 4q..4q+3 (slot q)
    [[maybe_unused]] i32x4 xb_cur, xb_next;    // mxfp8: B scales of this and the next k-tile, one per strip
    [[maybe_unused]] i32x4 xq4[4][2];          // mxfp4: A scale dwords of row tiles 4q..4q+3, both steps
    [[maybe_unused]] i32x4 xb4_next[2];        // mxfp4: the next k-tile's column dwords [strip][step]
    [[maybe_unused]] int eb4[4][2];            // mxfp4: this k-tile's column scale bytes [strip][step]
    [[maybe_unused]] const uint32_t xsh = 8u * (uint32_t)(lane >> 4);   // mxfp4: this lane's byte of a dword
    auto read_xb = [&](int t) {
        if constexpr (kMx) {
            xb_next = *reinterpret_cast<const i32x4 *>(xstage(t) + 256 + 4 * (wave * 16 + (lane & 15)));
        } else if constexpr (kMx4) {
            const uint32_t *b = xstage(t) + 512 + 8 * (wave * 16 + (lane & 15));
            xb4_next[0] = *reinterpret_cast<const i32x4 *>(b);
            xb4_next[1] = *reinterpret_cast<const i32x4 *>(b + 4);
        }
    };

    // B: this wave's kNT strips; strips >= N/16 are past the range (zero).
    const int strip0 = (n0 + wn * 16 * kNT) / 16;
    const auto rB = make_rsrc(p.Bs + (int64_t)strip0 * 16 * Kb, clamp_bytes((int64_t)(p.N / 16 - strip0) * 16 * Kb));
    const uint32_t b_voff = (uint32_t)lane * 16u;

    f32x4 acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (the zeroing stays ahead of the prologue's loads, far from the first MFMA)
    __builtin_amdgcn_sched_barrier(0);

    i32x4 breg[kDB][kNT][kCH];   // [set = tile % kDB][strip][chunk]
    Frag ring[kRA + 1];          // A fragments: slot = fragment index % (kRA + 1)

    auto kofs = [&](int t) { return kbase + (uint32_t)(t < ntiles ? t : ntiles - 1) * KT; };
    auto stage = [&](int t) { return (uint32_t)(t & (kRing - 1)) * kBuf; };
    auto load_b = [&](auto setc, int nt, int ch, uint32_t koff) {
        constexpr int SET = decltype(setc)::value;
        breg[SET][nt][ch] = load16<kAuxNone>(rB, b_voff + (uint32_t)nt * 16u * Kb + (uint32_t)ch * 1024u + koff * 16u);
    };
    auto dma = [&](int j, uint32_t st, uint32_t koff) {
        lds_dma16(rA, lds + st + (j * NW + wave) * 1024, dma_voff[j], koff);
    };
    // The register copy: the same 16 bytes per lane, to the same LDS place.
    [[maybe_unused]] i32x4 cp[SYNC ? kDma : 1];
    auto copy_load = [&](int j, uint32_t koff) { cp[j] = load16<kAuxNone>(rA, dma_voff[j] + koff); };
    auto copy_write = [&](int j, uint32_t st) {
        *reinterpret_cast<i32x4 *>(lds + st + (j * NW + wave) * 1024 + lane * 16) = cp[j];
    };
    auto read_frag = [&](int f, uint32_t st) {   // fragment f of the tile in stage st
        const int s = f / kMT, mt = f % kMT;
        if constexpr (kMx) {
            if (mt % 4 == 0)
                xq[mt / 4] = *reinterpret_cast<const i32x4 *>(lds + kRing * kBuf + (st / kBuf) * kXStage +
                                                              4 * (16 * (lane & 15) + mt));
        } else if constexpr (kMx4) {
            if (s == 0 && mt % 4 == 0) {
                const uint8_t *q = lds + kRing * kBuf + (st / kBuf) * kXStage + 8 * (16 * (lane & 15) + mt);
                xq4[mt / 4][0] = *reinterpret_cast<const i32x4 *>(q);
                xq4[mt / 4][1] = *reinterpret_cast<const i32x4 *>(q + 16);
            }
        }
        if constexpr (SWZ) {
            const uint8_t *row = lds + st + (wm * kMT + mt) * 2048;
            if constexpr (kStepCh == 1)
                ring[f % (kRA + 1)] = *reinterpret_cast<const i32x4 *>(row + a_off[s]);
            else
                ring[f % (kRA + 1)] = cat(*reinterpret_cast<const i32x4 *>(row + a_off[0]),
                                          *reinterpret_cast<const i32x4 *>(row + a_off[1]));
        } else {
            ring[f % (kRA + 1)] = lds_frag<DT>(lds + st + ((wm * kMT + mt) * kCH + s * kStepCh) * 1024 + lane * 16);
        }
    };

    // Prologue: copies of tiles 0..kDmaAhead-1, B of tiles 0..DB-1, all
    // landed; then the first kRA fragments of tile 0.  (The register copy
    // loads its last prologue tile into registers: tile 0 writes it.)
#pragma unroll
    for (int t = 0; t < kDmaAhead; ++t)
#pragma unroll
        for (int j = 0; j < kDma; ++j) {
            if constexpr (SYNC) {
                if (t == kDmaAhead - 1) {
                    copy_load(j, kofs(t));
                    continue;
                }
            }
            dma(j, stage(t), kofs(t));
            if (j == 0)
                dma_scales(t, kofs(t));
        }
    auto prologue_b = [&](auto setc) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
            for (int ch = 0; ch < kCH; ++ch)
                load_b(setc, nt, ch, kofs(decltype(setc)::value));
    };
    prologue_b(std::integral_constant<int, 0>{});
    prologue_b(std::integral_constant<int, 1>{});
    if constexpr (DB > 2)
        prologue_b(std::integral_constant<int, (DB > 2 ? 2 : 0)>{});
    if constexpr (DB > 3)
        prologue_b(std::integral_constant<int, (DB > 3 ? 3 : 0)>{});
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    read_xb(0);
#pragma unroll
    for (int f = 0; f < kRA; ++f)
        read_frag(f, stage(0));
    // mxfp4: fragment f's row scale byte, extracted (VALU) one fragment
    // ahead into slot f % 2 -- the hardware-scaled MFMA needs 2 wait states
    // after a vector-ALU write of its scale register, and the extraction sits
    // three MFMAs before the first one that reads it.
    [[maybe_unused]] int ea4v[2] = {0, 0};
    if constexpr (kMx4)
        ea4v[0] = (int)__builtin_amdgcn_ubfe((uint32_t)xq4[0][0][0], xsh, 8u);

    // One k-tile.  SET = t % kDB holds tile t's B (and receives tile t+kDB's
    // as it is consumed); the wrapped reloads at its start refill set
    // (t-1) % kDB with tile t-1+kDB.
    auto tile = [&](auto setc, int t) {
        constexpr int SET = decltype(setc)::value;
        constexpr int PREV = (SET + kDB - 1) % kDB;
        const uint32_t cur = stage(t), nx1 = stage(t + 1), nx3 = stage(t + kDmaAhead);
        const uint32_t k_prev = kofs(t - 1 + kDB), k_this = kofs(t + kDB), k_dma = kofs(t + kDmaAhead);
        [[maybe_unused]] const uint32_t nx2 = stage(t + kDmaAhead - 1);   // the register copy's write stage
#pragma unroll
        for (int f = 0; f < kFr; ++f) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kMx) {
                if (f == 0)
                    xb_cur = xb_next;
            } else if constexpr (kMx4) {
                if (f == 0) {
#pragma unroll
                    for (int c = 0; c < kNT; ++c)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
                            eb4[c][s2] = (int)__builtin_amdgcn_ubfe((uint32_t)xb4_next[c / 2][(c % 2) * 2 + s2], xsh, 8u);
                    // the first MFMA below reads one of these: 2 wait states
                    // after the extractions, in whatever order they issue
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("s_nop 1");
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (f == kBar) {
                if constexpr (SYNC)   // this wave's LDS writes of tile t+1 (and earlier) are done
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                else                  // this wave's async copy of tile t+1 has landed
                    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kVm) : "memory");
            }
            // The fragment's 4 MFMAs with one slot of other work between each
            // two (one wave per SIMD issues in order: work bunched between
            // two fragments would leave the matrix pipe idle): the LDS read
            // kRA fragments ahead (into tile t+1 past the barrier), then
            // this position's B reloads, then its A copies.
            const int st = f / kMT, mt = f % kMT;
            const Frag &a = ring[f % (kRA + 1)];
            [[maybe_unused]] const int ea4 = ea4v[f & 1];   // this fragment's row scale byte
            auto next_ea4 = [&]() {   // the next fragment's (that of the next k-tile after the last)
                if constexpr (kMx4) {
                    const int g = (f + 1) % kFr, st1 = g / kMT, mt1 = g % kMT;
                    ea4v[(f + 1) & 1] =
                        (int)__builtin_amdgcn_ubfe((uint32_t)xq4[mt1 / 4][(mt1 % 4) / 2][(mt1 % 2) * 2 + st1], xsh, 8u);
                }
            };
            auto mf = [&](int nt) {
                if constexpr (kMx4)
                    mfma_acc_mx4(acc[mt][nt], breg[SET][nt][st], a, eb4[nt][st], ea4);
                else if constexpr (DT == kDtypeBf16)
                    mfma_acc(acc[mt][nt], breg[SET][nt][st], a);
                else if constexpr (kMx)
                    mfma_acc_mx(acc[mt][nt], cat(breg[SET][nt][0], breg[SET][nt][1]), a, xb_cur[nt], xq[mt / 4][mt % 4]);
                else
                    mfma_acc(acc[mt][nt], cat(breg[SET][nt][0], breg[SET][nt][1]), a);
            };
            auto lds_read = [&]() {
                if (f == kBar)   // past the barrier: the next k-tile's column scales
                    read_xb(t + 1);
                if (f + kRA < kFr)
                    read_frag(f + kRA, cur);
                else
                    read_frag(f + kRA - kFr, nx1);
            };
            auto b_loads = [&]() {
#pragma unroll
                for (int i = 0; i < P::kBLoads; ++i) {
                    if (P::bload_pos(i) == f) {
                        const int st2 = i / (kNT * kStepCh), r = i % (kNT * kStepCh);
                        const int ch = st2 * kStepCh + r / kNT, nt = r % kNT;
                        if (P::bload_wraps(i))
                            load_b(std::integral_constant<int, PREV>{}, nt, ch, k_prev);
                        else
                            load_b(setc, nt, ch, k_this);
                    }
                }
            };
            auto a_copies = [&]() {
#pragma unroll
                for (int j = 0; j < kDma; ++j) {
                    if constexpr (SYNC) {
                        if (P::write_pos(j) == f)
                            copy_write(j, nx2);
                        if (P::dma_pos(j) == f)
                            copy_load(j, k_dma);
                    } else if (P::dma_pos(j) == f) {
                        dma(j, nx3, k_dma);
                        if (j == 0)
                            dma_scales(t + kDmaAhead, k_dma);
                    }
                }
            };
            if constexpr (ILV && WM == 2) {
                // 8 MFMAs per fragment: its LDS read after the first, B
                // reloads after the third, A copies after the fifth
                mf(0);
                __builtin_amdgcn_sched_barrier(0);
                next_ea4();
                lds_read();
                __builtin_amdgcn_sched_barrier(0);
                mf(1);
                mf(2);
                __builtin_amdgcn_sched_barrier(0);
                b_loads();
                __builtin_amdgcn_sched_barrier(0);
                mf(3);
                mf(4);
                __builtin_amdgcn_sched_barrier(0);
                a_copies();
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 5; nt < kNT; ++nt)
                    mf(nt);
            } else {
                if constexpr (ILV) {
                    mf(0);
                    __builtin_amdgcn_sched_barrier(0);
                    next_ea4();
                    lds_read();
                    __builtin_amdgcn_sched_barrier(0);
                    mf(1);
                    __builtin_amdgcn_sched_barrier(0);
                    b_loads();
                    __builtin_amdgcn_sched_barrier(0);
                    mf(2);
                    __builtin_amdgcn_sched_barrier(0);
                    a_copies();
                    __builtin_amdgcn_sched_barrier(0);
                } else {
                    lds_read();
                    b_loads();
                    a_copies();
                    __builtin_amdgcn_sched_barrier(0);
                    mf(0);
                    __builtin_amdgcn_sched_barrier(0);
                    next_ea4();
                    __builtin_amdgcn_sched_barrier(0);
                    mf(1);
                    mf(2);
                }
                mf(3);
#pragma unroll
                for (int nt = 4; nt < kNT; ++nt)
                    mf(nt);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Main loop unrolled by DB (the B set of every k-tile is a compile-time
    // index); the remaining ntiles % DB k-tiles follow.
    int t = 0;
    for (; t + DB <= ntiles; t += DB) {
        tile(std::integral_constant<int, 0>{}, t);
        tile(std::integral_constant<int, 1>{}, t + 1);
        if constexpr (DB > 2)
            tile(std::integral_constant<int, (DB > 2 ? 2 : 0)>{}, t + 2);
        if constexpr (DB > 3)
            tile(std::integral_constant<int, (DB > 3 ? 3 : 0)>{}, t + 3);
    }
    if (t < ntiles)
        tile(std::integral_constant<int, 0>{}, t++);
    if constexpr (DB > 2)
        if (t < ntiles)
            tile(std::integral_constant<int, 1>{}, t++);
    if constexpr (DB > 3)
        if (t < ntiles)
            tile(std::integral_constant<int, (DB > 3 ? 2 : 0)>{}, t++);
    // Drain: outstanding copies write LDS; the last MFMAs must finish before
    // their accumulators are read (the compiler does not count these
    // instructions as MFMAs, so it inserts no wait states for them).
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    float scale = 1.0f;
    if constexpr (SCALE == kScaleTensor)
        scale = static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0];
    if constexpr (OUT == kOutBf16) {
        // bf16 C through LDS, so that every store writes whole 128-byte
        // lines: the wave's block (256 x 64, or 128 x 128 as two 128 x 64
        // halves) is one line per row of each 64-column half.  Each wave
        // stages its block in its own 32 KiB of the (now idle) A ring, half
        // h row r at byte 128 (h kRowsW + r) with 16-byte chunk c stored at chunk
        // c ^ ((r >> 1) & 7), the swizzle of the A tile: the 8-byte writes
        // (lane l: row l%16 of a row tile, columns 4(l/16)..+3 of a strip)
        // and the 16-byte reads (8 lanes per row) are both conflict-free.
        // All waves must be done with the ring first (their last LDS reads
        // and copies): the wait above drained this wave's copies, the
        // barrier covers the others'.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        constexpr int kRowsW = TM / WM;                        // rows of the wave's block
        uint8_t *cst = lds + wave * (TM * 128);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int r = mt * 16 + (lane & 15);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                f32x4 v = acc[mt][nt];
                if constexpr (SCALE == kScaleTensor)
                    v = v * scale;
                u32x2 packed;
                packed.x = pack_bf16x2(v.x, v.y);
                packed.y = pack_bf16x2(v.z, v.w);
                const int c = 2 * (nt % 4) + (lane >> 5);        // 16-byte chunk of the half row
                *reinterpret_cast<u32x2 *>(cst + (nt / 4) * (kRowsW * 128) + r * 128 + 16 * (c ^ ((r >> 1) & 7)) +
                                           8 * ((lane >> 4) & 1)) = packed;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // own rows only: no barrier needed
#pragma unroll
        for (int h = 0; h < kNT / 4; ++h) {
            const int ncol = n0 + wn * 16 * kNT + 64 * h + 8 * (lane & 7);
            const bool col_ok = ncol < p.N;                   // N % 16 == 0: 8 columns in or out together
#pragma unroll
            for (int q = 0; q < kRowsW / 8; ++q) {
                const int r = 8 * q + (lane >> 3);
                const i32x4 d = *reinterpret_cast<const i32x4 *>(cst + h * (kRowsW * 128) + r * 128 +
                                                                 16 * ((lane & 7) ^ ((r >> 1) & 7)));
                const int m = m0 + wm * kRowsW + r;
                if (col_ok && m < p.M)
                    *reinterpret_cast<i32x4 *>(static_cast<uint8_t *>(p.C) + ((int64_t)m * p.N + ncol) * 2) = d;
            }
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int m = m0 + wm * (TM / WM) + mt * 16 + (lane & 15);
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const int n = n0 + wn * 16 * kNT + nt * 16 + (lane >> 4) * 4;
                f32x4 v = acc[mt][nt];
                if constexpr (SCALE == kScaleTensor)
                    v = v * scale;
                store_tile<OUT>(p, split, m, n, v);
            }
        }
    }
}

template <int DT, int SCALE, int OUT, int DB, int SWZ, int RA, int ILV, int SYNC, int WM, int TM>
void launch_w4(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    gemm_w4_kernel<DT, SCALE, OUT, DB, SWZ, RA, ILV, SYNC, WM, TM><<<grid, 256, 0, s>>>(a);
}

// Table entries: waves (WM x 4/WM), preload pair = (ILV, RA), layout, copy path.
#define DGP_W4T(DT, SC, OUT, DB, SWZ, RA, ILV, SYNC, WM, TM)                                  \
    {kTiled, DT, SC, OUT, TM, 256, 128, 4, WM, 4 / WM, ILV, RA, DB, kSchedW4,                   \
     &launch_w4<DT, SC, OUT, DB, SWZ, RA, ILV, SYNC, WM, TM>, SWZ ? kLaySwizzled : kLayBlocks,  \
     SYNC ? kCopyRegs : kCopyAsync}
#define DGP_W4X(DT, SC, OUT, DB, SWZ, RA, ILV, SYNC, WM) DGP_W4T(DT, SC, OUT, DB, SWZ, RA, ILV, SYNC, WM, 256)
#define DGP_W4(DT, SC, OUT, DB, SWZ, RA, ILV, SYNC) DGP_W4X(DT, SC, OUT, DB, SWZ, RA, ILV, SYNC, 1)
#define DGP_W4_BOTH_OUT(DT, SC, DB, SWZ, RA, ILV, SYNC)                                       \
    DGP_W4(DT, SC, kOutBf16, DB, SWZ, RA, ILV, SYNC), DGP_W4(DT, SC, kOutPartial, DB, SWZ, RA, ILV, SYNC)

static const KernelSpec kW4Kernels[] = {
    // one wave per SIMD, 256 x 256 (B k-tiles in flight, A layout, LDS
    // read-ahead, interleaved issue, register copy); the tuned kernel
    // first, then the ablations the design was measured against: A in
    // operand blocks, LDS read-ahead 3 and 1, the fragment's work bunched
    // ahead of its MFMAs, A copied through registers
    DGP_W4_BOTH_OUT(kDtypeBf16, kScaleNone, 3, 1, w4::kRA, 1, 0),
    DGP_W4_BOTH_OUT(kDtypeBf16, kScaleNone, 3, 0, w4::kRA, 1, 0),
    DGP_W4(kDtypeBf16, kScaleNone, kOutBf16, 3, 1, 3, 1, 0),
    DGP_W4(kDtypeBf16, kScaleNone, kOutBf16, 3, 1, 1, 1, 0),
    DGP_W4(kDtypeBf16, kScaleNone, kOutBf16, 3, 1, w4::kRA, 0, 0),
    DGP_W4(kDtypeBf16, kScaleNone, kOutBf16, 3, 1, w4::kRA, 1, 1),
    DGP_W4_BOTH_OUT(kDtypeFp8, kScaleTensor, 3, 1, w4::kRA, 1, 0),
    DGP_W4_BOTH_OUT(kDtypeFp8, kScaleTensor, 3, 0, w4::kRA, 1, 0),
    DGP_W4(kDtypeFp8, kScaleTensor, kOutBf16, 3, 1, 3, 1, 0),
    DGP_W4(kDtypeFp8, kScaleTensor, kOutBf16, 3, 1, 1, 1, 0),
    DGP_W4(kDtypeFp8, kScaleTensor, kOutBf16, 3, 1, w4::kRA, 0, 0),
    DGP_W4(kDtypeFp8, kScaleTensor, kOutBf16, 3, 1, w4::kRA, 1, 1),
    // mxfp8 and mxfp4: the hardware-scaled MFMA with the k-tile's E8M0
    // bytes staged beside the A tile
    DGP_W4_BOTH_OUT(kDtypeFp8, kScaleMx, 3, 1, w4::kRA, 1, 0),
    DGP_W4_BOTH_OUT(kDtypeFp4, kScaleMx32, 3, 1, w4::kRA, 1, 0),
    // 2 x 2 waves (each 128 x 128: half the A fragment reads per wave, twice
    // the B strips), B two k-tiles deep
    DGP_W4X(kDtypeBf16, kScaleNone, kOutBf16, 2, 1, 7, 1, 0, 2),
    DGP_W4X(kDtypeBf16, kScaleNone, kOutPartial, 2, 1, 7, 1, 0, 2),
    DGP_W4X(kDtypeBf16, kScaleNone, kOutBf16, 3, 1, 7, 1, 0, 2),
    DGP_W4X(kDtypeBf16, kScaleNone, kOutBf16, 2, 1, 3, 1, 0, 2),
    DGP_W4X(kDtypeFp8, kScaleTensor, kOutBf16, 2, 1, 7, 1, 0, 2),
    DGP_W4X(kDtypeFp8, kScaleTensor, kOutPartial, 2, 1, 7, 1, 0, 2),
    DGP_W4X(kDtypeFp8, kScaleTensor, kOutBf16, 2, 1, 3, 1, 0, 2),
    // 128 x 256 (up to two workgroups per CU, two waves per SIMD: 128 AGPR
    // accumulators per lane, B two k-tiles deep); the tuned read-ahead first
    DGP_W4T(kDtypeBf16, kScaleNone, kOutBf16, 2, 1, 7, 1, 0, 1, 128),
    DGP_W4T(kDtypeBf16, kScaleNone, kOutPartial, 2, 1, 7, 1, 0, 1, 128),
    DGP_W4T(kDtypeBf16, kScaleNone, kOutBf16, 2, 1, 3, 1, 0, 1, 128),
    DGP_W4T(kDtypeFp8, kScaleTensor, kOutBf16, 2, 1, 1, 1, 0, 1, 128),
    DGP_W4T(kDtypeFp8, kScaleTensor, kOutPartial, 2, 1, 1, 1, 0, 1, 128),
    DGP_W4T(kDtypeFp8, kScaleTensor, kOutBf16, 2, 1, 3, 1, 0, 1, 128),
};

const KernelSpec *w4_kernels(int *count)
{
    *count = (int)(sizeof(kW4Kernels) / sizeof(kW4Kernels[0]));
    return kW4Kernels;
}

}  // namespace dgp
