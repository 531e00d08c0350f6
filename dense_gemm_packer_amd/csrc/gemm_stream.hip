// Decode-sized-M GEMM kernels for C = A * B^T with B preshuffled
// (include/dgp.h) and their table entries.  Operand layout and epilogue:
// gemm_common.h.
//
// gemm_stream_kernel -- decode-sized M (aiter PR #5148, "Summary": split-K
//    preshuffle GEMM for small M).  A workgroup owns 16 rows of C and 2 or 4
//    16-column strips (a 16x32 or 16x64 tile); the A rows of its K range sit
//    in LDS and each wave streams its strips of B through a deep ring of
//    in-flight 16-byte loads.  It also carries the FP8 blockscale mode for any
//    M and the microscaling modes (mxfp8, mxfp4), whose E8M0 scales are staged
//    in LDS per panel.
// gemm_ksplit_kernel -- decode-sized M: a workgroup owns half a strip or 1,
//    2 or 4 strips, its K range split over 8 waves, partials added in LDS.

#include <atomic>

#include "gemm_common.h"

namespace dgp {

// =============================================================== stream

// Largest K range (bytes) of the 16 A rows held in LDS at once.  mxfp4
// also stages the panel's E8M0 scales in LDS, so its panel is smaller.
constexpr int kStreamPanelMax = 8192;
constexpr int kStreamPanelMax4 = 4096;
constexpr int stream_panel_max(int dt) { return dt == kDtypeFp4 ? kStreamPanelMax4 : kStreamPanelMax; }
// mxfp4 scale staging: a panel of S MFMA steps keeps, per A row and per
// column of the workgroup, its S scale dwords (one dword = the four 32-element
// blocks of one 64-byte step) plus one dword of padding, so the 16 rows a
// step reads fall in different LDS banks.
// Each region (A rows, then columns) is rounded up to whole 64-dword copies.
constexpr int stream_mx32_region_dwords(int rows, int nsteps) { return (rows * (nsteps + 1) + 63) / 64 * 64; }
constexpr size_t stream_mx32_scale_bytes(int cols, int panel)
{
    return (size_t)4 * (stream_mx32_region_dwords(16, panel / 64) + stream_mx32_region_dwords(cols, panel / 64));
}

template <int DT, int NW, int SPW, int DEPTH, int SCALE, int OUT>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
gemm_stream_kernel(const GemmArgs p, int panel)
{
    using Frag = typename Op<DT>::Frag;
    constexpr int kStepCh = Op<DT>::kBlocks;
    constexpr int kStepBytes = 64 * kStepCh;
    constexpr int kScaleCols = kStreamPanelMax / 128;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds_a[];   // 16 * panel bytes
    __shared__ float lds_sa[SCALE == kScaleBlock ? 16 : 1][kScaleCols];
    __shared__ float lds_sb[SCALE == kScaleBlock ? NW * SPW : 1][kScaleCols];
    // mxfp8: E8M0 bytes of the panel, per A row and per column of the workgroup.
    __shared__ uint8_t lds_xa[SCALE == kScaleMx ? 16 : 1][kScaleCols];
    __shared__ uint8_t lds_xb[SCALE == kScaleMx ? NW * SPW * 16 : 1][kScaleCols];
    // mxfp4: scale dwords after the A panel, a region of the 16 A rows m0..
    // then one of the workgroup's columns (row stride nsteps + 1 dwords).
    constexpr int kCols = NW * SPW * 16;
    uint32_t *lds_x4 = reinterpret_cast<uint32_t *>(lds_a + 16 * panel);
    if constexpr (kLdsPoison) {   // debug build: all of LDS poisoned before the first copy
        lds_poison_fill(lds_a, 16 * panel + (SCALE == kScaleMx32 ? (int)stream_mx32_scale_bytes(kCols, panel) : 0));
        lds_poison_fill(lds_sa, (int)sizeof(lds_sa));
        lds_poison_fill(lds_sb, (int)sizeof(lds_sb));
        lds_poison_fill(lds_xa, (int)sizeof(lds_xa));
        lds_poison_fill(lds_xb, (int)sizeof(lds_xb));
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const auto tc = tile_of_workgroup<int>((int)blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.remap, p.group_m);
    const int m0 = (int)tc.tm * 16;
    const int strip_wg = (int)tc.tn * (NW * SPW);
    const int strip_w = strip_wg + wave * SPW;
    const int split = (int)tc.s;
    const uint32_t Kb = (uint32_t)p.Kb;
    const uint32_t kbase = (uint32_t)split * (uint32_t)p.Ks;
    const int nsteps = panel / kStepBytes;
    // Scale columns per row: one per 128-K block (blockscale, mxfp8), one per
    // 32-K block (mxfp4).
    const int kblocks_row = SCALE == kScaleMx32 ? p.K / 32 : p.K / 128;

    const auto rA = make_rsrc(p.A + (int64_t)m0 * Kb, clamp_bytes((int64_t)(p.M - m0) * Kb));
    const uint32_t a_voff = (uint32_t)(lane & 15) * Kb + (uint32_t)(lane >> 4) * 16u;
    const auto rB = make_rsrc(p.Bs + (int64_t)strip_w * 16 * Kb,
                              clamp_bytes((int64_t)(p.N / 16 - strip_w) * 16 * Kb));
    // E8M0 scales (mxfp8, mxfp4) of rows m0.. and of the workgroup's columns
    constexpr bool kX4 = SCALE == kScaleMx32 || SCALE == kScaleMx;
    const auto rXa = make_rsrc(kX4 ? static_cast<const uint8_t *>(p.sA) + (int64_t)m0 * kblocks_row : nullptr,
                               kX4 ? clamp_bytes((int64_t)(p.M - m0) * kblocks_row) : 0);
    const auto rXb = make_rsrc(kX4 ? static_cast<const uint8_t *>(p.sB) + (int64_t)strip_wg * 16 * kblocks_row
                                   : nullptr,
                               kX4 ? clamp_bytes((int64_t)(p.N - strip_wg * 16) * kblocks_row) : 0);
    uint32_t b_voff[SPW];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
        b_voff[sp] = (uint32_t)sp * 16u * Kb + (uint32_t)lane * 16u;

    float tscale = 1.0f;
    if constexpr (SCALE == kScaleTensor)
        tscale = static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0];

    f32x4 acc[SPW];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
        acc[sp] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x4 breg[DEPTH][SPW][kStepCh];
    auto load_step = [&](int d, int st, uint32_t pk) {
        const uint32_t soff = (pk + (uint32_t)st * kStepBytes) * 16u;
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
            for (int cc = 0; cc < kStepCh; ++cc)
                breg[d][sp][cc] = load16<kAuxNonTemporal>(rB, b_voff[sp] + cc * 1024 + soff);
    };

    for (int p0 = 0; p0 < p.Ks; p0 += panel) {
        const uint32_t pk = kbase + (uint32_t)p0;   // first K byte of this panel
        if (p0 > 0)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

        // Blockscale: fetch this panel's scales into registers now (written
        // to LDS once the copies below are in flight).  Entry i of the sA
        // tile is (row i / cols, block i % cols); of the sB tile, (strip of
        // the workgroup i / cols, block i % cols).
        constexpr int kSaPer = SCALE == kScaleBlock ? (16 * kScaleCols + NW * 64 - 1) / (NW * 64) : 1;
        constexpr int kSbPer = SCALE == kScaleBlock ? (NW * SPW * kScaleCols + NW * 64 - 1) / (NW * 64) : 1;
        float sa_v[kSaPer], sb_v[kSbPer];
        const int cols = panel / 128, kb0 = (int)(pk / 128u);
        if constexpr (SCALE == kScaleBlock) {
#pragma unroll
            for (int u = 0; u < kSaPer; ++u) {
                const int i = threadIdx.x + u * NW * 64;
                const int r = i / cols, c = i % cols;
                sa_v[u] = (i < 16 * cols && m0 + r < p.M) ? static_cast<const float *>(p.sA)[(int64_t)(m0 + r) * kblocks_row + kb0 + c] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kSbPer; ++u) {
                const int i = threadIdx.x + u * NW * 64;
                const int st = i / cols, c = i % cols;
                const int strip = strip_wg + st;
                sb_v[u] = (i < NW * SPW * cols && strip < p.N / 16)
                              ? static_cast<const float *>(p.sB)[(int64_t)(strip * 16 / 128) * kblocks_row + kb0 + c]
                              : 0.f;
            }
        }

        // mxfp8: this panel's E8M0 bytes into registers, one staged row per
        // wave at a time and one K block per lane: rows 0..15 are A rows m0..,
        // rows 16.. the workgroup's columns.  Bytes past M or N read as 0 (a
        // finite 2^-127 that only ever scales zero data).
        constexpr int kXRows = 16 + NW * SPW * 16;
        constexpr int kXPer = SCALE == kScaleMx ? (kXRows + NW - 1) / NW : 1;
        uint32_t x_v[kXPer];
        if constexpr (SCALE == kScaleMx) {
            const uint32_t xoff = pk / 128u + (uint32_t)lane;
#pragma unroll
            for (int u = 0; u < kXPer; ++u) {
                const int r = wave + u * NW;
                x_v[u] = 0u;
                if (r < 16)
                    x_v[u] = __builtin_amdgcn_raw_buffer_load_b8(rXa, (uint32_t)r * kblocks_row + xoff, 0, 0);
                else if (r < kXRows)
                    x_v[u] = __builtin_amdgcn_raw_buffer_load_b8(rXb, (uint32_t)(r - 16) * kblocks_row + xoff, 0, 0);
            }
        }

        // mxfp4: this panel's scale dwords -> LDS with the async dword copy
        // (lane l of a copy lands at its destination + 4l).  Slot e of a
        // region is (row e / (nsteps+1), step e % (nsteps+1)); the padding
        // slot repeats the row's last step.  The dword at E8M0 byte
        // kb0 + 4*step of a row holds the scales of that step's four
        // 32-element blocks.  Rows >= M and columns >= N read as 0 (2^-127,
        // finite), which only ever multiplies zero data.
        if constexpr (SCALE == kScaleMx32) {
            const uint32_t kb0 = pk / 16u;
            const int stride = nsteps + 1;
            auto stage = [&](const auto &rs, uint32_t *dst, int rows) {
                for (int j = wave; j * 64 < rows * stride; j += NW) {
                    const int e = j * 64 + lane;
                    const int r = e / stride < rows ? e / stride : rows - 1;
                    const int st = e % stride < nsteps ? e % stride : nsteps - 1;
                    lds_dma<4>(rs, dst + j * 64, (uint32_t)r * (uint32_t)kblocks_row + kb0 + 4u * (uint32_t)st, 0u);
                }
            };
            stage(rXa, lds_x4, 16);
            stage(rXb, lds_x4 + stream_mx32_region_dwords(16, nsteps), kCols);
        }

        // A rows m0..m0+15 of this panel -> LDS, one 1 KiB operand block per
        // 64-byte K chunk (blocks dealt round-robin to the waves).
        for (int c = wave; c < panel / 64; c += NW)
            lds_dma16(rA, lds_a + c * 1024, a_voff, pk + (uint32_t)c * 64u);
        // Fill the ring of in-flight B loads (clamped to the last step).
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            load_step(d, d < nsteps ? d : nsteps - 1, pk);

        if constexpr (SCALE == kScaleBlock) {
#pragma unroll
            for (int u = 0; u < kSaPer; ++u) {
                const int i = threadIdx.x + u * NW * 64;
                if (i < 16 * cols)
                    lds_sa[i / cols][i % cols] = sa_v[u];
            }
#pragma unroll
            for (int u = 0; u < kSbPer; ++u) {
                const int i = threadIdx.x + u * NW * 64;
                if (i < NW * SPW * cols)
                    lds_sb[i / cols][i % cols] = sb_v[u];
            }
        }
        if constexpr (SCALE == kScaleMx) {
#pragma unroll
            for (int u = 0; u < kXPer; ++u) {
                const int r = wave + u * NW;
                if (lane < cols) {
                    if (r < 16)
                        lds_xa[r][lane] = (uint8_t)x_v[u];
                    else if (r < kXRows)
                        lds_xb[r - 16][lane] = (uint8_t)x_v[u];
                }
            }
        }
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(DEPTH * SPW * kStepCh) : "memory");

        // One MFMA step: consume ring slot d (step st).
        auto consume = [&](int d, int st) {
                {
                    const Frag a = lds_frag<DT>(lds_a + (st * kStepCh) * 1024 + lane * 16);
#pragma unroll
                    for (int sp = 0; sp < SPW; ++sp) {
                        Frag b;
                        if constexpr (kStepCh == 1)
                            b = breg[d][sp][0];
                        else
                            b = cat(breg[d][sp][0], breg[d][sp][1]);
                        if constexpr (SCALE == kScaleBlock) {
                            // One MFMA is exactly one 128-wide K block: its fp32
                            // partial scaled and added in one fused multiply-add
                            // (blockscale, aiter PR #5148).
                            const f32x4 part = mfma_op(b, a, f32x4{0.f, 0.f, 0.f, 0.f});
                            const float s = __fmul_rn(lds_sa[lane & 15][st], lds_sb[wave * SPW + sp][st]);
                            acc[sp].x = __builtin_fmaf(part.x, s, acc[sp].x);
                            acc[sp].y = __builtin_fmaf(part.y, s, acc[sp].y);
                            acc[sp].z = __builtin_fmaf(part.z, s, acc[sp].z);
                            acc[sp].w = __builtin_fmaf(part.w, s, acc[sp].w);
                        } else if constexpr (SCALE == kScaleMx) {
                            acc[sp] = mfma_mx(b, a, acc[sp], lds_xb[(wave * SPW + sp) * 16 + (lane & 15)][st],
                                              lds_xa[lane & 15][st]);
                        } else if constexpr (SCALE == kScaleMx32) {
                            // lane 16g+i: block g of the step, A row i / column i
                            const uint8_t *xa4 = reinterpret_cast<const uint8_t *>(lds_x4);
                            const uint8_t *xb4 = reinterpret_cast<const uint8_t *>(
                                lds_x4 + stream_mx32_region_dwords(16, nsteps));
                            const int ea = xa4[((lane & 15) * (nsteps + 1) + st) * 4 + (lane >> 4)];
                            const int eb = xb4[(((wave * SPW + sp) * 16 + (lane & 15)) * (nsteps + 1) + st) * 4 +
                                               (lane >> 4)];
                            acc[sp] = mfma_mx4(b, a, acc[sp], eb, ea);
                        } else {
                            acc[sp] = mfma_op(b, a, acc[sp]);
                        }
                    }
                }
        };
        // Main part: every load the ring issues is a real step.  Tail (the
        // last 2*DEPTH-1 steps or fewer): loads only for steps that exist,
        // so no wave ends waiting on repeats of its last step.
        int st0 = 0;
        for (; st0 + 2 * DEPTH <= nsteps; st0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                consume(d, st0 + d);
                load_step(d, st0 + d + DEPTH, pk);
            }
        }
        for (; st0 < nsteps; st0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int st = st0 + d;
                if (st < nsteps)
                    consume(d, st);
                if (st + DEPTH < nsteps)
                    load_step(d, st + DEPTH, pk);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int m = m0 + (lane & 15);
        const int n = (strip_w + sp) * 16 + (lane >> 4) * 4;
        f32x4 v = acc[sp];
        if constexpr (SCALE == kScaleTensor)
            v = v * tscale;
        store_tile<OUT>(p, split, m, n, v);
    }
}

// gemm_ksplit_kernel -- decode-sized M.  A workgroup owns a 16-row tile of C
// TN columns wide -- one strip of Bs (TN = 16), SPW = TN/16 strips (TN = 32,
// 64), or half a strip (TN = 8) -- and divides its K range into NW
// contiguous slices of whole MFMA steps, one per wave, so a weight spreads
// over many waves without a second pass: N = 2048 gives 128 workgroups of NW
// waves with whole strips where the 64-column streaming tile gives 32.  Each
// wave streams its slice of A and of its strips of B straight into
// registers through a ring of DEPTH MFMA steps of in-flight loads (A rows
// >= M and strips past N load as zero); each A fragment serves all SPW
// strips, so wider tiles read A fewer times.  Then the NW partial tiles are
// added in LDS in wave order -- a fixed order, so results are reproducible
// and the same for every TN -- and wave sp runs the epilogue of strip sp.
// Blockscale: one fp8 MFMA step is exactly one 128-wide K block, scaled as
// in gemm_stream_kernel with the scales read straight from global memory
// (the SPW strips of a tile lie in one 128-column block).
// TN = 8 (half strips): two workgroups share a strip, each owning 8 of its
// 16 columns, so a narrow weight fills twice as many CUs with no second
// pass.  Lanes whose B row (lane % 16) belongs to the other half load at an
// offset past the strip's buffer range, which returns zeros without a
// memory access: each workgroup reads only its half of every 1 KiB block
// (8 rows x 4 contiguous 128-byte pieces), and its MFMAs compute zeros for
// the other half's columns, which it does not store.
template <int DT, int NW, int DEPTH, int SCALE, int OUT, int TN>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
gemm_ksplit_kernel(const GemmArgs p)
{
    static_assert(TN == 8 || TN == 16 || TN == 32 || TN == 64, "half a strip, or 1, 2 or 4 strips");
    constexpr bool kHalf = TN == 8;
    constexpr int SPW = kHalf ? 1 : TN / 16;
    static_assert(SPW <= NW, "one wave per strip in the epilogue");
    using Frag = typename Op<DT>::Frag;
    constexpr int kStepCh = Op<DT>::kBlocks;
    constexpr int kStepBytes = 64 * kStepCh;
    __shared__ f32x4 red[NW][SPW][64];
    if constexpr (kLdsPoison) {   // debug build: the partial-sum array poisoned before its writes
        lds_poison_fill(red, (int)sizeof(red));
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const auto tc = tile_of_workgroup<int>((int)blockIdx.x, p.tiles_m, p.tiles_n, p.splits, p.remap, p.group_m);
    const int m0 = (int)tc.tm * 16;
    const int strip0 = kHalf ? (int)tc.tn >> 1 : (int)tc.tn * SPW;
    const int half = kHalf ? (int)tc.tn & 1 : 0;
    const int split = (int)tc.s;
    const uint32_t Kb = (uint32_t)p.Kb;
    const uint32_t kbase = (uint32_t)split * (uint32_t)p.Ks;
    const int nsteps = p.Ks / kStepBytes;
    // This wave's steps [s0, s1): the first nsteps % NW waves take one more.
    const int per = nsteps / NW, extra = nsteps % NW;
    const int s0 = wave * per + (wave < extra ? wave : extra);
    const int s1 = s0 + per + (wave < extra ? 1 : 0);
    // Scale columns per row: one per 128-K block (blockscale, mxfp8), one per
    // 32-K block (mxfp4).
    const int kblocks_row = SCALE == kScaleMx32 ? p.K / 32 : p.K / 128;

    const auto rA = make_rsrc(p.A + (int64_t)m0 * Kb, clamp_bytes((int64_t)(p.M - m0) * Kb));
    const uint32_t a_voff = (uint32_t)(lane & 15) * Kb + (uint32_t)(lane >> 4) * 16u;
    // Half strips: the resource covers exactly the strip (16 rows, at most
    // 128 MiB), and the other half's lanes start at 2^31, so every offset
    // they form stays past the range and below 2^32.
    const auto rB = kHalf
        ? make_rsrc(p.Bs + (int64_t)strip0 * 16 * Kb, strip0 < p.N / 16 ? 16u * Kb : 0u)
        : make_rsrc(p.Bs + (int64_t)strip0 * 16 * Kb, clamp_bytes((int64_t)(p.N / 16 - strip0) * 16 * Kb));
    const bool row_on = !kHalf || ((lane & 15) >> 3) == half;
    uint32_t b_voff[SPW];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
        b_voff[sp] = (uint32_t)sp * 16u * Kb + (uint32_t)lane * 16u + (row_on ? 0u : 0x80000000u);
    const int m = m0 + (lane & 15);
    // Blockscale: a step's two scales (this lane's A row of sA, rows past M
    // reading zero; the tile's row of sB, whose strips lie in one 128-column
    // block): loaded into the step's ring slot with its operands (ordered
    // ring) or read where the step is multiplied (guarded loop).
    static_assert(SCALE != kScaleBlock || 128 % (16 * SPW) == 0, "a tile's strips in one 128-column block");
    constexpr bool kBs = SCALE == kScaleBlock;
    [[maybe_unused]] const auto rSa = make_rsrc(kBs ? static_cast<const float *>(p.sA) + (int64_t)m0 * kblocks_row : nullptr,
                                                kBs ? clamp_bytes((int64_t)(p.M - m0) * kblocks_row * 4) : 0);
    [[maybe_unused]] const auto rSb = make_rsrc(kBs ? static_cast<const float *>(p.sB) + (int64_t)(strip0 * 16 / 128) * kblocks_row
                                                    : nullptr,
                                                kBs ? (uint32_t)kblocks_row * 4u : 0u);
    [[maybe_unused]] const uint32_t sa_off = (uint32_t)(lane & 15) * (uint32_t)kblocks_row * 4u;
    // mxfp8: a step's E8M0 bytes (this lane's A row, its B column in each
    // strip) are loaded with the step's operands into the same ring slot, so
    // they arrive with them and waiting for them never drains the ring.  With
    // 2 or 4 strips one byte load serves all of them (lane 16 s + i: column i
    // of strip s) and a cross-lane read hands each MFMA its strip's byte: one
    // load per step instead of one per strip (3-5 % faster at N = 8192 and
    // 16384).  The
    // resources cover rows m0.. < M and columns strip0*16.. < N: rows and
    // strips past the edge read zero (2^-127), which only scales zero data.
    constexpr bool kMx = SCALE == kScaleMx;
    [[maybe_unused]] const auto rXa8 = make_rsrc(kMx ? static_cast<const uint8_t *>(p.sA) + (int64_t)m0 * kblocks_row
                                                     : nullptr,
                                                 kMx ? clamp_bytes((int64_t)(p.M - m0) * kblocks_row) : 0);
    [[maybe_unused]] const auto rXb8 = make_rsrc(kMx ? static_cast<const uint8_t *>(p.sB) + (int64_t)strip0 * 16 * kblocks_row
                                                     : nullptr,
                                                 kMx ? clamp_bytes((int64_t)(p.N - strip0 * 16) * kblocks_row) : 0);
    [[maybe_unused]] const uint32_t x8_off = (uint32_t)(lane & 15) * (uint32_t)kblocks_row;
    [[maybe_unused]] int xs[DEPTH][1 + SPW];   // [ring slot][A row, then each strip's column]
    static_assert(!kMx || kStepBytes == 128, "mxfp8: one 128-K scale block per MFMA step");

    // mxfp4: the E8M0 bytes of a group of DEPTH = 4 steps are 16 contiguous
    // bytes of each row (step st, lane l: byte 4*st + l/16 of the row's
    // [K/32] scales, from byte kbase/16 on), so one 16-byte load per row and
    // group replaces a byte load per step; the next group's words are loaded
    // one group ahead (bytes past the wave's slice are read and unused).  The
    // load is dword-aligned (rows are whole dwords), and the buffer unit
    // range-checks each dword of such a load on its own: a group that runs
    // past the end of the scale array reads zero in the dwords beyond it only.
    // Rows past M and columns past N read as zero (2^-127, finite), which
    // only ever scales zero data.
    constexpr bool kXw = SCALE == kScaleMx32;
    static_assert(!kXw || (DEPTH == 4 && kStepBytes == 64), "mxfp4 scale words: 4 bytes per step, one 16-byte load per 4 steps");
    [[maybe_unused]] const auto rXa = make_rsrc(kXw ? static_cast<const uint8_t *>(p.sA) + (int64_t)m0 * kblocks_row
                                                    : nullptr,
                                                kXw ? clamp_bytes((int64_t)(p.M - m0) * kblocks_row) : 0);
    [[maybe_unused]] const auto rXb = make_rsrc(kXw ? static_cast<const uint8_t *>(p.sB) + (int64_t)strip0 * 16 * kblocks_row
                                                    : nullptr,
                                                kXw ? clamp_bytes((int64_t)(p.N - strip0 * 16) * kblocks_row) : 0);
    [[maybe_unused]] i32x4 xw[2][1 + SPW];   // [group parity][A row, then each strip's column]
    [[maybe_unused]] auto load_x = [&](auto setc, int st) {
        if constexpr (kXw) {
            constexpr int X = decltype(setc)::value;
            const uint32_t gb = kbase / 16u + 4u * (uint32_t)st;
            const uint32_t oa = (uint32_t)(lane & 15) * (uint32_t)kblocks_row + gb;
            xw[X][0] = load16<kAuxNone>(rXa, oa);
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp)
                xw[X][1 + sp] = load16<kAuxNone>(rXb, oa + (uint32_t)(sp * 16) * (uint32_t)kblocks_row);
        }
    };

    f32x4 acc[SPW];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
        acc[sp] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Ring schedule, chosen per tile from cold sweeps of both: the 16-column
    // tiles and the fp8 half-strip tiles keep their ring in order with exact
    // waits (ring_run, 1-15 % faster there); the wider tiles, whose ordered
    // ring needs too many registers for two workgroups per CU, the bf16
    // half strips and mxfp4 (scale words per group of 4 steps) run the
    // guarded loop below, which waits for a whole group at a time.
    constexpr bool kRing = !kXw && (TN == 16 || (TN == 8 && DT != kDtypeBf16));
    i32x4 areg[DEPTH][kStepCh], breg[DEPTH][SPW][kStepCh];
    [[maybe_unused]] float sav[DEPTH], sbv[DEPTH];
    // Step st of the split: K bytes kbase + st*kStepBytes; A chunk cc of it is
    // one 16-row x 64-byte operand read, B chunk cc of strip sp one 1 KiB block.
    auto load_step = [&](int d, int st) {
        const uint32_t k = kbase + (uint32_t)st * kStepBytes;
        if constexpr (kMx) {
            const uint32_t kb = k / 128u;   // one E8M0 byte per 128-K step
            xs[d][0] = __builtin_amdgcn_raw_buffer_load_b8(rXa8, x8_off + kb, 0, kAuxNone);
            if constexpr (SPW >= 2) {   // one load for all strips: lane l takes column l % 16 of strip (l / 16) % SPW
                xs[d][1] = __builtin_amdgcn_raw_buffer_load_b8(
                    rXb8, (uint32_t)(16 * ((lane >> 4) % SPW) + (lane & 15)) * (uint32_t)kblocks_row + kb, 0, kAuxNone);
            } else {
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp)
                    xs[d][1 + sp] = __builtin_amdgcn_raw_buffer_load_b8(
                        rXb8, x8_off + (uint32_t)(sp * 16) * (uint32_t)kblocks_row + kb, 0, kAuxNone);
            }
        }
        if constexpr (kBs && kRing) {
            const uint32_t kb = k / 128u;   // one fp32 scale per 128-K step
            sav[d] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rSa, sa_off + 4u * kb, 0, kAuxNone));
            sbv[d] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rSb, 4u * kb, 0, kAuxNone));
        }
#pragma unroll
        for (int cc = 0; cc < kStepCh; ++cc)
            areg[d][cc] = load16<kAuxNone>(rA, a_voff + k + cc * 64u);
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
            for (int cc = 0; cc < kStepCh; ++cc)
                breg[d][sp][cc] = load16<kAuxNonTemporal>(rB, b_voff[sp] + k * 16u + cc * 1024u);
    };
    // The MFMAs of step st in slot d (X: the mxfp4 scale words' parity).
    auto consume = [&](auto setc, int d, [[maybe_unused]] int st) {
        [[maybe_unused]] constexpr int X = decltype(setc)::value;
        Frag a;
        if constexpr (kStepCh == 1)
            a = areg[d][0];
        else
            a = cat(areg[d][0], areg[d][1]);
        [[maybe_unused]] float sc = 0.f;
        [[maybe_unused]] int ea = 127;
        if constexpr (kBs && kRing) {
            sc = __fmul_rn(sav[d], sbv[d]);
        } else if constexpr (kBs) {   // the guarded loop reads the two scales here
            const uint32_t kb = (kbase + (uint32_t)st * kStepBytes) / 128u;
            sc = __fmul_rn(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rSa, sa_off + 4u * kb, 0, kAuxNone)),
                           __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rSb, 4u * kb, 0, kAuxNone)));
        } else if constexpr (kMx) {
            ea = xs[d][0];
        } else if constexpr (kXw) {
            // this lane's 16 bytes are one 32-element block, byte l/16 of the step's word
            ea = (int)(((uint32_t)xw[X][0][d] >> (8u * (uint32_t)(lane >> 4))) & 0xFFu);
        }
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            Frag b;
            if constexpr (kStepCh == 1)
                b = breg[d][sp][0];
            else
                b = cat(breg[d][sp][0], breg[d][sp][1]);
            if constexpr (kBs) {
                const f32x4 part = mfma_op(b, a, f32x4{0.f, 0.f, 0.f, 0.f});
                acc[sp].x = __builtin_fmaf(part.x, sc, acc[sp].x);
                acc[sp].y = __builtin_fmaf(part.y, sc, acc[sp].y);
                acc[sp].z = __builtin_fmaf(part.z, sc, acc[sp].z);
                acc[sp].w = __builtin_fmaf(part.w, sc, acc[sp].w);
            } else if constexpr (kMx) {
                // (2 or 4 strips: strip sp's column bytes sit in lanes 16 sp + i)
                acc[sp] = mfma_mx(b, a, acc[sp], SPW >= 2 ? __shfl(xs[d][1], 16 * sp + (lane & 15)) : xs[d][1 + sp], ea);
            } else if constexpr (kXw) {
                const int eb = (int)(((uint32_t)xw[X][1 + sp][d] >> (8u * (uint32_t)(lane >> 4))) & 0xFFu);
                acc[sp] = mfma_mx4(b, a, acc[sp], eb, ea);
            } else {
                acc[sp] = mfma_op(b, a, acc[sp]);
            }
        }
    };
    if constexpr (kRing) {
        // The ring loads only steps of this wave's slice (an empty slice, when
        // nsteps < NW, loads nothing).
        ring_run<DEPTH>(
            s1 - s0, [&](int d, int i) { load_step(d, s0 + i); },
            [&](int d, int i) { consume(std::integral_constant<int, 0>{}, d, s0 + i); });
    } else {
        // Two ring groups per iteration, so the parity of the mxfp4 scale
        // words (loaded a group ahead) is a compile-time index; the ring
        // loads only steps of the wave's slice.
        if (s0 < s1)
            load_x(std::integral_constant<int, 0>{}, s0);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if (s0 + d < s1)
                load_step(d, s0 + d);
        auto group = [&](auto setc, int st0) {
            constexpr int X = decltype(setc)::value;
            if (st0 + DEPTH < s1)
                load_x(std::integral_constant<int, 1 - X>{}, st0 + DEPTH);
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int st = st0 + d;
                if (st < s1) {
                    consume(setc, d, st);
                    if (st + DEPTH < s1)
                        load_step(d, st + DEPTH);
                }
            }
        };
        for (int st0 = s0; st0 < s1; st0 += 2 * DEPTH) {
            group(std::integral_constant<int, 0>{}, st0);
            if (st0 + DEPTH < s1)
                group(std::integral_constant<int, 1>{}, st0 + DEPTH);
        }
    }
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
        red[wave][sp][lane] = acc[sp];
    __syncthreads();
    if (wave < SPW) {
        const int sp = wave;
        f32x4 v = red[0][sp][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const f32x4 u = red[w][sp][lane];
            v.x = __fadd_rn(v.x, u.x);
            v.y = __fadd_rn(v.y, u.y);
            v.z = __fadd_rn(v.z, u.z);
            v.w = __fadd_rn(v.w, u.w);
        }
        if constexpr (SCALE == kScaleTensor)
            v = v * (static_cast<const float *>(p.sA)[0] * static_cast<const float *>(p.sB)[0]);
        // lane l holds columns 4*(l/16) .. +3 of the strip
        if (!kHalf || ((lane >> 4) >> 1) == half)
            store_tile<OUT>(p, split, m, (strip0 + sp) * 16 + (lane >> 4) * 4, v);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int DT, int NW, int SPW, int DEPTH, int SCALE, int OUT>
void launch_stream(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    constexpr int kStepBytes = 64 * Op<DT>::kBlocks;
    constexpr int kMax = stream_panel_max(DT);
    // Panel: the whole K range of a split if its 16 rows fit, else the
    // largest step multiple <= kMax that divides it (K ranges are whole
    // multiples of 128 bytes, so one exists).
    int panel = a.Ks;
    if (panel > kMax) {
        panel = kMax - kMax % kStepBytes;
        while (panel > kStepBytes && a.Ks % panel != 0)
            panel -= kStepBytes;
    }
    auto lds_bytes = [](int pnl) {
        return (size_t)16 * pnl + (SCALE == kScaleMx32 ? stream_mx32_scale_bytes(NW * SPW * 16, pnl) : 0);
    };
    const size_t lds = lds_bytes(panel);
    // The LDS allowance is a per-device attribute of the kernel: set it once
    // on each device this launcher runs on (a failure surfaces at the launch).
    // Host threads may launch concurrently: the flags are atomics, and two
    // threads that both see a flag clear both set the same value.
    static std::atomic<bool> attr_set[64];
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
        (void)hipFuncSetAttribute((const void *)gemm_stream_kernel<DT, NW, SPW, DEPTH, SCALE, OUT>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes(kMax));
        if (dev >= 0 && dev < 64)
            attr_set[dev].store(true, std::memory_order_release);
    }
    gemm_stream_kernel<DT, NW, SPW, DEPTH, SCALE, OUT><<<grid, NW * 64, lds, s>>>(a, panel);
}

template <int DT, int NW, int DEPTH, int SCALE, int OUT, int TN>
void launch_ksplit(const GemmArgs &a, dim3 grid, hipStream_t s)
{
    gemm_ksplit_kernel<DT, NW, DEPTH, SCALE, OUT, TN><<<grid, NW * 64, 0, s>>>(a);
}

#define DGP_KSPLIT(DT, NW, DEPTH, SC, OUT, TN)                                                \
    {kStream, DT, SC, OUT, 16, TN, 0, NW, (TN >= 16 ? TN / 16 : 1), DEPTH, 0, 0, DEPTH, 0,          \
     &launch_ksplit<DT, NW, DEPTH, SC, OUT, TN>}
#define DGP_KSPLIT_BOTH_OUT(DT, NW, DEPTH, SC, TN)                                            \
    DGP_KSPLIT(DT, NW, DEPTH, SC, kOutBf16, TN), DGP_KSPLIT(DT, NW, DEPTH, SC, kOutPartial, TN)
#define DGP_STREAM(DT, NW, SPW, DEPTH, SC, OUT)                                               \
    {kStream, DT, SC, OUT, 16, 16 * NW * SPW, stream_panel_max(DT), NW, SPW, DEPTH, 0, 0, DEPTH, 0, \
     &launch_stream<DT, NW, SPW, DEPTH, SC, OUT>}

#define DGP_STREAM_BOTH_OUT(DT, NW, SPW, DEPTH, SC)                                           \
    DGP_STREAM(DT, NW, SPW, DEPTH, SC, kOutBf16), DGP_STREAM(DT, NW, SPW, DEPTH, SC, kOutPartial)

static const KernelSpec kStreamKernels[] = {
    // streaming (decode-sized M): waves per workgroup, strips per wave, ring depth
    DGP_STREAM_BOTH_OUT(kDtypeBf16, 4, 1, 16, kScaleNone),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 4, 1, 8, kScaleTensor),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 2, 2, 8, kScaleTensor),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 4, 1, 8, kScaleBlock),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 4, 1, 8, kScaleMx),
    DGP_STREAM_BOTH_OUT(kDtypeFp4, 4, 1, 8, kScaleMx32),
    // 16 x 32 tiles: twice the workgroups where the 64-column grid is short
    DGP_STREAM_BOTH_OUT(kDtypeBf16, 2, 1, 16, kScaleNone),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 2, 1, 8, kScaleTensor),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 2, 1, 8, kScaleBlock),
    DGP_STREAM_BOTH_OUT(kDtypeFp8, 2, 1, 8, kScaleMx),
    DGP_STREAM_BOTH_OUT(kDtypeFp4, 2, 1, 8, kScaleMx32),
    // one strip per workgroup, K split over the waves: waves, ring depth
    DGP_KSPLIT_BOTH_OUT(kDtypeBf16, 8, 4, kScaleNone, 16),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleTensor, 16),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleBlock, 16),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleMx, 16),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 8, 4, kScaleMx32, 16),
    // half a strip per workgroup (16 x 8 tiles)
    DGP_KSPLIT_BOTH_OUT(kDtypeBf16, 8, 4, kScaleNone, 8),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleTensor, 8),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleBlock, 8),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleMx, 8),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 8, 4, kScaleMx32, 8),
    // 2 and 4 strips per workgroup (16 x 32, 16 x 64 tiles; 8 waves, which
    // tells them apart from the streaming tiles of the same size)
    DGP_KSPLIT_BOTH_OUT(kDtypeBf16, 8, 4, kScaleNone, 32),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleTensor, 32),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleBlock, 32),
    // (mxfp8 at 32 columns: a 3-step ring, 126 VGPRs, so two workgroups fit
    // per CU; with 4 steps it needs 151 and one fits)
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 3, kScaleMx, 32),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 8, 4, kScaleMx32, 32),
    DGP_KSPLIT_BOTH_OUT(kDtypeBf16, 8, 4, kScaleNone, 64),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleTensor, 64),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleBlock, 64),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp8, 8, 4, kScaleMx, 64),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 8, 4, kScaleMx32, 64),
    // bf16, four strips, 16 waves (4 per SIMD where the 8-wave tile has 2;
    // the fp8 modes spill or lose with 16)
    DGP_KSPLIT_BOTH_OUT(kDtypeBf16, 16, 4, kScaleNone, 64),
    // mxfp4, 16 waves over half a strip, one or two strips: each wave's slice
    // of one pass fits one 4-step group of its guarded loop
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 16, 4, kScaleMx32, 8),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 16, 4, kScaleMx32, 16),
    DGP_KSPLIT_BOTH_OUT(kDtypeFp4, 16, 4, kScaleMx32, 32),
};

const KernelSpec *stream_kernels(int *count)
{
    *count = (int)(sizeof(kStreamKernels) / sizeof(kStreamKernels[0]));
    return kStreamKernels;
}

}  // namespace dgp
