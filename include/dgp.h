/*
 * dgp.h -- C ABI of the MI355X (gfx950) preshuffled-B GEMM library.
 *
 * The library computes C = A * B^T with B stored "preshuffled": reordered
 * once, offline, into the order in which the matrix cores consume it.  The
 * operation and its variants are the ones the following pages describe:
 *
 *   [P1] FlyDSL PR #1008, "Enable the gmem->LDS async copy for f16/bf16
 *        preshuffle GEMM" -- the bf16 preshuffle GEMM, its A-tile async copy
 *        into LDS, the A-tile granularity rule and the argument checks.
 *   [P2] FlyDSL PR #974 and its follow-up commit "Reject tiles whose A tile is
 *        only partially loaded" / "Restore per-k-step A-fragment LDS reads".
 *   [P3] aiter PR #5148, "FlyDSL split-K preshuffle decode GEMM for small-M
 *        shapes (FP8 + MX)" -- FP8 per-tensor and blockscale modes, the
 *        two-pass split-K (fp32 workspace partials + reduce kernel) and the
 *        direct split_k = 1 epilogue.
 *
 * Conventions for every entry point
 *   - A is [M][K] row-major, B is [N][K] row-major (K contiguous): C = A*B^T,
 *     C is [M][N] row-major bf16.  (m, k from A's shape and n from the weight's
 *     first dimension, as in the blockscale reference reviewed on [P3].)
 *   - Element types: DGP_BF16 (bf16 bit patterns, 2 bytes) or DGP_FP8_E4M3
 *     (OCP e4m3fn codes, 1 byte).  Accumulation is always fp32.
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees, synchronises or keeps a pointer past the
 *     call (one entry point, dgp_gemm_preshuffle_splitk_noalloc, uses a fixed
 *     array of the library's own instead of a caller workspace).  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and runs asynchronously: outputs are ready when the stream is.
 *   - Scales are device pointers to fp32 as well (so a launch never needs a
 *     host synchronisation).
 *   - Every argument is validated on the host before any HIP call.  On a bad
 *     argument the call returns a status != DGP_OK and enqueues nothing.
 *   - Aliasing between an output and any input is not supported.
 *   - No input needs padding past its last element.  The kernels read
 *     through gfx950 buffer resources whose range ends at the input's last
 *     byte; a load at or past that end returns zero and touches no memory.
 *     One kernel relies on a finer form of this rule: the 16-row K-split
 *     decode tiles read mxfp4 (DGP_SCALE_MX32) scale bytes 16 at a time,
 *     and such a 16-byte load near the end of sA or sB may run past it.  The
 *     buffer unit range-checks each dword of an aligned multi-dword buffer
 *     load on its own, so the dwords inside the range carry data and the
 *     dwords past it read as zero.  (The compiler merges adjacent aligned
 *     dword buffer loads into one wider load on the same rule.)
 */
#ifndef DGP_H
#define DGP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dgp_status {
    DGP_OK = 0,
    DGP_ERR_NULL = 1,        /* a required pointer is NULL                       */
    DGP_ERR_SHAPE = 2,       /* a size is negative or breaks a divisibility rule */
    DGP_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                 */
    DGP_ERR_DTYPE = 4,       /* unknown element type                             */
    DGP_ERR_SCALE_MODE = 5,  /* unknown scale mode, or not valid for the dtype   */
    DGP_ERR_SPLITK = 6,      /* split_k < 1 or does not divide the K range      */
    DGP_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required          */
    DGP_ERR_CONFIG = 8,      /* requested tile configuration not available       */
    DGP_ERR_ARCH = 9,        /* current device is not gfx950                     */
    DGP_ERR_HIP = 10         /* a HIP runtime call or kernel launch failed       */
} dgp_status;

/* Element types.  K always counts elements; a row of DGP_FP4_E2M1 (OCP E2M1,
 * two per byte, element 2j in the low nibble of byte j) is K/2 bytes. */
typedef enum dgp_dtype { DGP_BF16 = 0, DGP_FP8_E4M3 = 1, DGP_FP4_E2M1 = 2 } dgp_dtype;

/* DGP_SCALE_NONE: bf16 only; sA, sB unused.  DGP_SCALE_TENSOR: fp8 only; sA,
 * sB each point to one fp32 and C = bf16(acc * (sA*sB)).  DGP_SCALE_BLOCK128:
 * fp8 only; sA is [M][K/128] fp32 (A per row per 128-wide K block), sB is
 * [N/128][K/128] fp32 (B per 128x128 block), both row-major; each 128-K
 * block's fp32 partial sum p is multiplied by s = sA[m][kb]*sB[n/128][kb]
 * (rounded to fp32) and added to the fp32 accumulator in one fused
 * multiply-add, acc = fma(p, s, acc), one rounding per block ([P3] "Summary";
 * scale shapes from the run_torch_blockscale review; the rounding is not
 * stated there).  DGP_SCALE_MX128 (mxfp8): fp8 only; sA is
 * [M][K/128] and sB [N][K/128] bytes, both row-major, each an E8M0 scale
 * 2^(e-127) (255: NaN) for one row of A or one row of B (= one column of C)
 * over one 128-wide K block; the matrix-core instruction applies them to each
 * block's products ([P3] "What's included": mxfp8 with 128-element blocks on
 * the hardware-scaled MFMA).  DGP_SCALE_MX32 (mxfp4): the only mode of
 * DGP_FP4_E2M1, and only for it; as MX128 but one E8M0 byte per 32-element
 * block, sA [M][K/32], sB [N][K/32] ([P3] "What's included": mxfp4, 4-bit
 * packed with 32-element E8M0 blocks).  fp32 scales must be 4-byte aligned. */
typedef enum dgp_scale_mode {
    DGP_SCALE_NONE = 0,
    DGP_SCALE_TENSOR = 1,
    DGP_SCALE_BLOCK128 = 2,
    DGP_SCALE_MX128 = 3,
    DGP_SCALE_MX32 = 4
} dgp_scale_mode;

/* Optional tile configuration.  Pass NULL to use the built-in per-shape table.
 *   tile_m, tile_n : output tile of one workgroup (must name a compiled tile:
 *                    256x256, 128x256, 128x128 for bf16 and per-tensor fp8;
 *                    256x256 and 128x128 for fp8 blockscale, mxfp8 and mxfp4;
 *                    16x64 and 16x32 streaming (4 and 2 waves); K-split
 *                    (8 waves; also 16 for bf16 16x64 and for mxfp4
 *                    16x8, 16x16 and 16x32) over 16x8 -- half a strip, two
 *                    workgroups
 *                    per 16-column strip -- 16x16, 16x32 and 16x64; every
 *                    16-row tile for every mode; one-row VALU tiles 1x16
 *                    and 1x8 for bf16 and per-tensor fp8 -- [P3] file
 *                    table, the "Wave" decode policy -- one workgroup per
 *                    row of C, meant for M = 1)
 *   tile_k         : tiled kernels: K bytes staged per main-loop step (128,
 *                    the k-tile of every compiled tiled kernel); ignored by
 *                    the 16-row kernels
 *   xcd_remap      : 1 = map workgroup ids so neighbouring tiles share an XCD's
 *                    L2 (output is bit-identical either way), 0 = plain raster
 *   group_m        : tile rows per raster group when xcd_remap = 1 (>= 1)
 *   preload        : scheduling hint pair ([P1] "Changes" item 3 and its
 *                    review: a pair of non-negative integers, rejected
 *                    otherwise).  preload_dsrd = A fragments read from LDS
 *                    ahead of the matrix-core instructions that consume them;
 *                    preload_vmem = matrix-core instructions between two global
 *                    loads (0: loads placed by the compiler).  (0, 0) selects
 *                    the tile's tuned default; any other pair must name a
 *                    compiled kernel.
 *   waves_m        : tiled kernels: waves along M inside the workgroup; the
 *                    16-row streaming kernel (tile_m = 16, tile_n 32 or 64):
 *                    waves per workgroup, each owning tile_n / (16 * waves)
 *                    strips; the K-split kernel (8 or 16 waves): waves sharing
 *                    the tile's K range, which also tells the 16x32 and
 *                    16x64 K-split tiles from the streaming ones (0 = the
 *                    first compiled kernel for this tile: the streaming one);
 *                    the one-row tiles: waves sharing the K range (4, 8 or
 *                    16 compiled).
 *   prefetch       : tiled kernels: k-tiles loaded ahead of the one being
 *                    multiplied; 16-row and one-row kernels: steps of loads
 *                    in flight per wave (0 = any compiled depth for this
 *                    tile).
 *   schedule       : tiled kernels: how one workgroup's waves order their
 *                    work.  1 = interleaved: every wave mixes its LDS reads,
 *                    global loads and MFMAs, placed by the preload hints;
 *                    2 = ping-pong: each k-tile is cut into two phases, and
 *                    the two waves of every SIMD take turns, one issuing an
 *                    unbroken run of MFMAs while the other does its loads
 *                    (preload must be (0, 0)); 3 = both in LDS: A and the
 *                    preshuffled B tile both go global -> LDS with the async
 *                    copy (two stages), and the waves read both operands from
 *                    LDS; 4 = one wave per SIMD: 4 waves each owning all
 *                    256 rows and 64 columns of the 256x256 tile, 256
 *                    accumulators per lane in AGPRs (the built-in large-M
 *                    kernel for bf16, per-tensor fp8, mxfp8 and mxfp4);
 *                    0 = the tile's tuned default.
 *                    Must be 0 for the streaming kernel.  Zero-initialising
 *                    the whole struct and setting tile_m = 0 selects the
 *                    built-in table, like NULL. */
/*   a_layout       : tiled kernels: A's layout in LDS.  1 = 1 KiB operand
 *                    blocks (one async copy instruction = 16 rows x 64
 *                    bytes); 2 = row-major 128-byte rows with the 16-byte
 *                    chunks XOR-swizzled (one instruction = 8 whole rows,
 *                    the layout of [P1] "Changes" item 2); 0 = the tile's
 *                    tuned choice.  Schedules 1-3 use operand blocks;
 *                    schedule 4 compiles both.  Must be 0 for the 16-row
 *                    kernels.
 *   a_copy         : tiled kernels: how A reaches LDS.  1 = the async
 *                    global -> LDS buffer load ([P1] "Summary"); 2 = a
 *                    buffer load into registers and an LDS write (the path
 *                    [P1] replaced; schedule 4 keeps it to measure against);
 *                    0 = the tile's tuned choice (1).  Must be 0 for the
 *                    16-row kernels.
 *   preload pair, schedule 4: preload_dsrd = the LDS read-ahead in A
 *                    fragments (7 tuned; 3 and 1 compiled); preload_vmem =
 *                    1: a fragment's LDS read, B reloads and A copies sit
 *                    between its MFMAs, 0: all ahead of them. */
typedef struct dgp_config {
    int tile_m;
    int tile_n;
    int tile_k;
    int xcd_remap;
    int group_m;
    int preload_vmem;
    int preload_dsrd;
    int waves_m;
    int prefetch;
    int schedule;
    int a_layout;
    int a_copy;
} dgp_config;

/*
 * dgp_preshuffle_b -- reorder B into the layout the GEMM reads.
 *
 * B ([N][K] of `dtype`, row-major) -> Bs (same byte count).  With
 * Kb = K * element_bytes, Bs is a sequence of 1024-byte blocks, one per
 * (nb, kb) for nb < N/16, kb < Kb/64, block index nb*(Kb/64) + kb; inside a
 * block, byte g*256 + nn*16 + j (g < 4, nn < 16, j < 16) holds byte
 * kb*64 + g*16 + j of row nb*16 + nn.  A wave reading 16 bytes per lane from
 * one block therefore receives one 16x16 matrix-core operand tile: lane l gets
 * row 16*nb + l%16 of B, K-bytes 64*kb + 16*(l/16) .. +15.  The pages name this
 * preshuffled layout ([P1] title and file table, [P3] "bpreshuffle") without
 * writing it out; this is the library's own definition.  The layout is
 * byte-granular, so one packer serves both element types.
 *
 * Requires N % 16 == 0, (K * element_bytes) % 64 == 0, N, K >= 0, B and Bs
 * 16-byte aligned and not overlapping.  Run it ONCE per weight: Bs is always
 * treated as already preshuffled and no other entry point shuffles B again
 * (preshuffling twice corrupts the result, the hazard flagged on [P3]).
 */
dgp_status dgp_preshuffle_b(const void *B, void *Bs, int64_t N, int64_t K, int dtype, void *stream);

/* dgp_unshuffle_b -- the inverse permutation (Bs -> B).  Same rules. */
dgp_status dgp_unshuffle_b(const void *Bs, void *B, int64_t N, int64_t K, int dtype, void *stream);

/*
 * dgp_gemm_preshuffle -- C = A * B^T, single pass, bf16 output.
 *
 * A: [M][K] `dtype`, Bs: dgp_preshuffle_b(B), C: [M][N] bf16.  fp32
 * accumulation; scales per `scale_mode` (see dgp_scale_mode) applied in the
 * epilogue; the result is rounded to bf16 once, to nearest-even ([P1]
 * "Performance": bf16 in, bf16 out; [P3] "What's included": direct-output
 * epilogue for every scale mode).
 *
 * Requires M, N, K >= 0; N % 16 == 0; row bytes % 128 == 0 (bf16: K % 64,
 * fp8: K % 128 -- the fp8 matrix-core step is 128 deep, fp4: K % 256); blockscale
 * also N % 128 == 0 and K % 128 == 0 (rejected, never rounded up: the review
 * on [P3] flags the silent ceil-division), mxfp8 K % 128 == 0; A, Bs, C
 * 16-byte aligned.  sA, sB: device pointers to the scales of `scale_mode`.
 * M = 0 or N = 0 is a no-op returning DGP_OK.  The device must be gfx950.
 *
 * One pass puts the whole K range of a tile in one workgroup.  Decode-sized
 * M and small grids (M <= 256 with a weight of at most 8 MiB) take 16-row
 * tiles that spread K over the waves of each workgroup; other shapes whose
 * tile grid has fewer tiles than the GPU has CUs (256) leave CUs idle, and
 * for them dgp_gemm_preshuffle_splitk with split_k > 1 fills more of the
 * GPU (the library allocates no workspace of its own to split K here).
 */
dgp_status dgp_gemm_preshuffle(const void *A, const void *Bs, void *C, int64_t M, int64_t N, int64_t K,
                               int dtype, int scale_mode, const void *sA, const void *sB,
                               const dgp_config *cfg, void *stream);

/* Bytes of fp32 workspace dgp_gemm_preshuffle_splitk needs:
 * split_k * M * N * 4 for split_k > 1, 0 for split_k == 1. */
size_t dgp_splitk_workspace_bytes(int64_t M, int64_t N, int split_k);

/*
 * dgp_gemm_preshuffle_splitk -- two-pass split-K GEMM for decode-sized M.
 *
 * Pass 1 splits K into split_k equal contiguous ranges; each range's fp32
 * partial (scales applied) is written to ws[s][M][N].  Pass 2, a second kernel
 * on the same stream, sums the partials in order s = 0..split_k-1 in fp32 and
 * rounds to bf16 once ([P3] "What's included" and its file table: fp32
 * workspace partials, a reduction kernel that downcasts once, a two-pass
 * driver).  split_k == 1 takes the direct epilogue and ignores ws ([P3]: the
 * single-pass split_k = 1 epilogue).
 *
 * Requires everything dgp_gemm_preshuffle does, plus split_k >= 1,
 * K % split_k == 0 and ((K/split_k)*element_bytes) % 128 == 0 (blockscale and
 * mxfp8: (K/split_k) % 128 == 0); for split_k > 1, ws != NULL, 16-byte aligned, and
 * ws_bytes >= dgp_splitk_workspace_bytes(M, N, split_k).  ws is scratch owned
 * by the caller; its contents after the call are unspecified.
 */
dgp_status dgp_gemm_preshuffle_splitk(const void *A, const void *Bs, void *C, int64_t M, int64_t N,
                                      int64_t K, int dtype, int scale_mode, const void *sA,
                                      const void *sB, int split_k, float *ws, size_t ws_bytes,
                                      const dgp_config *cfg, void *stream);

/*
 * dgp_gemm_preshuffle_splitk_noalloc -- dgp_gemm_preshuffle_splitk without a
 * caller workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * allocation).
 *
 * Same arguments, rules, kernels and results as dgp_gemm_preshuffle_splitk
 * (bit-identical output), except that pass 1's fp32 partials go to an array
 * the library keeps in device memory: DGP_NOALLOC_SCRATCH_BYTES (16 MiB) per
 * GPU, held from its first use on that GPU until the process ends.  The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller passes A, Bs, C and the scales as usual.  Returns
 * DGP_ERR_WORKSPACE, with nothing enqueued, when split_k > 1 and
 * split_k * M * N * 4 > DGP_NOALLOC_SCRATCH_BYTES (e.g. M = 16, N = 16384
 * fits up to split_k = 16).  split_k == 1 uses no scratch.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap on one GPU (on different streams, or from
 * different host threads) race on it and may produce wrong results; order
 * them on one stream or use dgp_gemm_preshuffle_splitk with a workspace each.
 */
#define DGP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
dgp_status dgp_gemm_preshuffle_splitk_noalloc(const void *A, const void *Bs, void *C, int64_t M, int64_t N,
                                              int64_t K, int dtype, int scale_mode, const void *sA,
                                              const void *sB, int split_k, const dgp_config *cfg,
                                              void *stream);

/* dgp_check_arch -- DGP_OK if `gcn_arch_name` (as reported by the HIP device
 * properties, e.g. "gfx950:sramecc+:xnack-") names gfx950, else DGP_ERR_ARCH.
 * Pure host function.  The async global->LDS copy the GEMM depends on exists
 * on gfx950 only ([P1] review: fail early off gfx950). */
dgp_status dgp_check_arch(const char *gcn_arch_name);

/* dgp_status_string -- static, human-readable name of a status code. */
const char *dgp_status_string(int status);

/* dgp_last_error -- detail message of the last failing call on this thread
 * (static thread-local storage; empty string if none). */
const char *dgp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DGP_H */
