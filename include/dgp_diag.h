/*
 * dgp_diag.h -- diagnostic entry points of the gfx950 preshuffled-B GEMM
 * library: the workgroup -> tile map, and small probe kernels used to check
 * hardware facts the GEMM relies on and to measure the roofline walls.
 * Same conventions as dgp.h (device pointers owned by the caller, async on
 * `stream`, host-side validation first).
 */
#ifndef DGP_DIAG_H
#define DGP_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "dgp.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dgp_tile_of_workgroup -- host mirror of the device workgroup -> tile map.
 *
 * For a grid of tiles_m x tiles_n x splits workgroups, returns in out[0..2]
 * the (tile_m index, tile_n index, split index) that workgroup `wg` computes.
 * With xcd_remap = 1 the ids are first regrouped so that the workgroups the
 * hardware places on one XCD (ids congruent mod 8 -- 8 XCDs on gfx950) get
 * consecutive logical ids, and logical ids are rastered in groups of group_m
 * tile rows, keeping tiles that share A rows or B columns on one XCD's L2.
 * This is the workgroup-order swizzle exposed as xcd_swizzle on [P1]
 * "Performance" and re-derived from the linear workgroup id in the attention
 * XCD-remap commit on [P2]; the map is a bijection, so the output is
 * bit-identical with or without it.  Returns DGP_ERR_SHAPE for bad arguments.
 */
dgp_status dgp_tile_of_workgroup(int64_t wg, int64_t tiles_m, int64_t tiles_n, int64_t splits,
                                 int xcd_remap, int group_m, int64_t out[3]);

/*
 * dgp_tile_map -- the same map for every workgroup of the grid at once:
 * out[3*wg .. 3*wg+2] = (tile_m index, tile_n index, split index) for
 * wg = 0 .. tiles_m*tiles_n*splits - 1.  `out` is a caller-owned host array
 * of out_len int64 values (at least 3 per workgroup).  Pure host code, so a
 * test can check the map is a bijection over many grid sizes cheaply.
 * Returns DGP_ERR_NULL for a NULL out, DGP_ERR_SHAPE for bad arguments or
 * an out array that is too short.
 */
dgp_status dgp_tile_map(int64_t tiles_m, int64_t tiles_n, int64_t splits, int xcd_remap, int group_m,
                        int64_t *out, int64_t out_len);

/*
 * dgp_kernel_info -- describe compiled GEMM kernel number `index`
 * (0 <= index < dgp_kernel_count()).  Fills *cfg with the configuration that
 * selects exactly this kernel through dgp_gemm_preshuffle[_splitk] (xcd_remap
 * and group_m set to the defaults), and *dtype, *scale_mode with the element
 * type and scale mode it computes; *split_out = 1 if it is the fp32-partial
 * (split_k > 1) variant, 0 if it writes bf16 C directly.  Pure host function.
 */
int dgp_kernel_count(void);
dgp_status dgp_kernel_info(int index, dgp_config *cfg, int *dtype, int *scale_mode, int *split_out);

/*
 * dgp_lds_poison -- 1 in the LDS-poison debug build of the library
 * (libdgp_lds_poison.so: the same sources compiled with DGP_LDS_POISON=1),
 * 0 in the release build.  In the debug build every GEMM kernel fills its
 * LDS with 0xFF bytes before its first global -> LDS copy, and every copy
 * first overwrites its own destination with 0xFF and waits for that write:
 * a read of LDS that no copy filled, or one that runs ahead of the wait for
 * its copy, yields NaN (bf16, e4m3, E8M0 and fp32 bytes) or -6 (E2M1) and
 * fails a bit-exact parity check, instead of giving a plausible wrong
 * answer at full speed -- the failure mode of a tile only partly loaded
 * ([P2] follow-up commit, item 1).  Same entry points, same results on
 * correct kernels; slower, for tests only.  Pure host function.
 */
int dgp_lds_poison(void);

/*
 * dgp_select_kernel -- which compiled GEMM kernel a call would launch.
 *
 * Runs the shape and configuration checks of dgp_gemm_preshuffle_splitk
 * (dgp_gemm_preshuffle when split_k = 1) for these arguments -- no buffers,
 * no device -- and stores in *index the table index (as numbered by
 * dgp_kernel_info) of the GEMM kernel that call would launch, or -1 when it
 * would launch none (M = 0, N = 0 or K = 0).  Returns the status the GEMM
 * entry point would return for a shape or configuration error.
 * Pure host function.
 */
dgp_status dgp_select_kernel(int64_t M, int64_t N, int64_t K, int dtype, int scale_mode, int split_k,
                             const dgp_config *config, int *index);

/*
 * dgp_probe_mfma_layout -- run each matrix-core instruction the GEMM uses once
 * on operands the caller supplies and store the raw accumulator registers.
 *   which = 0: v_mfma_f32_16x16x32_bf16   (a, b: 64 lanes x 16 bytes)
 *   which = 1: v_mfma_f32_16x16x128_f8f6f4 with e4m3 operands (64 lanes x 32 bytes)
 * a, b: device buffers of 64*16 (which 0) or 64*32 (which 1) bytes, lane-major.
 * out: device buffer of 64*4 fp32 (lane-major, 4 accumulator registers).
 */
dgp_status dgp_probe_mfma_layout(int which, const void *a, const void *b, float *out, void *stream);

/*
 * dgp_probe_mfma_scaled -- one hardware-scaled matrix-core instruction
 * (v_mfma_scale_f32_16x16x128_f8f6f4) with per-lane E8M0 scales, operands in
 * the order the GEMM uses: the B fragment is the instruction's first operand
 * (scale sb[l]) and the A fragment its second (scale sa[l]).
 * which = 0: e4m3 operands, 32 bytes per lane; which = 1: e2m1 operands, 16
 * bytes (32 values) per lane taken from the first half of its 32-byte slot.
 * a, b: device buffers of 64 lanes x 32 bytes (lane-major); sa, sb: 64 bytes
 * each; out: 64 x 4 fp32 (lane-major accumulator registers).
 */
dgp_status dgp_probe_mfma_scaled(int which, const void *a, const void *b, const void *sa, const void *sb,
                                 float *out, void *stream);

/*
 * dgp_probe_lds_dma -- one wave copies 64 x 16 bytes from src (lane l reads
 * the 16 bytes at src + perm[l]*16) into LDS with the async global->LDS load
 * the GEMM uses, then copies LDS bytes 0..1023 to dst unchanged, revealing
 * where each lane's bytes landed.  src: >= 1024 bytes, perm: 64 int32 in
 * [0, 64), dst: 1024 bytes.
 */
dgp_status dgp_probe_lds_dma(const void *src, const int32_t *perm, void *dst, void *stream);

/*
 * dgp_probe_lds_dma_narrow -- the same async global->LDS load at 1, 2 or 4
 * bytes per lane (the width the GEMM uses to stage per-k-tile scales): LDS
 * bytes 0..1023 are set to 0xFF, lane l loads `width` bytes at
 * src + perm[l]*width, and LDS bytes 0..1023 are copied to dst, showing where
 * each lane's bytes landed and which bytes stayed 0xFF.
 * width: 1, 2 or 4 (else DGP_ERR_CONFIG); src: >= 64*width bytes, 16-byte
 * aligned; perm: 64 int32 in [0, 64); dst: 1024 bytes, 16-byte aligned.
 */
dgp_status dgp_probe_lds_dma_narrow(int width, const void *src, const int32_t *perm, void *dst, void *stream);

/*
 * dgp_probe_copy -- plain 16-byte-per-thread device copy of `bytes` bytes
 * (bytes % 16 == 0).  The reference kernel of known traffic used to calibrate
 * hardware byte counters.
 */
dgp_status dgp_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * dgp_probe_stream_read -- read `bytes` bytes (bytes % 16 == 0) with
 * `blocks` workgroups of 512 threads (1 <= blocks <= 65536), workgroup b
 * reading one contiguous span of about bytes/blocks front to back with
 * 16-byte non-temporal loads, 8 in flight per thread, and write one 32-bit
 * xor-fold per workgroup to `sink` (>= 4096 uint32, normally left untouched).
 * Measures the attainable HBM read rate for a range of that size (time it
 * for a few values of `blocks` and keep the best).
 */
dgp_status dgp_probe_stream_read(const void *src, int64_t bytes, int blocks, uint32_t *sink, void *stream);

/*
 * dgp_probe_mfma_peak -- sustained matrix-core rate on given operands.
 * `blocks` workgroups of 4 waves each; every wave loads 8 A and 8 B fragments
 * (operand set w % 256 for wave w) into registers and runs `rounds` rounds of
 * 64 MFMAs over 8 independent accumulators, with no memory traffic in the
 * loop.  which = 0 issues v_mfma_f32_16x16x32_bf16 (16384 FLOP each),
 * which = 1 the block-scaled e4m3 16x16x128 form and which = 2 the
 * block-scaled E2M1 16x16x128 form (65536 FLOP each; unit E8M0 scales);
 * total FLOP = blocks*4*rounds*64*that.  The matrix units draw more power on operands that
 * toggle, so timing this on the workload's own data gives the MFMA wall at
 * the clock the chip holds for that data; constant operands give the rate
 * near the spec clock.
 *   operands: device buffer of 256 sets x 16 fragments x 64 lanes x 16 bytes
 *             (which 0 and 2: 4 MiB) or x 32 bytes (which 1: 8 MiB), set-major,
 *             A fragments 0..7 then B fragments 0..7, lane-major inside a
 *             fragment.  Read once per wave.
 *   sink: >= 4096 uint32, normally left untouched.
 * which outside 0..2: DGP_ERR_CONFIG.  rounds in [1, 2^24], blocks in
 * [1, 65536], else DGP_ERR_SHAPE.
 */
dgp_status dgp_probe_mfma_peak(int which, int rounds, int blocks, const void *operands, uint32_t *sink,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DGP_DIAG_H */
