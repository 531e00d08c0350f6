/*
 * CPU oracle for the preshuffled-B GEMM  C = A * B^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, call or
 * link this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library under dense_gemm_packer_amd/csrc.
 *
 * What it computes, and where the pages say so:
 *
 *  - The operation: C[m][n] = sum_k A[m][k] * B[n][k] with fp32 accumulation
 *    and a bf16 result.  B is held as [N][K] (K contiguous): the blockscale
 *    review comment on aiter PR #5148 ("FlyDSL split-K preshuffle decode GEMM
 *    for small-M shapes") takes m, k from the activation's shape and n from the
 *    weight's first dimension.  The same PR validates every scale mode against
 *    an FP32 reference (section "Correctness").
 *  - Scale modes (aiter PR #5148, "Summary" / "What's included"): none (bf16),
 *    FP8 per-tensor (one fp32 scale each for A and B), FP8 blockscale (A per
 *    row per 128-wide K block, B per 128x128 block; shapes [M][K/128] and
 *    [N/128][K/128] from the run_torch_blockscale review comment), and the MX
 *    mode mxfp8 (same PR, "What's included": 128-element blocks with one E8M0
 *    scale each, applied by the hardware-scaled matrix instruction) and mxfp4
 *    (same list: 4-bit packed elements, 32-element blocks with one E8M0 scale
 *    each).
 *  - Split-K (aiter PR #5148, "What's included" and the file table): each of
 *    split_k K-chunks produces fp32 partials in a workspace and a second pass
 *    reduces them in fp32, rounding to the output type once.
 *  - The preshuffled layout of B ("bpreshuffle") is named on both FlyDSL PR
 *    #1008 and aiter PR #5148 but never written out; this file fixes one
 *    concrete byte permutation (oracle_preshuffle_b) and its inverse.
 *
 * Readings taken where the pages are silent:
 *  - fp8 is OCP e4m3fn: bias 7, no infinities, S.1111.111 is NaN, max 448.
 *  - fp32 -> bf16 rounds to nearest, ties to even; NaN stays a quiet NaN.
 *  - per-tensor scaling multiplies the fp32 sum by (sA*sB), the product of the
 *    two scales formed once in fp32; blockscale multiplies each 128-K block's
 *    fp32 partial sum by (sA[m][kb]*sB[n/128][kb]) and adds it to the running
 *    fp32 sum in one fused multiply-add (fmaf: one rounding per block; the
 *    pages leave that rounding open, and the fused form is what a GPU's
 *    fp32 multiply-add instruction computes).
 *  - split s covers K range [s*K/S, (s+1)*K/S); partials carry the scales; the
 *    reduce adds P_0 + P_1 + ... + P_{S-1} in that order.
 *  - mxfp8: an E8M0 byte e means 2^(e-127) (e = 255: NaN), as in the OCP
 *    microscaling format; A has one scale per row per 128-K block ([M][K/128]
 *    bytes) and B one per row of B, i.e. per output column, per 128-K block
 *    ([N][K/128] bytes), both row-major.  As for blockscale, each block's
 *    fp32 partial sum p is scaled and added: acc += p * 2^(eA-127) * 2^(eB-127),
 *    the power of two applied exactly (ldexpf).
 *  - mxfp4: elements are OCP E2M1 (1 sign, 2 exponent bits with bias 1, 1
 *    mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), packed two per byte with
 *    element 2j in the low nibble of byte j and 2j+1 in the high nibble; K
 *    counts elements, a row is K/2 bytes.  Scales as for mxfp8 but per 32-K
 *    block: A [M][K/32], B [N][K/32] E8M0 bytes; each 32-block's fp32 partial
 *    is scaled and added.
 *
 * Build: plain C11, -O2 -ffp-contract=off, no fast-math (so that every fp32
 * multiply and add rounds separately, in the order written here, and only
 * the explicit fmaf fuses).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_BF16 = 0, ORC_FP8_E4M3 = 1, ORC_FP4_E2M1 = 2 };
enum { ORC_SCALE_NONE = 0, ORC_SCALE_TENSOR = 1, ORC_SCALE_BLOCK128 = 2, ORC_SCALE_MX128 = 3, ORC_SCALE_MX32 = 4 };

/* ---------------------------------------------------------------- decode */

/* bf16 is the top half of an IEEE-754 binary32: widening is exact. */
float oracle_bf16_decode(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP 8-bit float E4M3 ("fn" variant): 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the single
 * code S.1111.111 is NaN and there is no infinity. */
float oracle_e4m3_decode(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int m = b & 0x7;
    float mag;
    if (e == 0xF && m == 0x7)
        return sign ? -NAN : NAN;
    if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -mag : mag;
}

/* OCP 4-bit float E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
 * bit; exponent field 0 is subnormal (m * 0.5).  All 16 codes are finite. */
float oracle_e2m1_decode(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int m = nibble & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------ fp32 -> bf16 */

/* E8M0 scale byte (OCP microscaling): 2^(e-127); e = 255 encodes NaN.  The
 * smallest, 2^-127, is an fp32 subnormal and exact. */
float oracle_e8m0_decode(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexpf(1.0f, (int)e - 127);
}

/* Round to nearest, ties to even, on the bit pattern: add 0x7FFF plus the
 * lowest kept bit, then truncate.  Overflow carries into the exponent and
 * gives +-inf; NaN inputs map to a quiet NaN with the sign kept. */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------- preshuffle layout */

/*
 * The preshuffled B, bytes.  Kb = K * element_bytes.  Bs is a sequence of
 * 1024-byte blocks, one per (nb, kb), nb in [0, N/16), kb in [0, Kb/64), the
 * block for (nb, kb) at block index nb*(Kb/64) + kb (so one 16-row strip is
 * contiguous along K).  Inside a block, byte g*256 + nn*16 + j (g < 4,
 * nn < 16, j < 16) holds byte kb*64 + g*16 + j of row nb*16 + nn.
 *
 * Requires N % 16 == 0 and Kb % 64 == 0; returns -1 otherwise.
 */
int oracle_preshuffle_b(const uint8_t *B, uint8_t *Bs, int64_t N, int64_t Kb)
{
    if (N % 16 != 0 || Kb % 64 != 0 || N < 0 || Kb < 0)
        return -1;
    int64_t kblocks = Kb / 64;
    for (int64_t nb = 0; nb < N / 16; ++nb)
        for (int64_t kb = 0; kb < kblocks; ++kb)
            for (int g = 0; g < 4; ++g)
                for (int nn = 0; nn < 16; ++nn)
                    for (int j = 0; j < 16; ++j) {
                        int64_t dst = (nb * kblocks + kb) * 1024 + g * 256 + nn * 16 + j;
                        int64_t src = (nb * 16 + nn) * Kb + kb * 64 + g * 16 + j;
                        Bs[dst] = B[src];
                    }
    return 0;
}

/* The inverse permutation of oracle_preshuffle_b. */
int oracle_unshuffle_b(const uint8_t *Bs, uint8_t *B, int64_t N, int64_t Kb)
{
    if (N % 16 != 0 || Kb % 64 != 0 || N < 0 || Kb < 0)
        return -1;
    int64_t kblocks = Kb / 64;
    for (int64_t nb = 0; nb < N / 16; ++nb)
        for (int64_t kb = 0; kb < kblocks; ++kb)
            for (int g = 0; g < 4; ++g)
                for (int nn = 0; nn < 16; ++nn)
                    for (int j = 0; j < 16; ++j) {
                        int64_t src = (nb * kblocks + kb) * 1024 + g * 256 + nn * 16 + j;
                        int64_t dst = (nb * 16 + nn) * Kb + kb * 64 + g * 16 + j;
                        B[dst] = Bs[src];
                    }
    return 0;
}

/* ------------------------------------------------------------------- GEMM */

typedef struct {
    const float *a;      /* decoded A, [M][K] */
    const float *b;      /* decoded B, [N][K] (unshuffled) */
    int64_t M, N, K;
    int scale_mode;
    const float *sA, *sB;      /* per-tensor and blockscale scales */
    const uint8_t *eA, *eB;    /* mxfp8 E8M0 scales */
    int split_k;
    const int64_t *rows; /* rows of C to compute; NULL = 0..nrows-1 */
    int64_t nrows;
    float *out_f32;      /* [nrows][N], value before the bf16 rounding (may be NULL) */
    uint16_t *out_bf16;  /* [nrows][N] (may be NULL) */
    float *partials;     /* [split_k][nrows][N] (may be NULL) */
    int64_t r_begin, r_end;
} gemm_job;

/* One split's fp32 partial for output (m, n) over K range [k0, k1),
 * scales applied. */
static float partial_sum(const gemm_job *j, int64_t m, int64_t n, int64_t k0, int64_t k1)
{
    const float *arow = j->a + m * j->K;
    const float *brow = j->b + n * j->K;
    if (j->scale_mode == ORC_SCALE_MX128 || j->scale_mode == ORC_SCALE_MX32) {
        const int64_t bs = j->scale_mode == ORC_SCALE_MX128 ? 128 : 32;   /* block size */
        int64_t kblocks = j->K / bs;
        float acc = 0.0f;
        for (int64_t kb = k0 / bs; kb < k1 / bs; ++kb) {
            float p = 0.0f;
            for (int64_t k = kb * bs; k < kb * bs + bs; ++k)
                p += arow[k] * brow[k];
            uint8_t ea = j->eA[m * kblocks + kb], eb = j->eB[n * kblocks + kb];
            if (ea == 255 || eb == 255)
                p = NAN;
            else
                p = ldexpf(p, ((int)ea - 127) + ((int)eb - 127));
            acc += p;
        }
        return acc;
    }
    if (j->scale_mode == ORC_SCALE_BLOCK128) {
        int64_t kblocks = j->K / 128;
        float acc = 0.0f;
        for (int64_t kb = k0 / 128; kb < k1 / 128; ++kb) {
            float p = 0.0f;
            for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
                p += arow[k] * brow[k];
            float s = j->sA[m * kblocks + kb] * j->sB[(n / 128) * kblocks + kb];
            acc = fmaf(p, s, acc);
        }
        return acc;
    }
    float acc = 0.0f;
    for (int64_t k = k0; k < k1; ++k)
        acc += arow[k] * brow[k];
    if (j->scale_mode == ORC_SCALE_TENSOR) {
        float s = j->sA[0] * j->sB[0];
        acc = acc * s;
    }
    return acc;
}

static void *gemm_worker(void *arg)
{
    gemm_job *j = (gemm_job *)arg;
    int S = j->split_k;
    for (int64_t i = j->r_begin; i < j->r_end; ++i) {
        int64_t m = j->rows ? j->rows[i] : i;
        for (int64_t n = 0; n < j->N; ++n) {
            float total = 0.0f;
            for (int s = 0; s < S; ++s) {
                int64_t k0 = (j->K / S) * s, k1 = (j->K / S) * (s + 1);
                float p = partial_sum(j, m, n, k0, k1);
                if (j->partials)
                    j->partials[((int64_t)s * j->nrows + i) * j->N + n] = p;
                total = (s == 0) ? p : total + p;
            }
            if (j->out_f32)
                j->out_f32[i * j->N + n] = total;
            if (j->out_bf16)
                j->out_bf16[i * j->N + n] = oracle_bf16_round(total);
        }
    }
    return NULL;
}

static float *decode_all(const void *src, int64_t count, int dtype)
{
    float *dst = (float *)malloc((size_t)(count > 0 ? count : 1) * sizeof(float));
    if (!dst)
        return NULL;
    if (dtype == ORC_BF16) {
        const uint16_t *h = (const uint16_t *)src;
        for (int64_t i = 0; i < count; ++i)
            dst[i] = oracle_bf16_decode(h[i]);
    } else if (dtype == ORC_FP8_E4M3) {
        const uint8_t *q = (const uint8_t *)src;
        for (int64_t i = 0; i < count; ++i)
            dst[i] = oracle_e4m3_decode(q[i]);
    } else {   /* E2M1, two per byte, element 2j in the low nibble */
        const uint8_t *q = (const uint8_t *)src;
        for (int64_t i = 0; i < count; ++i)
            dst[i] = oracle_e2m1_decode((uint8_t)((q[i / 2] >> (4 * (i & 1))) & 0xF));
    }
    return dst;
}

/*
 * Compute rows of C.  A is [M][K] and B is [N][K] (unshuffled), both of
 * element type dtype (bf16 bit patterns, e4m3 codes, or packed e2m1 pairs --
 * K elements = K/2 bytes per row).  sA, sB: fp32 scales (per-tensor,
 * blockscale) or E8M0 bytes (mxfp8, mxfp4), unused for scale mode none.
 * rows lists which rows
 * of C to produce (NULL: all M rows, nrows must equal M).  Outputs are indexed
 * by position in rows.  Returns 0, or -1 on an invalid argument.
 */
int oracle_gemm_rows(const void *A, const void *B, int64_t M, int64_t N, int64_t K,
                     int dtype, int scale_mode, const void *sA, const void *sB,
                     int split_k, const int64_t *rows, int64_t nrows,
                     float *out_f32, uint16_t *out_bf16, float *partials, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || split_k < 1)
        return -1;
    if (dtype != ORC_BF16 && dtype != ORC_FP8_E4M3 && dtype != ORC_FP4_E2M1)
        return -1;
    if (scale_mode < ORC_SCALE_NONE || scale_mode > ORC_SCALE_MX32)
        return -1;
    /* e2m1 comes with its 32-block scales and nothing else */
    if ((dtype == ORC_FP4_E2M1) != (scale_mode == ORC_SCALE_MX32))
        return -1;
    if (scale_mode == ORC_SCALE_MX32 && (K % 32 != 0 || (K / split_k) % 32 != 0 || K % 2 != 0))
        return -1;
    if (scale_mode == ORC_SCALE_MX128 && (dtype != ORC_FP8_E4M3 || K % 128 != 0 || (K / split_k) % 128 != 0))
        return -1;
    if (scale_mode != ORC_SCALE_NONE && (!sA || !sB))
        return -1;
    if (K % split_k != 0)
        return -1;
    if (scale_mode == ORC_SCALE_BLOCK128 && (K % 128 != 0 || N % 128 != 0 || (K / split_k) % 128 != 0))
        return -1;
    if (!rows && nrows != M)
        return -1;
    if (rows)
        for (int64_t i = 0; i < nrows; ++i)
            if (rows[i] < 0 || rows[i] >= M)
                return -1;

    float *a = decode_all(A, M * K, dtype);
    float *b = decode_all(B, N * K, dtype);
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
    if (nthreads <= 0)
        nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nrows)
        nthreads = nrows > 0 ? (int)nrows : 1;

    const int mx = scale_mode == ORC_SCALE_MX128 || scale_mode == ORC_SCALE_MX32;
    gemm_job base = {a, b, M, N, K, scale_mode, mx ? NULL : (const float *)sA, mx ? NULL : (const float *)sB,
                     mx ? (const uint8_t *)sA : NULL, mx ? (const uint8_t *)sB : NULL, split_k, rows, nrows,
                     out_f32, out_bf16, partials, 0, 0};
    gemm_job *jobs = (gemm_job *)malloc(sizeof(gemm_job) * (size_t)nthreads);
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    char *made = (char *)calloc((size_t)nthreads, 1);
    int rc = 0;
    if (!jobs || !tids || !made) {
        rc = -1;
    } else {
        for (int t = 0; t < nthreads; ++t) {
            jobs[t] = base;
            jobs[t].r_begin = nrows * t / nthreads;
            jobs[t].r_end = nrows * (t + 1) / nthreads;
            if (nthreads > 1 && pthread_create(&tids[t], NULL, gemm_worker, &jobs[t]) == 0)
                made[t] = 1;
            else
                gemm_worker(&jobs[t]);
        }
        for (int t = 0; t < nthreads; ++t)
            if (made[t])
                pthread_join(tids[t], NULL);
    }
    free(made);
    free(jobs);
    free(tids);
    free(a);
    free(b);
    return rc;
}

/* Number of threads the oracle uses when nthreads <= 0 is passed. */
int oracle_default_threads(void)
{
    return (int)sysconf(_SC_NPROCESSORS_ONLN);
}
