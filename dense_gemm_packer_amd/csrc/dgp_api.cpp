// C-ABI layer of the gfx950 preshuffled-B GEMM library (include/dgp.h).
//
// Every entry point validates its arguments on the host first -- no HIP call
// is made for a rejected call -- then checks the device architecture, picks a
// compiled kernel and enqueues it on the caller's stream.  Nothing here
// allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/dgp.h"
#include "../../include/dgp_diag.h"
#include "common.h"
#include "launch.h"

using namespace dgp;

namespace dgp {

const KernelSpec *kernel_table(int *count)
{
    static const std::vector<KernelSpec> all = [] {
        std::vector<KernelSpec> v;
        int n = 0;
        const KernelSpec *t = tiled_kernels(&n);
        v.insert(v.end(), t, t + n);
        t = lds_kernels(&n);
        v.insert(v.end(), t, t + n);
        t = w4_kernels(&n);
        v.insert(v.end(), t, t + n);
        t = stream_kernels(&n);
        v.insert(v.end(), t, t + n);
        t = wave_kernels(&n);
        v.insert(v.end(), t, t + n);
        return v;
    }();
    *count = (int)all.size();
    return all.data();
}

}  // namespace dgp

namespace {

thread_local char g_err[512];

dgp_status fail(dgp_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

dgp_status ok()
{
    g_err[0] = '\0';
    return DGP_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Bytes of a row of K elements (fp4 packs two elements per byte).
int64_t row_bytes(int dtype, int64_t K) { return dtype == DGP_BF16 ? 2 * K : dtype == DGP_FP4_E2M1 ? K / 2 : K; }
bool known_dtype(int dtype) { return dtype == DGP_BF16 || dtype == DGP_FP8_E4M3 || dtype == DGP_FP4_E2M1; }

// Per-row byte limit: keeps every in-tile offset of the kernels in 32 bits.
constexpr int64_t kMaxRowBytes = int64_t(1) << 23;

// ---------------------------------------------------------------- arch

dgp_status check_device_arch()
{
    // Per-device answer, 0 unknown, 1 gfx950, 2 other.  Atomic: host threads
    // may make their first calls concurrently (both then store the same value).
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(DGP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64 && cached[dev].load(std::memory_order_acquire) == 1)
        return DGP_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
        return fail(DGP_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    dgp_status st = dgp_check_arch(prop.gcnArchName);
    if (dev >= 0 && dev < 64)
        cached[dev].store(st == DGP_OK ? 1 : 2, std::memory_order_release);
    if (st != DGP_OK)
        return fail(DGP_ERR_ARCH, "device %d is %s; this library runs on gfx950 only", dev,
                    prop.gcnArchName);
    return DGP_OK;
}

dgp_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(DGP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ------------------------------------------------------- kernel choice

struct Plan {
    const KernelSpec *spec;
    int tiles_m, tiles_n;
    int remap, group_m;
};

bool spec_fits(const KernelSpec &k, int64_t Ks)
{
    if (k.family == kTiled)
        return Ks % k.kt == 0;
    return true;   // stream: any K range that is a multiple of 128 bytes
}

// A kernel-table query; -1 in a field means "any".
struct Query {
    int family, dtype, scale, out, tm, tn;
    int kt = -1, wm = -1, depth = -1, pv = -1, pd = -1, sched = -1, lay = -1, copy = -1;
};

const KernelSpec *find_spec(const Query &q)
{
    int n = 0;
    const KernelSpec *t = kernel_table(&n);
    for (int i = 0; i < n; ++i) {
        const KernelSpec &k = t[i];
        const int wm = k.family == kTiled ? k.p0 : k.waves;
        if (k.family == q.family && k.dtype == q.dtype && k.scale == q.scale && k.out == q.out && k.tm == q.tm &&
            k.tn == q.tn && (q.kt < 0 || k.kt == q.kt) && (q.wm < 0 || wm == q.wm) &&
            (q.depth < 0 || k.depth == q.depth) && (q.pv < 0 || k.pv == q.pv) && (q.pd < 0 || k.pd == q.pd) &&
            (q.sched < 0 || k.sched == q.sched) && (q.lay < 0 || (k.family == kTiled && k.lay == q.lay)) &&
            (q.copy < 0 || (k.family == kTiled && k.copy == q.copy)))
            return &k;
    }
    return nullptr;
}

// Built-in per-shape choice.
const KernelSpec *default_spec(int dtype, int scale, int out, int64_t M, int64_t N, int64_t Ks, int split_k)
{
    // Decode-sized M streams the weight through the 16-row and one-row
    // tiles.  Larger M takes the tiled kernels, every scale mode included.
    if (M <= 32) {
        // Rules from cold sweeps of every 16-row and one-row tile at K = 7168
        // (every mode; M = 1, 2, 4 and 16; N 2048-16384; split 1-4).
        // u = strips x splits; ks(t, w) = the K-split tile t columns wide
        // (w waves, 8 unless given), st(t) = the streaming tile, wv(t, w, d) = the one-row VALU
        // tile with w waves and a d-step ring.
        const int64_t u = N / 16 * split_k;
        const bool fp8t = dtype == DGP_FP8_E4M3 && scale == DGP_SCALE_TENSOR;
        const bool mx4 = scale == DGP_SCALE_MX32;
        const bool bs = scale == DGP_SCALE_BLOCK128, mx8 = scale == DGP_SCALE_MX128;
        const auto ks = [&](int tn, int waves = 8) {
            Query q{kStream, dtype, scale, out, 16, tn};
            q.wm = waves;
            return find_spec(q);
        };
        const auto st = [&](int tn) {
            Query q{kStream, dtype, scale, out, 16, tn};
            q.wm = tn == 64 ? 4 : 2;
            return find_spec(q);
        };
        const auto wv = [&](int tn, int waves, int depth) {
            Query q{kWave, dtype, scale, out, 1, tn};
            q.wm = waves, q.depth = depth;
            return find_spec(q);
        };
        // One row, bf16 or per-tensor fp8: the one-row VALU tile (split 1 at
        // N = 2048: 6.4 vs 8.3 us bf16, 4.5 vs 5.3 us fp8; 0-4 % ahead of
        // the 16-row tiles at larger N and 1-11 % with splits), half strips
        // while one pass has fewer strips than CUs.
        if (M == 1 && (dtype == DGP_BF16 || fp8t)) {
            const KernelSpec *k = nullptr;
            if (split_k == 1 && N / 16 < 256)
                k = wv(8, 4, 8);
            else if (split_k == 1)
                k = dtype == DGP_BF16 ? wv(16, 8, 8) : wv(16, 4, 8);
            else
                k = (dtype == DGP_BF16 || split_k == 2) ? wv(16, 4, 8) : wv(16, 4, 4);
            if (k)
                return k;
        }
        // Blockscale and mxfp8 from 4 splits over at least 2048 strips x
        // splits: the streaming 16x64 tile (5-19 % ahead), whose A panel in
        // LDS serves four strips per wave.
        if (u >= 2048 && (bs || mx8) && split_k >= 4)
            return st(64);
        // mxfp4 in one pass over at most 512 strips: 16 waves per workgroup,
        // so each wave's K slice is one 4-step group of the guarded loop
        // (N = 2048: 5.6 vs 6.1 us at M = 16, 4.4 vs 5.0 at M = 1; N = 4096:
        // 6.2 vs 6.7 and 4.9 vs 5.4).
        if (mx4 && split_k == 1 && u <= 512) {
            const KernelSpec *k = u < 256 ? ks(M <= 4 ? 16 : 8, 16) : ks(u < 512 ? 16 : 32, 16);
            if (k)
                return k;
        }
        // Fewer strips x splits than CUs: half a strip per workgroup doubles
        // the workgroups with no second pass.
        if (u < 256)
            return ks(8);
        if (M <= 4) {
            // A few rows: A is cheap to re-read.  One pass: one strip per
            // workgroup with K over 8 waves.  With splits each wave's slice
            // is short, so 2 strips per workgroup lead (4-13 %), until the
            // streaming tile takes over from 2048 strips x splits at 4
            // splits; bf16 keeps one strip at 2 splits.
            if (fp8t || dtype == DGP_BF16 || mx4) {
                if (split_k == 1)
                    return ks(16);
                if (dtype == DGP_BF16)
                    return split_k == 2 ? ks(16) : ks(32);
                if (u < 1024)
                    return ks(16);
                return (split_k == 2 || u == 1024) ? ks(32) : st(64);
            }
            if (u < 512)
                return ks(16);
            // (mxfp8 in one or two passes: the 32-column tile, whose 3-step
            // ring keeps two workgroups per CU: 20.3-20.7 vs 20.9-21.1 us at
            // N = 16384)
            return (mx8 && u >= 1024 && split_k > 2) ? ks(64) : ks(32);
        }
        // More rows: A is read once per workgroup, so wider K-split tiles
        // (2 or 4 strips sharing each A fragment) lead from 512 strips x
        // splits (4-22 %); for mxfp4 the streaming tile leads again from
        // 2048.
        if (u < 512)
            return ks(16);
        if (mx4 && u >= 2048)
            return st(64);
        // (mxfp8 at 2 splits: 24.9 vs 25.6 us for the streaming tile at M =
        // 16, N = 16384)
        if (u < 1024 || fp8t || (mx8 && split_k == 2))
            return ks(32);
        // bf16 in one pass: the same 4 strips over 16 waves (M = 16, N =
        // 16384: 37.5 vs 38.8 us)
        if (dtype == DGP_BF16 && split_k == 1)
            if (const KernelSpec *k = ks(64, 16))
                return k;
        return ks(64);
    }
    // Small grids above 32 rows (e.g. bf16 128 x 256 x 256): fewer than 64
    // tiles of 128 x 128 and a weight of at most 8 MiB, in one pass.  The
    // 16-row K-split tile over ceil(M / 16) row tiles spreads K over the 8
    // waves of each workgroup where the 128 x 128 tile runs two workgroups
    // through K in sequence (2.8 vs 7.6 us per launch in a graph at 128 x 256
    // x 256); each row tile re-reads the weight, which at this size stays in
    // the L2.
    if (split_k == 1 && M <= 256 && ((M + 127) / 128) * ((N + 127) / 128) < 64 && N * Ks <= (int64_t(8) << 20)) {
        Query q{kStream, dtype, scale, out, 16, 16};
        q.wm = 8;
        if (const KernelSpec *k = find_spec(q))
            return k;
    }
    // Larger M: the tile whose grid finishes first.  A grid of t tiles (x
    // splits) runs in ceil(t / 256) rounds over the 256 CUs, and one round of
    // a 256x256 or 128x128 tile takes about 1.45 : 1 (bf16, fp8, mxfp8,
    // mxfp4; K = 2048 and 8192; blockscale's 8-wave 256x256 tile about
    // 2.05 : 1): 4096 x 4096 and 3072 x 3072 take the 256x256 tile, 2048 x
    // 2048 the 128x128 tile (91 vs 134 us; bf16 there now takes the 128x256
    // tile below).  Ties go to the larger tile.
    // bf16 and per-tensor fp8 run their 128x256 tile one wave per SIMD, two
    // workgroups per CU at once: the busiest CU's k tiles cost about 1.05
    // rounds of the 256x256 tile per pair and 0.74 for one alone (K = 8192:
    // 4096 x 6144 281 vs 314 us for the 256x256 tile, 4096 x 5120 260 vs
    // 307, 3072 x 4096 168 vs 153, 4096 x 4096 187 vs 178; fp8 alike).  A
    // lone tile against a 128x128 round: bf16 0.95 (2048 x 2048 x 8192: 77.8
    // vs 89.7 us), fp8 1.07 (51.0 vs 48.1 us).
    const auto rounds = [&](int64_t tm, int64_t tn) {
        return ((M + tm - 1) / tm * ((N + tn - 1) / tn) * split_k + 255) / 256;
    };
    const bool has_128x256 = scale == DGP_SCALE_NONE || scale == DGP_SCALE_TENSOR;   // (bf16 and fp8 per-tensor)
    const int64_t k128x256 = rounds(128, 256);   // 128x256 tiles on the busiest CU
    const int64_t c256 = (scale == DGP_SCALE_BLOCK128 ? 205 : 145) * rounds(256, 256),
                  c128x256 = has_128x256 ? 153 * (k128x256 / 2) + (dtype == DGP_BF16 ? 95 : 107) * (k128x256 % 2)
                                         : INT64_MAX,
                  c128 = 100 * rounds(128, 128);
    const KernelSpec *k = nullptr;
    if (c256 <= c128x256 && c256 <= c128) {
        // bf16, per-tensor fp8, mxfp8 and mxfp4: the one-wave-per-SIMD tile
        // with swizzled A rows (measured 8-18 % ahead of the 8-wave tile at
        // 4096 x 4096 x 8192); blockscale: the 8-wave tile.
        Query q{kTiled, dtype, scale, out, 256, 256};
        q.kt = 128;
        if (scale != DGP_SCALE_BLOCK128) {
            q.sched = kSchedW4, q.lay = kLaySwizzled;
        } else {
            q.wm = 1, q.depth = 2, q.pv = 0, q.pd = 4;
        }
        k = find_spec(q);
    } else if (c128x256 < c128) {
        // bf16 and per-tensor fp8: the one-wave-per-SIMD tile, 128 rows
        // (2048 x 4096 x 8192: 105.9 vs 123.8 us bf16, 60.5 vs 66.6 us fp8
        // against the 8-wave 128x256 tile in a sweep; bit-identical results)
        Query q{kTiled, dtype, scale, out, 128, 256};
        q.kt = 128, q.sched = kSchedW4, q.lay = kLaySwizzled;
        k = find_spec(q);
        if (!k) {
            q.sched = -1, q.lay = -1;
            k = find_spec(q);
        }
    }
    if (!k || !spec_fits(*k, Ks)) {
        Query q{kTiled, dtype, scale, out, 128, 128};
        q.kt = 128, q.pv = 0, q.pd = 4;
        k = find_spec(q);
    }
    return (k && spec_fits(*k, Ks)) ? k : nullptr;
}

// ---------------------------------------------------------- validation

struct GemmCall {
    const void *A, *Bs;
    void *C;
    int64_t M, N, K;
    int dtype, scale;
    const void *sA, *sB;
    int split_k;
    float *ws;
    size_t ws_bytes;
    const dgp_config *cfg;
    bool select_only = false;   // shapes and configuration only: no buffers checked
    bool lib_scratch = false;   // split-K partials go to the library's fixed array (ws unused)
};

// Kernel choice for a validated call: the configured tile, or the built-in
// per-shape table.
dgp_status select_kernel(const GemmCall &c, int64_t Ks, Plan *plan)
{
    const int out = c.split_k > 1 ? kOutPartial : kOutBf16;
    const KernelSpec *spec = nullptr;
    if (c.cfg && c.cfg->tile_m > 0) {
        const int fam = c.cfg->tile_m == 16 ? kStream : c.cfg->tile_m == 1 ? kWave : kTiled;
        if (c.cfg->waves_m < 0 || c.cfg->prefetch < 0)
            return fail(DGP_ERR_CONFIG, "waves_m and prefetch must be >= 0");
        if (c.cfg->schedule < 0 || c.cfg->schedule > kSchedW4)
            return fail(DGP_ERR_CONFIG, "schedule must be 0, 1, 2, 3 or 4 (got %d)", c.cfg->schedule);
        if (c.cfg->a_layout < 0 || c.cfg->a_layout > 2)
            return fail(DGP_ERR_CONFIG, "a_layout must be 0, 1 or 2 (got %d)", c.cfg->a_layout);
        if (c.cfg->a_copy < 0 || c.cfg->a_copy > 2)
            return fail(DGP_ERR_CONFIG, "a_copy must be 0, 1 or 2 (got %d)", c.cfg->a_copy);
        Query q{fam, c.dtype, c.scale, out, c.cfg->tile_m, c.cfg->tile_n};
        if (fam == kTiled) {
            q.kt = c.cfg->tile_k;
            q.wm = c.cfg->waves_m > 0 ? c.cfg->waves_m : -1;
            q.depth = c.cfg->prefetch > 0 ? c.cfg->prefetch : -1;
            // (0, 0) = this tile's tuned default hints; any other pair must
            // name a compiled kernel exactly.
            if (c.cfg->preload_vmem != 0 || c.cfg->preload_dsrd != 0) {
                q.pv = c.cfg->preload_vmem;
                q.pd = c.cfg->preload_dsrd;
            }
            if (c.cfg->schedule > 0)
                q.sched = c.cfg->schedule;
            if (c.cfg->a_layout > 0)
                q.lay = c.cfg->a_layout - 1;
            q.copy = c.cfg->a_copy > 0 ? c.cfg->a_copy - 1 : kCopyAsync;
        } else {
            if (c.cfg->preload_vmem != 0 || c.cfg->preload_dsrd != 0)
                return fail(DGP_ERR_CONFIG, "the 16-row and one-row kernels take no preload hints");
            if (c.cfg->schedule != 0)
                return fail(DGP_ERR_CONFIG, "the 16-row and one-row kernels have no schedule choice");
            if (c.cfg->a_layout != 0 || c.cfg->a_copy != 0)
                return fail(DGP_ERR_CONFIG, "the 16-row and one-row kernels have no A layout or copy choice");
            q.wm = c.cfg->waves_m > 0 ? c.cfg->waves_m : -1;   // matched against waves per workgroup
            q.depth = c.cfg->prefetch > 0 ? c.cfg->prefetch : -1;
        }
        spec = find_spec(q);
        if (!spec)
            return fail(DGP_ERR_CONFIG,
                        "no compiled kernel for tile %dx%dx%d (waves_m %d, prefetch %d, preload %d,%d, schedule %d, "
                        "a_layout %d, a_copy %d) with this dtype/scale", c.cfg->tile_m, c.cfg->tile_n, c.cfg->tile_k,
                        c.cfg->waves_m, c.cfg->prefetch, c.cfg->preload_vmem, c.cfg->preload_dsrd, c.cfg->schedule,
                        c.cfg->a_layout, c.cfg->a_copy);
        if (!spec_fits(*spec, Ks))
            return fail(DGP_ERR_CONFIG, "tile_k=%d does not divide the K range of a split (%lld bytes)",
                        spec->kt, (long long)Ks);
    } else {
        spec = default_spec(c.dtype, c.scale, out, c.M, c.N, Ks, c.split_k);
        if (!spec)
            return fail(DGP_ERR_CONFIG, "no compiled kernel fits this shape");
    }
    plan->spec = spec;
    plan->tiles_m = (int)((c.M + spec->tm - 1) / spec->tm);
    plan->tiles_n = (int)((c.N + spec->tn - 1) / spec->tn);
    if (c.cfg && c.cfg->tile_m > 0) {
        plan->remap = c.cfg->xcd_remap;
        plan->group_m = c.cfg->group_m < 1 ? 1 : c.cfg->group_m;
    } else {
        plan->remap = spec->family == kTiled ? 1 : 0;
        plan->group_m = 8;
    }
    const int64_t grid = (int64_t)plan->tiles_m * plan->tiles_n * c.split_k;
    if (grid > INT32_MAX)
        return fail(DGP_ERR_SHAPE, "grid of %lld workgroups too large", (long long)grid);
    return ok();
}

dgp_status validate(const GemmCall &c, Plan *plan)
{
    if (!known_dtype(c.dtype))
        return fail(DGP_ERR_DTYPE, "dtype %d is not DGP_BF16, DGP_FP8_E4M3 or DGP_FP4_E2M1", c.dtype);
    if (c.M < 0 || c.N < 0 || c.K < 0)
        return fail(DGP_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld", (long long)c.M, (long long)c.N,
                    (long long)c.K);
    if (c.scale < DGP_SCALE_NONE || c.scale > DGP_SCALE_MX32)
        return fail(DGP_ERR_SCALE_MODE, "unknown scale mode %d", c.scale);
    if ((c.dtype == DGP_FP4_E2M1) != (c.scale == DGP_SCALE_MX32))
        return fail(DGP_ERR_SCALE_MODE, "DGP_FP4_E2M1 takes DGP_SCALE_MX32, and only it");
    if (c.dtype == DGP_BF16 && c.scale != DGP_SCALE_NONE)
        return fail(DGP_ERR_SCALE_MODE, "bf16 takes DGP_SCALE_NONE");
    if (c.dtype == DGP_FP8_E4M3 && (c.scale == DGP_SCALE_NONE || c.scale == DGP_SCALE_MX32))
        return fail(DGP_ERR_SCALE_MODE, "fp8 takes DGP_SCALE_TENSOR, DGP_SCALE_BLOCK128 or DGP_SCALE_MX128");
    if (c.split_k < 1)
        return fail(DGP_ERR_SPLITK, "split_k %d < 1", c.split_k);
    if (c.cfg) {
        if (c.cfg->preload_vmem < 0 || c.cfg->preload_dsrd < 0)
            return fail(DGP_ERR_CONFIG, "preload must be a pair of non-negative integers (got %d, %d)",
                        c.cfg->preload_vmem, c.cfg->preload_dsrd);
        if (c.cfg->xcd_remap != 0 && c.cfg->xcd_remap != 1)
            return fail(DGP_ERR_CONFIG, "xcd_remap must be 0 or 1");
        if (c.cfg->xcd_remap == 1 && c.cfg->group_m < 1)
            return fail(DGP_ERR_CONFIG, "group_m must be >= 1");
    }
    if (c.N % 16 != 0)
        return fail(DGP_ERR_SHAPE, "N=%lld is not a multiple of 16 (preshuffle block rows)", (long long)c.N);
    if (c.dtype == DGP_FP4_E2M1 && c.K % 2 != 0)
        return fail(DGP_ERR_SHAPE, "fp4 K=%lld is odd", (long long)c.K);
    const int64_t Kb = row_bytes(c.dtype, c.K);
    if (Kb % 128 != 0)
        return fail(DGP_ERR_SHAPE, "row bytes %lld (K=%lld) are not a multiple of 128", (long long)Kb, (long long)c.K);
    if (Kb > kMaxRowBytes)
        return fail(DGP_ERR_SHAPE, "K*element_bytes=%lld exceeds %lld", (long long)Kb, (long long)kMaxRowBytes);
    if (c.M > INT32_MAX / 2 || c.N > INT32_MAX / 2)
        return fail(DGP_ERR_SHAPE, "M or N too large");
    if (c.scale == DGP_SCALE_BLOCK128 && (c.K % 128 != 0 || c.N % 128 != 0))
        return fail(DGP_ERR_SHAPE, "blockscale needs K %% 128 == 0 and N %% 128 == 0 (K=%lld N=%lld)",
                    (long long)c.K, (long long)c.N);
    if (c.scale == DGP_SCALE_MX128 && c.K % 128 != 0)
        return fail(DGP_ERR_SHAPE, "mxfp8 needs K %% 128 == 0 (K=%lld)", (long long)c.K);
    if (c.K % c.split_k != 0)
        return fail(DGP_ERR_SPLITK, "split_k=%d does not divide K=%lld", c.split_k, (long long)c.K);
    const int64_t Ks = Kb / c.split_k;
    if (Ks % 128 != 0)
        return fail(DGP_ERR_SPLITK, "K range per split (%lld bytes) is not a multiple of 128", (long long)Ks);
    if ((c.scale == DGP_SCALE_BLOCK128 || c.scale == DGP_SCALE_MX128) && (c.K / c.split_k) % 128 != 0)
        return fail(DGP_ERR_SPLITK, "block scales need (K/split_k) %% 128 == 0");

    if (c.M == 0 || c.N == 0 || (c.select_only && c.K == 0)) {
        plan->spec = nullptr;
        return ok();
    }
    if (c.select_only)
        return select_kernel(c, Ks, plan);
    if (!c.C)
        return fail(DGP_ERR_NULL, "C is NULL");
    if (!aligned16(c.C))
        return fail(DGP_ERR_ALIGN, "C is not 16-byte aligned");
    if (c.K == 0) {
        plan->spec = nullptr;
        return ok();
    }
    if (!c.A || !c.Bs)
        return fail(DGP_ERR_NULL, "A or Bs is NULL");
    if (!aligned16(c.A) || !aligned16(c.Bs))
        return fail(DGP_ERR_ALIGN, "A and Bs must be 16-byte aligned");
    if (c.scale != DGP_SCALE_NONE) {
        if (!c.sA || !c.sB)
            return fail(DGP_ERR_NULL, "scale mode needs sA and sB");
        if (c.scale != DGP_SCALE_MX128 && (((uintptr_t)c.sA & 3u) || ((uintptr_t)c.sB & 3u)))
            return fail(DGP_ERR_ALIGN, "fp32 scales sA and sB must be 4-byte aligned");
    }
    if (c.split_k > 1) {
        const size_t need = dgp_splitk_workspace_bytes(c.M, c.N, c.split_k);
        if (c.lib_scratch) {
            if (need > kNoAllocScratchBytes)
                return fail(DGP_ERR_WORKSPACE,
                            "split_k*M*N*4 = %zu bytes exceeds the library's fixed scratch of %zu bytes "
                            "(DGP_NOALLOC_SCRATCH_BYTES); pass a workspace to dgp_gemm_preshuffle_splitk",
                            need, kNoAllocScratchBytes);
        } else {
            if (!c.ws)
                return fail(DGP_ERR_WORKSPACE, "split_k > 1 needs a workspace");
            if (!aligned16(c.ws))
                return fail(DGP_ERR_ALIGN, "workspace is not 16-byte aligned");
            if (c.ws_bytes < need)
                return fail(DGP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", c.ws_bytes, need);
        }
    }

    return select_kernel(c, Ks, plan);
}

dgp_status run_gemm(const GemmCall &c, hipStream_t stream)
{
    Plan plan{};
    dgp_status st = validate(c, &plan);
    if (st != DGP_OK)
        return st;
    if (c.M == 0 || c.N == 0)
        return ok();
    st = check_device_arch();
    if (st != DGP_OK)
        return st;
    if (c.K == 0)
        return hip_status(launch_splitk_reduce(nullptr, c.C, c.M, c.N, 0, stream), "zero fill");
    float *ws = c.ws;
    if (c.lib_scratch && c.split_k > 1) {
        st = hip_status(noalloc_scratch(&ws), "address of the library's split-K scratch");
        if (st != DGP_OK)
            return st;
    }

    GemmArgs a{};
    a.A = (const uint8_t *)c.A;
    a.Bs = (const uint8_t *)c.Bs;
    a.C = c.C;
    a.ws = ws;
    a.sA = c.sA;
    a.sB = c.sB;
    a.M = (int)c.M;
    a.N = (int)c.N;
    a.K = (int)c.K;
    a.Kb = (int)row_bytes(c.dtype, c.K);
    a.Ks = a.Kb / c.split_k;
    a.tiles_m = plan.tiles_m;
    a.tiles_n = plan.tiles_n;
    a.splits = c.split_k;
    a.remap = plan.remap;
    a.group_m = plan.group_m;
    const dim3 grid((unsigned)((int64_t)plan.tiles_m * plan.tiles_n * c.split_k));
    plan.spec->launch(a, grid, stream);
    st = hip_status(hipGetLastError(), "GEMM launch");
    if (st != DGP_OK || c.split_k == 1)
        return st;
    return hip_status(launch_splitk_reduce(ws, c.C, c.M, c.N, c.split_k, stream), "split-K reduce launch");
}

dgp_status shuffle(const void *src, void *dst, int64_t N, int64_t K, int dtype, void *stream, bool inverse)
{
    if (!known_dtype(dtype))
        return fail(DGP_ERR_DTYPE, "dtype %d is not DGP_BF16, DGP_FP8_E4M3 or DGP_FP4_E2M1", dtype);
    if (N < 0 || K < 0)
        return fail(DGP_ERR_SHAPE, "negative size N=%lld K=%lld", (long long)N, (long long)K);
    if (dtype == DGP_FP4_E2M1 && K % 2 != 0)
        return fail(DGP_ERR_SHAPE, "fp4 K=%lld is odd", (long long)K);
    const int64_t Kb = row_bytes(dtype, K);
    if (N % 16 != 0)
        return fail(DGP_ERR_SHAPE, "N=%lld is not a multiple of 16", (long long)N);
    if (Kb % 64 != 0)
        return fail(DGP_ERR_SHAPE, "K*element_bytes=%lld is not a multiple of 64", (long long)Kb);
    if (Kb >= (int64_t(1) << 27))
        return fail(DGP_ERR_SHAPE, "K*element_bytes=%lld too large", (long long)Kb);
    if (N / 16 > INT32_MAX)
        return fail(DGP_ERR_SHAPE, "N too large");
    if (N == 0 || K == 0)
        return ok();
    if (!src || !dst)
        return fail(DGP_ERR_NULL, "source or destination is NULL");
    if (!aligned16(src) || !aligned16(dst))
        return fail(DGP_ERR_ALIGN, "source and destination must be 16-byte aligned");
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst, n = (uintptr_t)(N * Kb);
    if (s < d + n && d < s + n)
        return fail(DGP_ERR_SHAPE, "source and destination overlap");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_preshuffle(src, dst, N, Kb, inverse, (hipStream_t)stream), "preshuffle launch");
}

}  // namespace

// ====================================================================== ABI

extern "C" {

dgp_status dgp_preshuffle_b(const void *B, void *Bs, int64_t N, int64_t K, int dtype, void *stream)
{
    return shuffle(B, Bs, N, K, dtype, stream, false);
}

dgp_status dgp_unshuffle_b(const void *Bs, void *B, int64_t N, int64_t K, int dtype, void *stream)
{
    return shuffle(Bs, B, N, K, dtype, stream, true);
}

dgp_status dgp_gemm_preshuffle(const void *A, const void *Bs, void *C, int64_t M, int64_t N, int64_t K,
                               int dtype, int scale_mode, const void *sA, const void *sB,
                               const dgp_config *cfg, void *stream)
{
    GemmCall c{A, Bs, C, M, N, K, dtype, scale_mode, sA, sB, 1, nullptr, 0, cfg};
    return run_gemm(c, (hipStream_t)stream);
}

size_t dgp_splitk_workspace_bytes(int64_t M, int64_t N, int split_k)
{
    if (split_k <= 1 || M <= 0 || N <= 0)
        return 0;
    return (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

dgp_status dgp_gemm_preshuffle_splitk(const void *A, const void *Bs, void *C, int64_t M, int64_t N,
                                      int64_t K, int dtype, int scale_mode, const void *sA,
                                      const void *sB, int split_k, float *ws, size_t ws_bytes,
                                      const dgp_config *cfg, void *stream)
{
    GemmCall c{A, Bs, C, M, N, K, dtype, scale_mode, sA, sB, split_k, ws, ws_bytes, cfg};
    return run_gemm(c, (hipStream_t)stream);
}

dgp_status dgp_gemm_preshuffle_splitk_noalloc(const void *A, const void *Bs, void *C, int64_t M, int64_t N,
                                              int64_t K, int dtype, int scale_mode, const void *sA,
                                              const void *sB, int split_k, const dgp_config *cfg, void *stream)
{
    GemmCall c{A, Bs, C, M, N, K, dtype, scale_mode, sA, sB, split_k, nullptr, 0, cfg};
    c.lib_scratch = true;
    return run_gemm(c, (hipStream_t)stream);
}

dgp_status dgp_check_arch(const char *name)
{
    if (!name)
        return DGP_ERR_ARCH;
    // "gfx950" optionally followed by ":feature" suffixes.
    if (strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':'))
        return DGP_OK;
    return DGP_ERR_ARCH;
}

const char *dgp_status_string(int s)
{
    switch (s) {
    case DGP_OK: return "DGP_OK";
    case DGP_ERR_NULL: return "DGP_ERR_NULL";
    case DGP_ERR_SHAPE: return "DGP_ERR_SHAPE";
    case DGP_ERR_ALIGN: return "DGP_ERR_ALIGN";
    case DGP_ERR_DTYPE: return "DGP_ERR_DTYPE";
    case DGP_ERR_SCALE_MODE: return "DGP_ERR_SCALE_MODE";
    case DGP_ERR_SPLITK: return "DGP_ERR_SPLITK";
    case DGP_ERR_WORKSPACE: return "DGP_ERR_WORKSPACE";
    case DGP_ERR_CONFIG: return "DGP_ERR_CONFIG";
    case DGP_ERR_ARCH: return "DGP_ERR_ARCH";
    case DGP_ERR_HIP: return "DGP_ERR_HIP";
    default: return "DGP_ERR_UNKNOWN";
    }
}

const char *dgp_last_error(void) { return g_err; }

// ------------------------------------------------------------ diagnostics

dgp_status dgp_tile_of_workgroup(int64_t wg, int64_t tiles_m, int64_t tiles_n, int64_t splits, int xcd_remap,
                                 int group_m, int64_t out[3])
{
    if (!out)
        return fail(DGP_ERR_NULL, "out is NULL");
    if (tiles_m < 1 || tiles_n < 1 || splits < 1 || wg < 0 || wg >= tiles_m * tiles_n * splits ||
        (xcd_remap != 0 && xcd_remap != 1) || tiles_m * tiles_n * splits > INT32_MAX)
        return fail(DGP_ERR_SHAPE, "bad tile-map arguments");
    const TileCoord c = tile_of_workgroup<int64_t>(wg, tiles_m, tiles_n, splits, xcd_remap, group_m);
    out[0] = c.tm;
    out[1] = c.tn;
    out[2] = c.s;
    return ok();
}

dgp_status dgp_tile_map(int64_t tiles_m, int64_t tiles_n, int64_t splits, int xcd_remap, int group_m,
                        int64_t *out, int64_t out_len)
{
    if (!out)
        return fail(DGP_ERR_NULL, "out is NULL");
    if (tiles_m < 1 || tiles_n < 1 || splits < 1 || (xcd_remap != 0 && xcd_remap != 1) ||
        tiles_m * tiles_n * splits > INT32_MAX)
        return fail(DGP_ERR_SHAPE, "bad tile-map arguments");
    const int64_t total = tiles_m * tiles_n * splits;
    if (out_len < 3 * total)
        return fail(DGP_ERR_SHAPE, "out holds %lld values, the grid needs %lld", (long long)out_len,
                    (long long)(3 * total));
    for (int64_t wg = 0; wg < total; ++wg) {
        const TileCoord c = tile_of_workgroup<int64_t>(wg, tiles_m, tiles_n, splits, xcd_remap, group_m);
        out[3 * wg] = c.tm;
        out[3 * wg + 1] = c.tn;
        out[3 * wg + 2] = c.s;
    }
    return ok();
}

int dgp_lds_poison(void)
{
    return dgp::kLdsPoison ? 1 : 0;
}

int dgp_kernel_count(void)
{
    int n = 0;
    kernel_table(&n);
    return n;
}

dgp_status dgp_kernel_info(int index, dgp_config *cfg, int *dtype, int *scale_mode, int *split_out)
{
    int n = 0;
    const KernelSpec *t = kernel_table(&n);
    if (index < 0 || index >= n)
        return fail(DGP_ERR_SHAPE, "kernel index %d out of range [0, %d)", index, n);
    if (!cfg || !dtype || !scale_mode || !split_out)
        return fail(DGP_ERR_NULL, "NULL output");
    const KernelSpec &k = t[index];
    cfg->tile_m = k.tm;
    cfg->tile_n = k.tn;
    cfg->tile_k = k.family == kTiled ? k.kt : 0;
    cfg->xcd_remap = k.family == kTiled ? 1 : 0;
    cfg->group_m = 8;
    cfg->preload_vmem = k.pv;
    cfg->preload_dsrd = k.pd;
    cfg->waves_m = k.family == kTiled ? k.p0 : k.waves;
    cfg->prefetch = k.depth;
    cfg->schedule = k.sched;
    cfg->a_layout = k.family == kTiled ? k.lay + 1 : 0;
    cfg->a_copy = k.family == kTiled ? k.copy + 1 : 0;
    *dtype = k.dtype;
    *scale_mode = k.scale;
    *split_out = k.out == kOutPartial ? 1 : 0;
    return ok();
}

dgp_status dgp_select_kernel(int64_t M, int64_t N, int64_t K, int dtype, int scale_mode, int split_k,
                             const dgp_config *cfg, int *index)
{
    if (!index)
        return fail(DGP_ERR_NULL, "NULL index");
    GemmCall c{nullptr, nullptr, nullptr, M, N, K, dtype, scale_mode, nullptr, nullptr, split_k, nullptr, 0, cfg};
    c.select_only = true;
    Plan plan{};
    const dgp_status st = validate(c, &plan);
    if (st != DGP_OK)
        return st;
    *index = -1;
    if (plan.spec) {
        int n = 0;
        *index = (int)(plan.spec - kernel_table(&n));
    }
    return ok();
}

dgp_status dgp_probe_mfma_layout(int which, const void *a, const void *b, float *out, void *stream)
{
    if (which != 0 && which != 1)
        return fail(DGP_ERR_CONFIG, "which must be 0 or 1");
    if (!a || !b || !out)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(a) || !aligned16(b) || !aligned16(out))
        return fail(DGP_ERR_ALIGN, "buffers must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_mfma(which, a, b, out, (hipStream_t)stream), "probe launch");
}

dgp_status dgp_probe_mfma_scaled(int which, const void *a, const void *b, const void *sa, const void *sb,
                                 float *out, void *stream)
{
    if (which != 0 && which != 1)
        return fail(DGP_ERR_CONFIG, "which must be 0 or 1");
    if (!a || !b || !sa || !sb || !out)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(a) || !aligned16(b) || !aligned16(out))
        return fail(DGP_ERR_ALIGN, "a, b and out must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_mfma_scaled(which, a, b, sa, sb, out, (hipStream_t)stream), "probe launch");
}

dgp_status dgp_probe_lds_dma(const void *src, const int32_t *perm, void *dst, void *stream)
{
    if (!src || !perm || !dst)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(src) || !aligned16(dst))
        return fail(DGP_ERR_ALIGN, "buffers must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_lds_dma(src, perm, dst, (hipStream_t)stream), "probe launch");
}

dgp_status dgp_probe_lds_dma_narrow(int width, const void *src, const int32_t *perm, void *dst, void *stream)
{
    if (width != 1 && width != 2 && width != 4)
        return fail(DGP_ERR_CONFIG, "width must be 1, 2 or 4 (got %d)", width);
    if (!src || !perm || !dst)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(src) || !aligned16(dst))
        return fail(DGP_ERR_ALIGN, "buffers must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_lds_dma_narrow(width, src, perm, dst, (hipStream_t)stream), "probe launch");
}

dgp_status dgp_probe_copy(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (bytes < 0 || bytes % 16 != 0)
        return fail(DGP_ERR_SHAPE, "bytes must be a non-negative multiple of 16");
    if (bytes == 0)
        return ok();
    if (!src || !dst)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(src) || !aligned16(dst))
        return fail(DGP_ERR_ALIGN, "buffers must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_copy(src, dst, bytes, (hipStream_t)stream), "probe launch");
}

dgp_status dgp_probe_stream_read(const void *src, int64_t bytes, int blocks, uint32_t *sink, void *stream)
{
    if (bytes < 0 || bytes % 16 != 0)
        return fail(DGP_ERR_SHAPE, "bytes must be a non-negative multiple of 16");
    if (blocks < 1 || blocks > 65536)
        return fail(DGP_ERR_SHAPE, "blocks must be in [1, 65536] (got %d)", blocks);
    if (bytes == 0)
        return ok();
    if (!src || !sink)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(src))
        return fail(DGP_ERR_ALIGN, "source must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_stream_read(src, bytes, blocks, sink, (hipStream_t)stream), "probe launch");
}

dgp_status dgp_probe_mfma_peak(int which, int rounds, int blocks, const void *operands, uint32_t *sink,
                               void *stream)
{
    if (which < 0 || which > 2)
        return fail(DGP_ERR_CONFIG, "which must be 0, 1 or 2");
    if (rounds < 1 || rounds > (1 << 24) || blocks < 1 || blocks > 65536)
        return fail(DGP_ERR_SHAPE, "rounds must be in [1, 2^24] and blocks in [1, 65536]");
    if (!operands || !sink)
        return fail(DGP_ERR_NULL, "NULL buffer");
    if (!aligned16(operands))
        return fail(DGP_ERR_ALIGN, "operands must be 16-byte aligned");
    dgp_status st = check_device_arch();
    if (st != DGP_OK)
        return st;
    return hip_status(launch_probe_mfma_peak(which, rounds, blocks, operands, sink, (hipStream_t)stream), "probe launch");
}

}  // extern "C"
