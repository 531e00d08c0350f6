"""Host-side tests of the C-ABI library: it loads, exports every symbol the
headers declare, and rejects every invalid argument with the documented
status before making any HIP call (only invalid calls are made here, so no
device is touched).  Also: the workgroup -> tile map is a bijection, and the
product path shares nothing with the oracle."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

OK, NULL, SHAPE, ALIGN, DTYPE, SCALE, SPLITK, WS, CONFIG, ARCH, HIP = range(11)
BF16, FP8, FP4 = 0, 1, 2
NONE, TENSOR, BLOCK, MX, MX32 = 0, 1, 2, 3, 4
P = 0x10000          # aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def dgp():
    import dense_gemm_packer_amd as d
    if not os.path.exists(d.LIB_PATH):
        from dense_gemm_packer_amd import build
        build.build()
    return d


@pytest.fixture(scope="module")
def L(dgp):
    return dgp.lib()


def declared_symbols():
    names = set()
    for h in os.listdir(INCLUDE):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(dgp_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol(dgp, L):
    names = declared_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(dgp.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", dgp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dgp_\w+)", out))
    assert names <= exported


def test_lds_poison_build_exports_the_same_symbols(dgp, L):
    """The debug build is the same library with the LDS poison compiled in:
    every declared symbol, the same kernel table, and dgp_lds_poison() = 1
    (0 in the release build)."""
    names = declared_symbols()
    out = subprocess.run(["nm", "-D", "--defined-only", dgp.LDS_POISON_LIB_PATH], capture_output=True,
                         text=True).stdout
    assert names <= set(re.findall(r"\bT (dgp_\w+)", out))
    assert L.dgp_lds_poison() == 0
    release = [(c.tile_m, c.tile_n, c.waves_m, c.prefetch, c.schedule, dt, sm, so)
               for c, dt, sm, so in dgp.kernels()]
    with dgp.lds_poison_build() as P:
        assert P.dgp_lds_poison() == 1 and dgp.lib() is P
        assert P.dgp_kernel_count() == L.dgp_kernel_count() == len(release)
        for i, (tm, tn, wm, pf, sch, dt, sm, so) in enumerate(release):
            cfg, d, m, o = dgp.Config(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
            assert P.dgp_kernel_info(i, ctypes.byref(cfg), ctypes.byref(d), ctypes.byref(m), ctypes.byref(o)) == OK
            assert (cfg.tile_m, cfg.tile_n, cfg.waves_m, cfg.prefetch, cfg.schedule, d.value, m.value,
                    bool(o.value)) == (tm, tn, wm, pf, sch, dt, sm, bool(so))
    assert dgp.lib() is L


def test_check_arch(L):
    assert L.dgp_check_arch(b"gfx950") == OK
    assert L.dgp_check_arch(b"gfx950:sramecc+:xnack-") == OK
    for bad in (b"gfx942", b"gfx942:sramecc+:xnack-", b"gfx9500", b"gfx90a", b"", None):
        assert L.dgp_check_arch(bad) == ARCH


def test_status_strings(L):
    names = ["DGP_OK", "DGP_ERR_NULL", "DGP_ERR_SHAPE", "DGP_ERR_ALIGN", "DGP_ERR_DTYPE",
             "DGP_ERR_SCALE_MODE", "DGP_ERR_SPLITK", "DGP_ERR_WORKSPACE", "DGP_ERR_CONFIG",
             "DGP_ERR_ARCH", "DGP_ERR_HIP"]
    for i, n in enumerate(names):
        assert L.dgp_status_string(i).decode() == n
    assert L.dgp_status_string(99).decode() == "DGP_ERR_UNKNOWN"


def gemm(L, A=P, Bs=P, C=P, M=16, N=128, K=256, dtype=FP8, scale=TENSOR, sA=P, sB=P, cfg=None):
    return L.dgp_gemm_preshuffle(A, Bs, C, M, N, K, dtype, scale, sA, sB, cfg, None)


def splitk(L, split, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(A=P, Bs=P, C=P, M=16, N=128, K=1024, dtype=FP8, scale=TENSOR, sA=P, sB=P)
    a.update(kw)
    return L.dgp_gemm_preshuffle_splitk(a["A"], a["Bs"], a["C"], a["M"], a["N"], a["K"], a["dtype"],
                                        a["scale"], a["sA"], a["sB"], split, ws, ws_bytes, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), DTYPE),
    (dict(M=-1), SHAPE), (dict(N=-16), SHAPE), (dict(K=-128), SHAPE),
    (dict(dtype=BF16, scale=TENSOR), SCALE), (dict(dtype=FP8, scale=NONE), SCALE), (dict(scale=5), SCALE),
    (dict(N=24), SHAPE),                                  # N % 16
    (dict(dtype=BF16, scale=NONE, K=32), SHAPE),          # K*2 bytes % 128
    (dict(K=192), SHAPE),                                 # fp8 K % 128
    (dict(scale=BLOCK, N=64), SHAPE),                     # blockscale N % 128
    (dict(dtype=BF16, scale=MX, K=64), SCALE),            # mxfp8 is fp8 only
    (dict(scale=MX, sA=0), NULL),                          # E8M0 bytes need pointers too
    (dict(dtype=FP4, scale=MX), SCALE),                    # fp4 takes only its 32-block scales
    (dict(dtype=FP8, scale=MX32), SCALE),                  # and they only fp4
    (dict(dtype=FP4, scale=MX32, K=128), SHAPE),           # fp4 rows of 64 bytes
    (dict(dtype=FP4, scale=MX32, K=255), SHAPE),           # odd K
    (dict(C=0), NULL), (dict(A=0), NULL), (dict(Bs=0), NULL),
    (dict(sA=0), NULL), (dict(sB=0), NULL),
    (dict(A=P + 8), ALIGN), (dict(Bs=P + 4), ALIGN), (dict(C=P + 2), ALIGN), (dict(sA=P + 1), ALIGN),
])
def test_gemm_rejects(L, kw, status):
    assert gemm(L, **kw) == status
    assert L.dgp_last_error().decode() != ""


def test_mx128_accepts_byte_aligned_scales_and_any_n16(dgp):
    # E8M0 scales are bytes (no 4-byte alignment) and B's are per column, so
    # N need only be a multiple of 16; split ranges must be whole 128-K blocks.
    assert dgp.select_kernel(16, 48, 1024, dgp.FP8_E4M3, dgp.SCALE_MX128) >= 0
    with pytest.raises(dgp.DgpError) as e:
        dgp.select_kernel(16, 48, 1024, dgp.FP8_E4M3, dgp.SCALE_MX128, 16)   # 64-K ranges
    assert e.value.name == "DGP_ERR_SPLITK"


def test_empty_problems_are_noops(L):
    assert gemm(L, M=0, A=0, Bs=0, C=0) == OK
    assert gemm(L, N=0, A=0, Bs=0, C=0) == OK


def test_config_validation(dgp, L):
    Cfg = dgp.Config
    bad = [Cfg(256, 256, 128, 1, 4, -1, 0), Cfg(256, 256, 128, 1, 4, 0, -3), Cfg(256, 256, 128, 2, 4, 0, 0),
           Cfg(256, 256, 128, 1, 0, 0, 0), Cfg(100, 100, 128, 1, 4, 0, 0), Cfg(256, 256, 64, 1, 4, 0, 0),
           Cfg(256, 256, 128, 1, 4, 3, 3)]
    for c in bad:
        assert gemm(L, M=4096, N=4096, K=8192, cfg=ctypes.byref(c)) == CONFIG, (c.tile_m, c.preload_vmem)


def test_splitk_validation(L):
    assert splitk(L, 0) == SPLITK
    assert splitk(L, 3) == SPLITK                          # 3 does not divide K=1024
    assert splitk(L, 16) == SPLITK                         # 64-byte K range per split
    assert splitk(L, 2, ws=0) == WS
    assert splitk(L, 2, ws_bytes=2 * 16 * 128 * 4 - 1) == WS
    assert splitk(L, 2, ws=P + 4) == ALIGN
    assert L.dgp_splitk_workspace_bytes(16, 16384, 8) == 8 * 16 * 16384 * 4
    assert L.dgp_splitk_workspace_bytes(16, 16384, 1) == 0
    assert L.dgp_splitk_workspace_bytes(0, 16384, 4) == 0


@pytest.mark.parametrize("args,status", [
    ((P, P + 4096 * 64, 24, 64, FP8), SHAPE),              # N % 16
    ((P, P + 4096 * 64, 16, 48, FP8), SHAPE),              # K bytes % 64
    ((P, P + 4096 * 64, 16, 16, BF16), SHAPE),             # 32 bytes
    ((P, P + 512, 16, 64, FP8), SHAPE),                    # overlap
    ((0, P, 16, 64, FP8), NULL), ((P, 0, 16, 64, FP8), NULL),
    ((P + 8, P + 65536, 16, 64, FP8), ALIGN),
    ((P, P + 65536, 16, 64, 3), DTYPE),
    ((P, P + 65536, -16, 64, FP8), SHAPE),
])
def test_preshuffle_rejects(L, args, status):
    assert L.dgp_preshuffle_b(*args, None) == status
    assert L.dgp_unshuffle_b(*args, None) == status


def test_preshuffle_empty_is_noop(L):
    assert L.dgp_preshuffle_b(0, 0, 0, 64, FP8, None) == OK
    assert L.dgp_preshuffle_b(0, 0, 16, 0, FP8, None) == OK


def test_probe_validation(L):
    assert L.dgp_probe_mfma_layout(2, P, P, P, None) == CONFIG
    assert L.dgp_probe_mfma_layout(0, 0, P, P, None) == NULL
    assert L.dgp_probe_copy(P, P, 17, None) == SHAPE
    assert L.dgp_probe_copy(P, P, 0, None) == OK
    assert L.dgp_probe_stream_read(P, 4088, 512, P, None) == SHAPE     # not whole 16-byte units
    assert L.dgp_probe_stream_read(P, 4096, 0, P, None) == SHAPE
    assert L.dgp_probe_stream_read(P, 4096, 65537, P, None) == SHAPE
    assert L.dgp_probe_stream_read(0, 4096, 512, P, None) == NULL
    assert L.dgp_probe_stream_read(P, 0, 512, P, None) == OK
    assert L.dgp_probe_mfma_peak(3, 1, 1, P, P, None) == CONFIG
    assert L.dgp_probe_mfma_peak(-1, 1, 1, P, P, None) == CONFIG
    assert L.dgp_probe_mfma_peak(0, 0, 1, P, P, None) == SHAPE
    assert L.dgp_probe_mfma_peak(1, 1, 0, P, P, None) == SHAPE
    assert L.dgp_probe_mfma_peak(0, 1, 65537, P, P, None) == SHAPE
    assert L.dgp_probe_mfma_peak(0, 1, 1, 0, P, None) == NULL
    assert L.dgp_probe_mfma_peak(0, 1, 1, P, 0, None) == NULL
    assert L.dgp_probe_mfma_peak(0, 1, 1, P + 8, P, None) == ALIGN
    assert L.dgp_probe_lds_dma_narrow(3, P, P, P, None) == CONFIG
    assert L.dgp_probe_lds_dma_narrow(16, P, P, P, None) == CONFIG
    assert L.dgp_probe_lds_dma_narrow(1, 0, P, P, None) == NULL
    assert L.dgp_probe_lds_dma_narrow(4, P, P, P + 4, None) == ALIGN


@pytest.mark.parametrize("remap,group_m", [(0, 1), (1, 1), (1, 4), (1, 8)])
def test_tile_map_is_a_bijection(dgp, remap, group_m):
    for tm in (1, 2, 3, 7, 16):
        for tn in (1, 5, 16):
            for sp in (1, 2, 3, 8):
                W = tm * tn * sp
                seen = {dgp.tile_of_workgroup(w, tm, tn, sp, remap, group_m) for w in range(W)}
                assert len(seen) == W
                assert all(0 <= a < tm and 0 <= b < tn and 0 <= c < sp for a, b, c in seen)


def _grid_shapes(W):
    """A few ways to factor a grid of W workgroups as tiles_m x tiles_n x splits."""
    def near_square(n):
        d = max(x for x in range(1, math.isqrt(n) + 1) if n % x == 0)
        return n // d, d
    shapes = {(W, 1, 1), (1, W, 1), (*near_square(W), 1)}
    if W % 2 == 0:
        shapes.add((*near_square(W // 2), 2))
    return shapes


@pytest.mark.parametrize("remap,group_m", [(0, 1), (1, 1), (1, 4), (1, 8)])
def test_tile_map_bijective_over_grid_sizes(dgp, remap, group_m):
    """Every grid size W = 1..4096 and every 97th size up to 65536 (and 65536
    itself), each factored several ways: the workgroup -> (tile_m, tile_n,
    split) map of the library hits every tile of every split exactly once."""
    import numpy as np
    sizes = list(range(1, 4097)) + list(range(4097, 65536, 97)) + [65536]
    for W in sizes:
        for tm, tn, sp in _grid_shapes(W):
            assert tm * tn * sp == W
            c = dgp.tile_map(tm, tn, sp, remap, group_m)
            assert c[:, 0].min() >= 0 and c[:, 0].max() < tm
            assert c[:, 1].min() >= 0 and c[:, 1].max() < tn
            assert c[:, 2].min() >= 0 and c[:, 2].max() < sp
            lin = (c[:, 2] * tm + c[:, 0]) * tn + c[:, 1]
            assert np.all(np.bincount(lin, minlength=W) == 1), (W, tm, tn, sp)


def test_tile_map_agrees_with_the_single_workgroup_mirror(dgp):
    for tm, tn, sp, remap, gm in ((7, 5, 3, 1, 4), (16, 16, 1, 1, 8), (3, 9, 2, 0, 1), (9, 33, 1, 1, 4)):
        c = dgp.tile_map(tm, tn, sp, remap, gm)
        for w in range(tm * tn * sp):
            assert tuple(c[w]) == dgp.tile_of_workgroup(w, tm, tn, sp, remap, gm)


def test_tile_map_rejects_short_output(dgp, L):
    import numpy as np
    out = np.zeros(3 * 11, dtype=np.int64)
    assert L.dgp_tile_map(3, 4, 1, 1, 8, out.ctypes.data, out.size) == 2        # DGP_ERR_SHAPE
    assert L.dgp_tile_map(3, 4, 1, 1, 8, None, 36) == 1                         # DGP_ERR_NULL
    assert L.dgp_tile_map(3, 4, 1, 2, 8, out.ctypes.data, out.size) == 2        # remap flag not 0/1


def test_tile_map_remap_groups_xcd_neighbours(dgp):
    # 16 x 16 tiles, group_m 4: the 32 workgroups the hardware deals to XCD 0
    # (ids 0, 8, 16, ...) cover a 4 x 8 block of tiles.
    tiles = {dgp.tile_of_workgroup(w, 16, 16, 1, 1, 4)[:2] for w in range(0, 256, 8)}
    assert {t[0] for t in tiles} == {0, 1, 2, 3} and {t[1] for t in tiles} == set(range(8))
    # without remap the same ids are a plain raster
    assert dgp.tile_of_workgroup(17, 16, 16, 1, 0, 4) == (1, 1, 0)


def test_kernel_table(dgp, L):
    ks = dgp.kernels()
    assert len(ks) == L.dgp_kernel_count() > 0
    seen = set()
    for cfg, dt, sm, split_out in ks:
        key = (cfg.tile_m, cfg.tile_n, cfg.tile_k, cfg.waves_m, cfg.prefetch, cfg.preload_vmem,
               cfg.preload_dsrd, cfg.schedule, cfg.a_layout, cfg.a_copy, dt, sm, split_out)
        assert key not in seen
        seen.add(key)
        assert (dt, sm) in ((0, 0), (1, 1), (1, 2), (1, 3), (2, 4))
        if cfg.tile_m > 16:
            # the A-tile granularity rule: whole 16-byte loads per thread
            assert (cfg.tile_m * cfg.tile_k) % 1024 == 0 and cfg.prefetch >= 1
    with pytest.raises(dgp.DgpError):
        import ctypes
        c = dgp.Config()
        i = ctypes.c_int()
        dgp._check(L.dgp_kernel_info(len(ks), ctypes.byref(c), ctypes.byref(i), ctypes.byref(i),
                                     ctypes.byref(i)))


def test_every_kernel_is_selected_by_its_reported_config(dgp):
    # The configuration dgp_kernel_info reports must select exactly that
    # kernel, so iterating the table really runs every compiled kernel.
    for i, (cfg, dt, sm, split_out) in enumerate(dgp.kernels()):
        M = 37 if cfg.tile_m == 16 else 2 * cfg.tile_m + 44
        N = 384 if cfg.tile_m == 16 else 2 * cfg.tile_n + 128
        K = 1024 if dt == dgp.FP8_E4M3 else 512
        assert dgp.select_kernel(M, N, K, dt, sm, 2 if split_out else 1, cfg) == i, dgp.describe_kernel(i)
        assert dgp.describe_kernel(i)


def _pick(dgp, M, N, split, dt, sm):
    """The built-in choice as 'k<tile_n>' (K-split tiles, 8 waves; 'K<tile_n>' with 16) or
    's<tile_n>' (streaming)."""
    c = dgp.kernels()[dgp.select_kernel(M, N, 7168, dt, sm, split)][0]
    if c.tile_m == 1:   # one-row VALU tile
        return f"w{c.tile_n}"
    if c.tile_m != 16:
        return f"t{c.tile_m}x{c.tile_n}"
    return {8: "k", 16: "K"}.get(c.waves_m, "s") + str(c.tile_n)


def test_default_selection(dgp):
    # Headline shapes take a 256x256 tile; empty calls launch nothing.
    for dt, sm in ((dgp.BF16, dgp.SCALE_NONE), (dgp.FP8_E4M3, dgp.SCALE_TENSOR)):
        cfg = dgp.kernels()[dgp.select_kernel(4096, 4096, 8192, dt, sm)][0]
        # the one-wave-per-SIMD tile with swizzled A rows
        assert (cfg.tile_m, cfg.tile_n, cfg.schedule, cfg.a_layout) == (256, 256, 4, 2)
    # blockscale, mxfp8 and mxfp4: the tiled kernels above decode-sized M
    # (the MX modes on the one-wave-per-SIMD tile, blockscale on the 8-wave
    # tile), the 16-row tiles at it
    for dt, sm in ((dgp.FP8_E4M3, dgp.SCALE_BLOCK128), (dgp.FP8_E4M3, dgp.SCALE_MX128),
                   (dgp.FP4_E2M1, dgp.SCALE_MX32)):
        i = dgp.select_kernel(4096, 4096, 7168, dt, sm)
        assert (dgp.kernels()[i][0].tile_m, dgp.kernels()[i][0].tile_n, dgp.kernels()[i][2]) == (256, 256, sm)
        assert dgp.kernels()[i][0].schedule == (1 if sm == dgp.SCALE_BLOCK128 else 4)
        i = dgp.select_kernel(300, 1024, 7168, dt, sm, 2)
        assert (dgp.kernels()[i][0].tile_m, dgp.kernels()[i][3]) == (128, True)
        assert dgp.kernels()[dgp.select_kernel(32, 16384, 7168, dt, sm)][0].tile_m == 16
    # Decode-sized M, K = 7168: the per-shape table (M/N/split -> tile), from
    # cold sweeps of every 16-row tile.
    want = {
        "tensor": "16/16384/1:k32 16/16384/2:k32 16/8192/1:k32 16/4096/1:k16 16/4096/4:k32 16/2048/1:k8 "
                  "16/2048/2:k16 16/2048/8:k32 4/16384/1:k16 1/16384/1:w16 1/8192/1:w16 1/2048/1:w8 1/16384/2:w16 "
                  "1/2048/2:w16 4/16384/2:k32 4/4096/4:k32 4/16384/4:s64 2/2048/1:k8",
        "bf16": "16/16384/1:K64 32/16384/1:K64 16/16384/2:k64 16/8192/1:k32 16/8192/2:k64 16/4096/2:k32 16/2048/8:k64 4/16384/1:k16 "
                "1/16384/1:w16 1/2048/1:w8 1/16384/2:w16 2/2048/1:k8 4/16384/2:k16 4/8192/4:k32",
        "mx32": "16/16384/1:k64 16/16384/2:s64 16/8192/1:K32 16/8192/2:k64 16/4096/2:k32 16/4096/4:k64 "
                "16/2048/4:k32 16/2048/2:k16 4/16384/1:k16 4/8192/1:K32 1/16384/1:k16 1/16384/2:k32 1/2048/1:K16 "
                "4/16384/4:s64 16/2048/1:K8 16/4096/1:K16 4/4096/1:K16 1/8192/1:K32",
        "block128": "16/16384/1:k64 16/8192/1:k32 16/4096/4:k64 16/2048/4:k32 4/2048/4:k32 1/16384/1:k32 "
                    "1/8192/1:k32 16/16384/4:s64 16/8192/4:s64 16/16384/2:k64",
        "mx128": "16/16384/1:k64 16/8192/1:k32 16/2048/8:k64 4/8192/1:k32 1/16384/1:k32 1/8192/1:k32 "
                 "16/16384/2:k32 1/16384/4:s64 16/8192/2:k32 4/16384/2:k32 16/16384/4:s64",
    }
    modes = {"tensor": (dgp.FP8_E4M3, dgp.SCALE_TENSOR), "bf16": (dgp.BF16, dgp.SCALE_NONE),
             "mx32": (dgp.FP4_E2M1, dgp.SCALE_MX32), "block128": (dgp.FP8_E4M3, dgp.SCALE_BLOCK128),
             "mx128": (dgp.FP8_E4M3, dgp.SCALE_MX128)}
    for mode, table in want.items():
        dt, sm = modes[mode]
        for entry in table.split():
            shape, tile = entry.split(":")
            M, N, split = (int(x) for x in shape.split("/"))
            assert _pick(dgp, M, N, split, dt, sm) == tile, (mode, shape)
    # Small grids above 32 rows: the 16-row K-split tile (C1 = 128 x 256 x 256), until the 128 x 128
    # grid has 64 tiles, the weight passes 8 MiB, M passes 256 or the call splits K
    for M, N, K, split, want in ((128, 256, 256, 1, 16), (256, 2048, 2048, 1, 16), (256, 4096, 2048, 1, 128),
                                 (128, 4096, 4096, 1, 128), (300, 256, 256, 1, 128), (128, 256, 256, 2, 128)):
        i = dgp.select_kernel(M, N, K, dgp.BF16, dgp.SCALE_NONE, split)
        assert dgp.kernels()[i][0].tile_m == want, (M, N, K, split)
    # Larger M: the tile whose grid needs the fewest weighted rounds over 256 CUs
    for M, N, K, sm, want in ((4096, 4096, 8192, dgp.SCALE_NONE, (256, 256)), (3072, 3072, 8192, dgp.SCALE_NONE, (256, 256)),
                              (2048, 4096, 8192, dgp.SCALE_NONE, (128, 256)), (2048, 2048, 8192, dgp.SCALE_TENSOR, (128, 128)),
                              (768, 16384, 4096, dgp.SCALE_NONE, (256, 256)), (1536, 1536, 8192, dgp.SCALE_TENSOR, (128, 128)),
                              # a lone bf16 128x256 tile one wave per SIMD beats a 128x128 round
                              (2048, 2048, 8192, dgp.SCALE_NONE, (128, 256)), (1536, 1536, 8192, dgp.SCALE_NONE, (128, 256)),
                              (2048, 4096, 8192, dgp.SCALE_BLOCK128, (128, 128)), (3072, 3072, 8192, dgp.SCALE_BLOCK128, (256, 256)),
                              # two 256x256 rounds against three 128x256 tiles on the busiest CU, two at once
                              (4096, 6144, 8192, dgp.SCALE_NONE, (128, 256)), (6144, 4096, 8192, dgp.SCALE_TENSOR, (128, 256)),
                              (4096, 5120, 8192, dgp.SCALE_NONE, (128, 256)), (3072, 4096, 8192, dgp.SCALE_TENSOR, (256, 256)),
                              (4096, 6144, 8192, dgp.SCALE_BLOCK128, (256, 256))):
        dt = dgp.BF16 if sm == dgp.SCALE_NONE else dgp.FP8_E4M3
        c = dgp.kernels()[dgp.select_kernel(M, N, K, dt, sm)][0]
        assert (c.tile_m, c.tile_n) == want, (M, N, K, sm)
    # bf16 and per-tensor fp8 take the 128 x 256 tile in its one-wave-per-SIMD form, split-K
    # partials included
    for dt, sm in ((dgp.BF16, dgp.SCALE_NONE), (dgp.FP8_E4M3, dgp.SCALE_TENSOR)):
        for M, split in ((2048, 1), (1024, 2)):
            c, _, _, so = dgp.kernels()[dgp.select_kernel(M, 4096, 8192, dt, sm, split)]
            assert (c.tile_m, c.tile_n, c.schedule, bool(so)) == (128, 256, 4, split > 1), (dt, M, split)
    assert dgp.select_kernel(0, 4096, 8192, dgp.BF16, dgp.SCALE_NONE) == -1
    assert dgp.select_kernel(16, 4096, 0, dgp.BF16, dgp.SCALE_NONE) == -1


def test_schedule_validation(dgp):
    base = dict(tile_m=256, tile_n=256, tile_k=128, xcd_remap=1, group_m=8)
    for sched in (1, 2, 3, 4):
        i = dgp.select_kernel(1024, 1024, 1024, dgp.BF16, dgp.SCALE_NONE, 1, dgp.Config(**base, schedule=sched))
        assert dgp.kernels()[i][0].schedule == sched
    for lay in (1, 2):
        i = dgp.select_kernel(1024, 1024, 1024, dgp.BF16, dgp.SCALE_NONE, 1,
                              dgp.Config(**base, schedule=4, a_layout=lay))
        assert dgp.kernels()[i][0].a_layout == lay
    bad = (dgp.Config(**base, schedule=5), dgp.Config(**base, schedule=-1),
           dgp.Config(**base, schedule=4, a_layout=3), dgp.Config(**base, schedule=1, a_layout=2),
           dgp.Config(16, 64, 0, 0, 1, 0, 0, 0, 0, 0, 1), dgp.Config(16, 64, 0, 0, 1, 0, 0, 0, 0, 0, 0, 1),
           dgp.Config(**base, schedule=4, a_copy=3), dgp.Config(**base, schedule=1, a_copy=2),
           dgp.Config(**base, schedule=2, preload_dsrd=8),
           dgp.Config(16, 64, 0, 0, 1, 0, 0, 0, 0, 1))
    for cfg in bad:
        with pytest.raises(dgp.DgpError) as e:
            dgp.select_kernel(1024, 1024, 1024, dgp.BF16, dgp.SCALE_NONE, 1, cfg)
        assert e.value.name == "DGP_ERR_CONFIG"
    with pytest.raises(dgp.DgpError) as e:
        dgp.select_kernel(1024, 1000, 1024, dgp.BF16, dgp.SCALE_NONE)
    assert e.value.name == "DGP_ERR_SHAPE"


def test_tile_map_rejects_bad_arguments(dgp):
    with pytest.raises(dgp.DgpError):
        dgp.tile_of_workgroup(6, 2, 3, 1, 1, 4)
    with pytest.raises(dgp.DgpError):
        dgp.tile_of_workgroup(0, 0, 3, 1, 1, 4)


def test_product_shares_nothing_with_the_oracle(dgp):
    pkg = os.path.join(ROOT, "dense_gemm_packer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text.replace("no oracle", "")), f
    deps = subprocess.run(["ldd", dgp.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".c", ".py")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "dense_gemm_packer_amd" not in text.replace("dense_gemm_packer_amd/csrc", "")


def test_binding_fails_loudly_without_the_library(dgp, monkeypatch, tmp_path):
    monkeypatch.setattr(dgp, "_lib", None)
    monkeypatch.setattr(dgp, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        dgp.lib()


def test_tune_spec_parsing(dgp):
    from dense_gemm_packer_amd import tune
    assert tune.parse("bf16:4096x4096x8192") == ("bf16", dgp.BF16, dgp.SCALE_NONE, 4096, 4096, 8192, 1)
    assert tune.parse("mx4:16x16384x7168:7") == ("mx4", dgp.FP4_E2M1, dgp.SCALE_MX32, 16, 16384, 7168, 7)
    assert tune.parse("fp8b:16x256x1024")[2] == dgp.SCALE_BLOCK128
    for spec in tune.DEFAULT_SHAPES:
        kind, dt, sm, M, N, K, split = tune.parse(spec)
        assert dgp.select_kernel(M, N, K, dt, sm, split) >= 0     # every default shape is valid


def _t(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype)


def test_binding_operand_checks(dgp):
    """The binding's shape and dtype checks (the C ABI sees pointers only):
    an undersized output, a mismatched weight or undersized scales raise
    ValueError before anything is launched.  Pure host code on CPU tensors."""
    import torch
    f8, bf = torch.float8_e4m3fn, torch.bfloat16
    chk = dgp.check_gemm_operands
    A, Bs = _t((16, 1024), f8), _t((256, 1024), f8)
    one = _t((1,), torch.float32)
    chk(A, Bs, one, one, dgp.SCALE_TENSOR, _t((16, 256), bf))            # good call
    bad = [
        (A, Bs, one, one, dgp.SCALE_TENSOR, _t((16, 128), bf)),          # out too narrow
        (A, Bs, one, one, dgp.SCALE_TENSOR, _t((16, 256), torch.float32)),  # out not bf16
        (A, _t((256, 512), f8), one, one, dgp.SCALE_TENSOR, None),      # K of Bs differs
        (A, _t((256, 1024), bf), one, one, dgp.SCALE_TENSOR, None),     # Bs dtype differs
        (_t((16, 1024, 1), f8), Bs, one, one, dgp.SCALE_TENSOR, None),  # A not 2-D
        (A, Bs, _t((16, 7), torch.float32), _t((2, 8), torch.float32), dgp.SCALE_BLOCK128, None),
        (A, Bs, _t((16, 8), torch.float32), _t((256, 8), torch.float32), dgp.SCALE_BLOCK128, None),
        (A, Bs, _t((16, 8), torch.float32), _t((2, 8), torch.float32), dgp.SCALE_MX128, None),
        (A, Bs, _t((16, 8), torch.uint8), _t((255, 8), torch.uint8), dgp.SCALE_MX128, None),
        (_t((16, 512), torch.float4_e2m1fn_x2), _t((256, 512), torch.float4_e2m1fn_x2),
         _t((16, 8), torch.uint8), _t((256, 32), torch.uint8), dgp.SCALE_MX32, None),
    ]
    for args in bad:
        with pytest.raises(ValueError):
            chk(*args)
    chk(A, Bs, _t((16, 8), torch.float32), _t((2, 8), torch.float32), dgp.SCALE_BLOCK128, None)
    chk(A, Bs, _t((16, 8), torch.uint8), _t((256, 8), torch.uint8), dgp.SCALE_MX128, None)
    chk(_t((16, 512), torch.float4_e2m1fn_x2), _t((256, 512), torch.float4_e2m1fn_x2),
        _t((16, 32), torch.uint8), _t((256, 32), torch.uint8), dgp.SCALE_MX32, None)
    # K that breaks the mode's rule is left to the C ABI's own status
    chk(_t((16, 192), f8), _t((256, 192), f8), one, one, dgp.SCALE_BLOCK128, None)


def test_binding_scale_mode_inference(dgp):
    import torch
    f8 = torch.float8_e4m3fn
    A = _t((1, 128), f8)
    one, many = _t((1,), torch.float32), _t((2, 1), torch.float32)
    assert dgp._scale_mode(A, one, one, None) == dgp.SCALE_TENSOR
    assert dgp._scale_mode(_t((4, 128), f8), _t((4, 1), torch.float32), many, None) == dgp.SCALE_BLOCK128
    # blockscale with M = 1, K = 128: sA holds one value, sB more -- ambiguous, never per-tensor
    with pytest.raises(ValueError):
        dgp._scale_mode(A, one, many, None)
    assert dgp._scale_mode(A, one, many, dgp.SCALE_BLOCK128) == dgp.SCALE_BLOCK128
    assert dgp._scale_mode(A, _t((1, 1), torch.uint8), _t((16, 1), torch.uint8), None) == dgp.SCALE_MX128
    assert dgp._scale_mode(_t((1, 128), torch.bfloat16), None, None, None) == dgp.SCALE_NONE
    assert dgp._scale_mode(_t((1, 64), torch.float4_e2m1fn_x2), None, None, None) == dgp.SCALE_MX32


def test_noalloc_rejects_sizes_past_its_scratch(dgp, L):
    """dgp_gemm_preshuffle_splitk_noalloc refuses split_k * M * N * 4 bytes
    beyond its fixed scratch before any HIP call (no device here)."""
    f = L.dgp_gemm_preshuffle_splitk_noalloc
    # 32 x 16384 x 14 partials = 28 MiB > 16 MiB
    assert f(P, P, P, 32, 16384, 7168, FP8, TENSOR, P, P, 14, None, None) == WS
    assert "scratch" in L.dgp_last_error().decode()
    assert f(P, P, P, 32, 16384, 7168, FP8, TENSOR, P, P, 3, None, None) == SPLITK   # 7168 % 3
    assert f(P, P, P, 32, 16384, 7168, FP8, TENSOR, P, None, 8, None, None) == NULL
    assert dgp.NOALLOC_SCRATCH_BYTES == 16 << 20
    hdr = open(os.path.join(INCLUDE, "dgp.h")).read()
    assert "#define DGP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in hdr
