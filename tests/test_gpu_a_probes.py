"""Hardware facts the GEMM relies on, checked on the device: the register
layout of the two matrix-core instructions, and where the async
global->LDS copy puts each lane's 16 bytes."""
import numpy as np
import pytest
import torch

import dense_gemm_packer_amd as dgp
from gpu_common import DEV

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_mfma_bf16_16x16x32_layout():
    """First operand lane l: row l%16, K 8*(l//16)+j; second operand lane l:
    column l%16, same K; result lane l: rows 4*(l//16)+r, column l%16."""
    g = np.random.Generator(np.random.PCG64(1))
    X = g.integers(-3, 4, size=(16, 32)).astype(np.float32)   # first operand, 16 x K
    Y = g.integers(-3, 4, size=(32, 16)).astype(np.float32)   # second operand, K x 16
    a = np.zeros((64, 8), np.float32)
    b = np.zeros((64, 8), np.float32)
    for l in range(64):
        for j in range(8):
            a[l, j] = X[l % 16, 8 * (l // 16) + j]
            b[l, j] = Y[8 * (l // 16) + j, l % 16]
    ta = torch.from_numpy(_bf16_bits(a).view(np.uint8).copy()).to(DEV)
    tb = torch.from_numpy(_bf16_bits(b).view(np.uint8).copy()).to(DEV)
    out = dgp.probe_mfma_layout(0, ta, tb).cpu().numpy()
    D = X @ Y
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)], np.float32)
    assert np.array_equal(out, want)


def test_mfma_fp8_16x16x128_layout():
    """e4m3 operands, 32 bytes per lane assembled as the library does: bytes
    0..15 = K 16*(l//16)+j, bytes 16..31 = K 64+16*(l//16)+j.  Any K order the
    hardware uses is shared by both operands, so the product must come out
    exact; the result layout is as for bf16."""
    g = np.random.Generator(np.random.PCG64(2))
    X = g.integers(-4, 5, size=(16, 128)).astype(np.float32)
    Y = g.integers(-4, 5, size=(128, 16)).astype(np.float32)
    a = np.zeros((64, 32), np.float32)
    b = np.zeros((64, 32), np.float32)
    for l in range(64):
        ks = [16 * (l // 16) + j for j in range(16)] + [64 + 16 * (l // 16) + j for j in range(16)]
        a[l] = X[l % 16, ks]
        b[l] = Y[ks, l % 16]
    to8 = lambda v: torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).contiguous().to(DEV)
    out = dgp.probe_mfma_layout(1, to8(a), to8(b)).cpu().numpy()
    D = X @ Y
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)], np.float32)
    assert np.array_equal(out, want)


@pytest.mark.parametrize("per_group", [False, True])
def test_mfma_scaled_e8m0_semantics(per_group):
    """Hardware-scaled e4m3 MFMA with the library's operand assembly (lane l:
    bytes 0..15 = K 16*(l//16)+j, bytes 16..31 = K 64+16*(l//16)+j).  The
    scales act on 32-wide K blocks in that logical K order, [32q, 32q+32),
    and lane 16q+i supplies block q's scale for row i of the first operand
    (B fragment) and column i of the second (A fragment) -- so the byte order
    of the preshuffled layout is the instruction's own K order.  With
    per_group False the four blocks of a row/column share one scale (the
    128-K block of the mxfp8 mode); with True they differ.  Exact small
    integers and scales 2^-2..2^2: every product and sum is exact."""
    g = np.random.Generator(np.random.PCG64(4 + per_group))
    X = g.integers(-4, 5, size=(16, 128)).astype(np.float32)   # first operand: 16 rows x K
    Y = g.integers(-4, 5, size=(128, 16)).astype(np.float32)   # second operand: K x 16
    if per_group:
        sb = g.integers(125, 130, size=64).astype(np.uint8)
        sa = g.integers(125, 130, size=64).astype(np.uint8)
    else:
        sb = np.tile(g.integers(125, 130, size=16), 4).astype(np.uint8)
        sa = np.tile(g.integers(125, 130, size=16), 4).astype(np.uint8)
    xa = np.zeros((64, 32), np.float32)   # first-operand lanes (rows of X)
    yb = np.zeros((64, 32), np.float32)   # second-operand lanes (columns of Y)
    groups = []
    for l in range(64):
        ks = [16 * (l // 16) + j for j in range(16)] + [64 + 16 * (l // 16) + j for j in range(16)]
        xa[l] = X[l % 16, ks]
        yb[l] = Y[ks, l % 16]
    for q in range(4):
        groups.append(list(range(32 * q, 32 * q + 32)))
    to8 = lambda v: torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).contiguous().to(DEV)
    u8 = lambda v: torch.from_numpy(v).to(DEV)
    # the probe passes its `b` buffer as the first operand and `a` as the second
    out = dgp.probe_mfma_scaled(to8(yb), to8(xa), u8(sa), u8(sb), which=0).cpu().numpy()
    D = np.zeros((16, 16))
    for q in range(4):
        ks = groups[q]
        sub = X[:, ks].astype(np.float64) @ Y[ks, :].astype(np.float64)
        D += sub * np.exp2(sb[16 * q:16 * q + 16].astype(np.float64) - 127)[:, None] \
                 * np.exp2(sa[16 * q:16 * q + 16].astype(np.float64) - 127)[None, :]
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)], np.float32)
    assert np.array_equal(out, want)


def _pack_e2m1(vals):
    """values on the E2M1 grid -> packed bytes, even element in the low nibble."""
    import synth
    return synth.pack_e2m1(synth.to_e2m1_codes(np.asarray(vals, np.float32)))


def test_mfma_scaled_e2m1_semantics():
    """Hardware-scaled MFMA on E2M1 operands (cbsz = blgp = 4) with the
    library's fp4 operand assembly: lane l holds the 16 bytes = 32 values of
    K [32g, 32g+32) (g = l//16) of its row -- in the preshuffled layout, a
    lane's 16-byte read of a 64-byte chunk.  Each lane's block is then
    exactly one 32-element microscaling block, and lane 16q+i's scale byte
    scales block q of row i (first operand) / column i (second operand)."""
    g = np.random.Generator(np.random.PCG64(6))
    X = g.integers(-4, 5, size=(16, 128)).astype(np.float32)   # first operand
    Y = g.integers(-4, 5, size=(128, 16)).astype(np.float32)   # second operand
    sb = g.integers(125, 130, size=64).astype(np.uint8)
    sa = g.integers(125, 130, size=64).astype(np.uint8)
    first = np.zeros((64, 32), np.uint8)
    second = np.zeros((64, 32), np.uint8)
    for l in range(64):
        q, i = l // 16, l % 16
        first[l, :16] = _pack_e2m1(X[i, 32 * q:32 * q + 32])
        second[l, :16] = _pack_e2m1(Y[32 * q:32 * q + 32, i])
    u8 = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    # the probe passes its `b` buffer as the first operand and `a` as the second
    out = dgp.probe_mfma_scaled(u8(second), u8(first), u8(sa), u8(sb), which=1).cpu().numpy()
    D = np.zeros((16, 16))
    for q in range(4):
        ks = slice(32 * q, 32 * q + 32)
        D += (X[:, ks].astype(np.float64) @ Y[ks, :].astype(np.float64)) \
            * np.exp2(sb[16 * q:16 * q + 16].astype(np.float64) - 127)[:, None] \
            * np.exp2(sa[16 * q:16 * q + 16].astype(np.float64) - 127)[None, :]
    want = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)], np.float32)
    assert np.array_equal(out, want)


def test_lds_dma_destination_is_linear_per_lane():
    g = np.random.Generator(np.random.PCG64(3))
    src = g.integers(0, 256, size=1024, dtype=np.uint8)
    perm = g.permutation(64).astype(np.int32)
    out = dgp.probe_lds_dma(torch.from_numpy(src).to(DEV), torch.from_numpy(perm).to(DEV)).cpu().numpy()
    want = np.concatenate([src[16 * p:16 * p + 16] for p in perm])
    assert np.array_equal(out, want)


@pytest.mark.parametrize("width", [1, 2, 4])
def test_lds_dma_narrow_lands_one_dword_per_lane(width):
    # The per-k-tile scale staging of the tiled GEMM relies on this: a load of
    # 1, 2 or 4 bytes per lane writes lane l's value, zero-extended, as LDS
    # dword l, and nothing beyond the first 256 bytes is touched.
    g = np.random.Generator(np.random.PCG64(4 + width))
    src = g.integers(0, 256, size=1024, dtype=np.uint8)
    perm = g.permutation(64).astype(np.int32)
    out = dgp.probe_lds_dma_narrow(width, torch.from_numpy(src).to(DEV),
                                   torch.from_numpy(perm).to(DEV)).cpu().numpy()
    got = out[:256].reshape(64, 4)
    want = np.stack([src[width * p:width * p + width] for p in perm])
    assert np.array_equal(got[:, :width], want)
    assert np.all(got[:, width:] == 0)
    assert np.all(out[256:] == 0xFF)


def test_probe_copy_copies():
    x = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(x)
    dgp.probe_copy(x, y)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_probe_mfma_peak_runs_and_leaves_sink(which):
    # The register-only loop touches memory only on a practically impossible
    # value, so the sink stays as written; the FLOP count is the documented one.
    ops = torch.randint(0, 255, (dgp.MFMA_PEAK_OPERAND_BYTES[which],), dtype=torch.uint8, device=DEV)
    ops[ops == 0x7F] = 0   # no e4m3 NaN codes
    ops[ops == 0xFF] = 0
    sink = torch.full((4096,), 7, dtype=torch.int32, device=DEV)
    flop = dgp.probe_mfma_peak(which, 16, 8, ops, sink)
    torch.cuda.synchronize()
    assert flop == 8 * 4 * 16 * 64 * (16384 if which == 0 else 65536)
    assert dgp.MFMA_PEAK_OPERAND_BYTES[which] == 256 * 16 * 64 * (32 if which == 1 else 16)
    assert bool((sink == 7).all())
