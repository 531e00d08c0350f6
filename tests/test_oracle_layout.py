"""Pins for the oracle's preshuffle layout (a byte permutation of B).

No page writes the layout out, so it is this library's own definition; the
pins are the properties the GEMM relies on: it is a bijection on bytes, the
unshuffle undoes it bit-exactly for every byte value (NaN codes included),
and a wave that reads 16 bytes per lane from a 1 KiB block receives, lane by
lane, the B operand of a 16x16 MFMA tile (lane l: column l % 16, a run of 16
consecutive K-bytes starting at 16*(l // 16)).
"""
import numpy as np
import pytest


def _perm(orc, N, Kb):
    """Source byte index of each destination byte, via four byte planes."""
    idx = np.arange(N * Kb, dtype=np.uint32)
    planes = []
    for sh in (0, 8, 16, 24):
        plane = ((idx >> sh) & 0xFF).astype(np.uint8).reshape(N, Kb)
        planes.append(orc.preshuffle_b(plane).reshape(-1).astype(np.uint32) << sh)
    return planes[0] | planes[1] | planes[2] | planes[3]


@pytest.mark.parametrize("N,Kb", [(16, 64), (32, 192), (48, 1024), (256, 512)])
def test_preshuffle_is_a_bijection(orc, N, Kb):
    p = _perm(orc, N, Kb)
    counts = np.bincount(p, minlength=N * Kb)
    assert counts.shape[0] == N * Kb and np.all(counts == 1)


@pytest.mark.parametrize("dtype,N,K", [("u8", 16, 64), ("u8", 64, 448), ("u16", 32, 96),
                                       ("u16", 128, 256)])
def test_unshuffle_inverts_preshuffle_bit_exact(orc, dtype, N, K):
    g = np.random.Generator(np.random.PCG64(5))
    if dtype == "u8":
        B = g.integers(0, 256, size=(N, K), dtype=np.uint8)
        B[0, :8] = [0x7F, 0xFF, 0x00, 0x80, 0x7E, 0xFE, 0x01, 0x81]
    else:
        B = g.integers(0, 65536, size=(N, K), dtype=np.uint16)
        B[0, :4] = [0x7FC0, 0xFFC1, 0x7F80, 0x8000]
    Bs = orc.preshuffle_b(B)
    assert Bs.shape == B.shape and Bs.dtype == B.dtype
    assert not np.array_equal(Bs, B)
    assert np.array_equal(orc.unshuffle_b(Bs), B)
    assert np.array_equal(orc.preshuffle_b(orc.unshuffle_b(Bs)), Bs)


@pytest.mark.parametrize("N,Kb", [(32, 128), (64, 256)])
def test_wave_read_of_a_block_is_an_mfma_b_operand(orc, N, Kb):
    """Every 1 KiB block, read 16 B per lane, gives lane l the bytes of one
    B row (column n of B^T) = 16*nb + l%16, K-bytes 64*kb + 16*(l//16) + [0,16),
    with blocks ordered strip-major (all K blocks of rows 16nb..16nb+15 first)."""
    p = _perm(orc, N, Kb).reshape(-1, 64, 16)    # [block][lane][byte]
    kblocks = Kb // 64
    for blk in range(p.shape[0]):
        nb, kb = divmod(blk, kblocks)
        for lane in range(64):
            src = p[blk, lane]
            row, col = np.divmod(src.astype(np.int64), Kb)
            assert np.all(row == 16 * nb + lane % 16)
            assert np.array_equal(col, 64 * kb + 16 * (lane // 16) + np.arange(16))


def test_rejects_unsupported_shapes(orc):
    with pytest.raises(ValueError):
        orc.preshuffle_b(np.zeros((24, 64), np.uint8))     # N % 16
    with pytest.raises(ValueError):
        orc.preshuffle_b(np.zeros((16, 48), np.uint8))     # K bytes % 64
    with pytest.raises(ValueError):
        orc.preshuffle_b(np.zeros((16, 40), np.uint16))    # 80 bytes
