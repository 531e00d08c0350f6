"""The kernels that issue MFMAs from inline assembly keep the 2 wait states a
matrix-core read needs after a vector-ALU write of the same VGPR (the
compiler enforces them for builtins only).  The sources are compiled to
gfx950 assembly here (no GPU) and scanned; the scanner itself is checked on
planted cases first."""
import os
import tempfile

import pytest

import asm_hazards
from dense_gemm_packer_amd import build

MFMA = "v_mfma_scale_f32_16x16x128_f8f6f4 a[0:3], v[4:7], v[8:11], a[0:3], v12, v13 op_sel_hi:[0,0,0] cbsz:4 blgp:4"


def test_scanner_finds_planted_hazards():
    head = "k:\n"
    assert asm_hazards.find(head + "\tv_bfe_u32 v13, v1, v2, 8\n\t" + MFMA + "\n")
    assert asm_hazards.find(head + "\tv_mov_b32 v5, 0\n\ts_nop 0\n\t" + MFMA + "\n")
    assert not asm_hazards.find(head + "\tv_mov_b32 v5, 0\n\ts_nop 1\n\t" + MFMA + "\n")
    assert not asm_hazards.find(head + "\tv_mov_b32 v5, 0\n\tv_mov_b32 v20, 0\n\ts_nop 0\n\t" + MFMA + "\n")
    assert not asm_hazards.find(head + "\tv_mov_b32 v30, 0\n\t" + MFMA + "\n")      # an unrelated VGPR
    # across a loop back edge: the write at the end of the body, the read at its head
    loop = head + ".LBB0_1:\n\t" + MFMA + "\n\tv_mov_b32 v12, 1\n\ts_cbranch_scc1 .LBB0_1\n"
    assert asm_hazards.find(loop)


@pytest.mark.parametrize("src", ["gemm_w4.hip", "probe.hip"])
def test_inline_asm_mfma_sources_keep_the_wait_states(src):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        build.asm(src, out)
        text = open(out).read()
    assert "v_mfma" in text
    found = asm_hazards.find(text)
    assert not found, found[:5]
