"""Pins for the oracle's element decoders and its fp32 -> bf16 rounding.

Each decoder is checked exhaustively against torch's own conversions (an
independent library implementation) and against format facts stored under
tests/golden with their source.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split()[:2])
    return rows


def test_e4m3_exhaustive_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = orc.decode_array(codes, orc.FP8_E4M3)
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(got[c]), hex(c)
        else:
            assert got[c] == ref[c] and math.copysign(1, got[c]) == math.copysign(1, ref[c]), hex(c)


def test_e4m3_ocp_table(orc):
    rows = _load_pairs("e4m3fn_ocp_values.txt")
    assert len(rows) >= 15
    for code, val in rows:
        got = orc.e4m3_decode(int(code, 16))
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e4m3_nan_codes_only_two(orc):
    nans = [c for c in range(256) if math.isnan(orc.e4m3_decode(c))]
    assert nans == [0x7F, 0xFF]
    finite = [abs(orc.e4m3_decode(c)) for c in range(256) if c not in (0x7F, 0xFF)]
    assert max(finite) == 448.0


def test_bf16_decode_exhaustive_matches_torch(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    got = orc.decode_array(codes, orc.BF16)
    both_nan = np.isnan(ref) & np.isnan(got)
    same = (got.view(np.uint32) == ref.view(np.uint32))
    assert np.all(same | both_nan)


def test_bf16_round_golden_cases(orc):
    rows = _load_pairs("bf16_rne_cases.txt")
    assert len(rows) >= 15
    for f32, b16 in rows:
        x = np.array([int(f32, 16)], dtype=np.uint32).view(np.float32)[0]
        assert orc.bf16_round(x) == int(b16, 16), f32


def test_bf16_round_matches_torch_random(orc):
    g = np.random.Generator(np.random.PCG64(7))
    bits = g.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # include many exact ties and near-ties
    bits[:20000] = (bits[:20000] & 0xFFFF0000) | 0x8000
    bits[20000:30000] = (bits[20000:30000] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lib = orc.lib()
    got = np.fromiter((lib.oracle_bf16_round(float(v)) for v in x), dtype=np.uint16, count=x.size)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN: quiet NaN with the sign kept
    g16 = got[nan]
    assert np.all((g16 & 0x7F80) == 0x7F80) and np.all(g16 & 0x0040)
    assert np.array_equal(g16 >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_bf16_round_is_identity_on_bf16_values(orc):
    codes = np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16)
    for c in codes:
        f = orc.bf16_decode(int(c))
        if math.isnan(f):
            continue
        assert orc.bf16_round(f) == c
