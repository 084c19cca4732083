"""Pins for the oracle's scalar decoders (E4M3-FN and fp16).

E4M3-FN: colibri PR #528 "fmt=7: fp8-e4m3-b128 passthrough weight format",
section "Design" -- the decode must agree with torch.float8_e4m3fn on all 256
codes, NaN only at exponent 15 / mantissa 7, both zeros, subnormals.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
from conftest import golden_lines


def f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


def e4m3_table(o):
    return np.array([o.e4m3(c) for c in range(256)], dtype=np.float64)


def e4m3_matches_torch(o):
    mine = e4m3_table(o).astype(np.float32)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan_m, nan_r = np.isnan(mine), np.isnan(ref)
    if not np.array_equal(nan_m, nan_r):
        return False
    ok = ~nan_m
    return np.array_equal(mine[ok].view(np.uint32), ref[ok].view(np.uint32))


def e4m3_matches_golden(o):
    for code, val in golden_lines("e4m3_codes.txt"):
        got = o.e4m3(int(code, 16))
        if val == "nan":
            if not math.isnan(got):
                return False
        elif f32_bits(float(val)) != f32_bits(got):  # sign of zero included
            return False
    return True


def test_e4m3_all_codes_match_library(qref):
    assert e4m3_matches_torch(qref)


def test_e4m3_spot_codes_from_pages(qref):
    assert e4m3_matches_golden(qref)


def test_e4m3_nan_set_and_range(qref):
    t = e4m3_table(qref)
    assert set(np.flatnonzero(np.isnan(t)).tolist()) == {0x7F, 0xFF}
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    assert not np.isinf(t).any()
    # sign symmetry: code c and c|0x80 are negatives of each other
    for c in range(128):
        if c != 0x7F:
            assert t[c | 0x80] == -t[c]
    # subnormals are m * 2^-9
    assert [t[m] for m in range(8)] == [m * 2.0 ** -9 for m in range(8)]


def test_f16_all_codes_match_numpy(qref):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    mine = np.array([qref.f16(int(c)) for c in codes])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok].astype(np.float32).view(np.uint32),
                          ref[ok].astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("n", [5, 6])
def test_planted_e4m3_mistakes_are_caught(n, mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(n, mutant_dir))
    assert m.mutation == n
    assert not (e4m3_matches_torch(m) and e4m3_matches_golden(m))
