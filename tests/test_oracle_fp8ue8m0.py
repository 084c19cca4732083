"""Pins for the fp8-e4m3 oracle with UE8M0 block scales.

colibri PR #528 "fmt=7: fp8-e4m3-b128 passthrough weight format", section
"Design": the same E4M3 128x128-block geometry ships with one scale byte per
block holding a power-of-two exponent (dtype F8_E8M0) instead of an f32.
The page names the dtype but not its decode; the oracle takes that dtype's
definition, 2^(e - 127) with 255 = NaN, and these tests pin it to
torch.float8_e8m0fnu (a library routine), to closed forms, and to the f32
block-scale oracle fed with the decoded scales.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from test_oracle_fp8 import torch_decode


def torch_e8m0(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e8m0fnu)
    with np.errstate(invalid="ignore"):
        return t.to(torch.float32).numpy().astype(np.float64)


@pytest.fixture(scope="module")
def o():
    return oracle.load()


def pin_all_codes(o):
    codes = np.arange(256, dtype=np.uint8)
    got = np.array([o.e8m0(int(c)) for c in codes])
    ref = torch_e8m0(codes)
    same_nan = np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    return same_nan and np.array_equal(got[ok], ref[ok]) and np.isnan(got[255])


def pin_closed_forms(o):
    return (o.e8m0(127) == 1.0 and o.e8m0(128) == 2.0 and o.e8m0(126) == 0.5
            and o.e8m0(0) == 2.0 ** -127 and o.e8m0(254) == 2.0 ** 127)


def dense_from_draws(d):
    O, I = d["O"], d["I"]
    s = np.repeat(np.repeat(torch_e8m0(d["scale_e8m0"]), 128, 0), 128, 1)[:O, :I]
    return torch_decode(d["w"]) * s


def pin_dequant_exact(o, O=130, I=300, seed=5):
    d = W.gen_fp8ue8m0(O, I, seed=seed)
    got = o.fp8ue8m0_dequant(d["w"], d["scale_e8m0"], O, I)
    return np.array_equal(got.view(np.uint32), dense_from_draws(d).astype(np.float32).view(np.uint32))


def pin_brute_force(o, O=130, I=200, S=2, seed=6):
    d = W.gen_fp8ue8m0(O, I, S=S, seed=seed)
    yref = d["x"].astype(np.float64) @ dense_from_draws(d).T
    y = o.fp8ue8m0_gemv(d["w"], d["scale_e8m0"], d["x"], O, I)
    return np.allclose(y, yref, rtol=1e-6, atol=1e-6 * np.abs(yref).max())


def pin_equals_f32_scales(o, O=257, I=384, S=2, seed=7):
    # the same weights with the decoded scales as f32 give the same y, bit for bit
    d = W.gen_fp8ue8m0(O, I, S=S, seed=seed)
    sc = torch_e8m0(d["scale_e8m0"]).astype(np.float32)
    a = o.fp8ue8m0_gemv(d["w"], d["scale_e8m0"], d["x"], O, I)
    b = o.fp8b128_gemv(d["w"], sc, d["x"], O, I)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def run_pins(o):
    return {"all_codes": pin_all_codes(o), "closed_forms": pin_closed_forms(o),
            "dequant": pin_dequant_exact(o), "brute": pin_brute_force(o),
            "f32_scales": pin_equals_f32_scales(o)}


def test_pins_hold(o):
    r = run_pins(o)
    assert all(r.values()), r


def test_extremes_decode(o):
    # 448 * 2^127 overflows f32 (inf), 2^-9 * 2^-127 is an exact f32 subnormal,
    # a NaN scale byte poisons its block
    w = np.array([[0x7E, 0x01, 0x38]], np.uint8)
    for e, want in [(254, [np.inf, 2.0 ** 118, 2.0 ** 127]), (0, [448 * 2.0 ** -127, 2.0 ** -136, 2.0 ** -127])]:
        got = o.fp8ue8m0_dequant(w, np.array([[e]], np.uint8), 1, 3)[0]
        assert np.array_equal(got, np.array(want, np.float32))
    got = o.fp8ue8m0_dequant(w, np.array([[255]], np.uint8), 1, 3)[0]
    assert np.isnan(got).all()


def test_planted_bias_mistake_is_caught(mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(11, mutant_dir))
    assert m.mutation == 11
    r = run_pins(m)
    assert not all(r.values()), r
