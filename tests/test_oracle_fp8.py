"""Pins for the fp8-e4m3 128x128-block oracle ("fmt=7").

colibri PR #528 "fmt=7: fp8-e4m3-b128 passthrough weight format": section
"Design" (O*I raw E4M3-FN bytes; one f32 per 128x128 block, row-major block
order, ceil(O/128)*ceil(I/128) entries; w = decode(byte) * scale, a multiply)
and section "Metal validation record" (block-edge shapes 130x200, 129x128,
128x129, 1x1, the stride audit 384x6144 with a 3x48 block grid, the
[2048,6144] / [6144,2048] projection shapes at S = 1 and S = 4, and the
review's 130x130 partial-block tensor checked at all 16,900 positions; NaN
weights poison their row).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def dense_from_draws(d):
    O, I = d["O"], d["I"]
    dec = torch_decode(d["w"])
    s = np.repeat(np.repeat(d["scale_inv"].astype(np.float64), 128, 0), 128, 1)[:O, :I]
    return dec * s


def pin_dequant_exact(o, O=130, I=130, seed=1):
    d = W.gen_fp8b128(O, I, seed=seed)
    return np.array_equal(o.fp8b128_dequant(d["w"], d["scale_inv"], O, I).view(np.uint32),
                          dense_from_draws(d).astype(np.float32).view(np.uint32))


def pin_brute_force(o, O=130, I=200, S=2, seed=2):
    d = W.gen_fp8b128(O, I, S=S, seed=seed)
    yref = d["x"].astype(np.float64) @ dense_from_draws(d).T
    y = o.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I)
    return np.allclose(y, yref, rtol=1e-6, atol=1e-6 * np.abs(yref).max())


def pin_single_block(o, O=100, I=77, seed=3):
    d = W.gen_fp8b128(O, I, seed=seed)
    yref = float(d["scale_inv"][0, 0]) * (torch_decode(d["w"]) @ d["x"][0].astype(np.float64))
    y = o.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I)[0]
    return np.allclose(y, yref, rtol=1e-6, atol=1e-9)


def pin_nan_row(o, O=6, I=300):
    d = W.gen_fp8b128(O, I, seed=4)
    d["w"][2, 150] = 0x7F
    d["w"][4, 7] = 0xFF
    y = o.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I)[0]
    return bool(np.isnan(y[2]) and np.isnan(y[4]) and np.isfinite(np.delete(y, [2, 4])).all())


def run_pins(o):
    return {"dequant": pin_dequant_exact(o), "brute": pin_brute_force(o),
            "grid": pin_brute_force(o, O=384, I=6144, S=3, seed=7),
            "single": pin_single_block(o), "nan": pin_nan_row(o)}


def test_pins_hold(qref):
    r = run_pins(qref)
    assert all(r.values()), r


@pytest.mark.parametrize("O,I,S", [(130, 200, 2), (129, 128, 1), (128, 129, 1), (1, 1, 1),
                                   (384, 6144, 3), (256, 6144, 4), (300, 2048, 1)])
def test_shape_matrix(qref, O, I, S):
    assert pin_brute_force(qref, O=O, I=I, S=S, seed=O * 7 + I)


def test_partial_block_dequant_all_positions(qref):
    assert pin_dequant_exact(qref, 130, 130, seed=9)


def test_negative_zero_survives(qref):
    w = np.array([[0x80, 0x00]], np.uint8)
    s = np.array([[0.5]], np.float32)
    W_ = qref.fp8b128_dequant(w, s, 1, 2)
    assert W_.view(np.uint32).tolist() == [[0x80000000, 0]]


@pytest.mark.parametrize("n", [4, 5])
def test_planted_fp8_mistakes_are_caught(n, mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(n, mutant_dir))
    r = run_pins(m)
    assert not all(r.values()), r
