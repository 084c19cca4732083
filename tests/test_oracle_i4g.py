"""Pins for the grouped-int4 ("fmt=4") oracle.

colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV support": section 1 (one f32
scale per gs-element group along I), section 3 (nibble layout and
w = (q - 8) * scale[row][col/gs], scale applied per group before the
cross-group sum), section 5 (shape matrix: I a multiple of gs, I = 200 / 201
not a multiple, I <= gs, S = 1..4, an activation forced to 50.0 in group 0)
and section 10 (the mutation classes the tests must catch: off-by-one group
index, swapped nibbles, a uniform 1% scale error).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from conftest import golden_kv, unpack_nibbles


def dense_from_draws(d):
    """f64 dense W built from the drawn nibbles and scales (no oracle code)."""
    O, I, gs = d["O"], d["I"], d["gs"]
    q = unpack_nibbles(d["w"], I)
    s = np.repeat(d["scales"].astype(np.float64), gs, axis=1)[:, :I]
    return (q - 8) * s


def pin_golden(o):
    g = golden_kv("i4g_handbuilt.txt")
    O, I, gs = int(g["O"][0]), int(g["I"][0]), int(g["gs"][0])
    wb = np.array([int(b, 16) for b in g["bytes"]], np.uint8).reshape(O, -1)
    s = np.array(g["scales"], np.float32).reshape(O, -1)
    Wx = np.array(g["W"], np.float32).reshape(O, I)
    x = np.array(g["x"], np.float32)
    y = np.array(g["y"], np.float32)
    return (np.array_equal(o.i4g_dequant(wb, s, O, I, gs), Wx)
            and np.array_equal(o.i4g_gemv(wb, s, x, O, I, gs)[0], y))


def pin_brute_force(o, O=37, I=200, gs=64, S=2, seed=3):
    d = W.gen_i4g(O, I, gs, S=S, seed=seed)
    Wd = dense_from_draws(d)
    if not np.array_equal(o.i4g_dequant(d["w"], d["scales"], O, I, gs), Wd.astype(np.float32)):
        return False
    yref = (d["x"].astype(np.float64) @ Wd.T)
    y = o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs)
    return np.allclose(y, yref, rtol=1e-6, atol=1e-6 * np.abs(yref).max())


def pin_per_row_form(o, O=16, I=96, seed=4):
    # gs >= I: a single group per row, so y = s_o * sum (q - 8) x  (the
    # per-row-scale int4 form of colibri PR #457, section 3)
    d = W.gen_i4g(O, I, gs=128, seed=seed)
    q = unpack_nibbles(d["w"], I)
    yref = d["scales"][:, 0].astype(np.float64) * ((q - 8) @ d["x"][0].astype(np.float64))
    y = o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, 128)[0]
    return np.allclose(y, yref, rtol=1e-6, atol=1e-7)


def pin_one_hot_columns(o, O=8, I=130, gs=32, seed=5):
    d = W.gen_i4g(O, I, gs, seed=seed)
    Wd = dense_from_draws(d).astype(np.float32)
    for c in (0, 1, 31, 32, 63, 64, 129):
        x = np.zeros(I, np.float32)
        x[c] = 1.0
        if not np.array_equal(o.i4g_gemv(d["w"], d["scales"], x, O, I, gs)[0], Wd[:, c]):
            return False
    return True


def run_pins(o):
    return {"golden": pin_golden(o), "brute": pin_brute_force(o),
            "brute_odd": pin_brute_force(o, O=5, I=201, gs=64, S=3, seed=8),
            "per_row": pin_per_row_form(o), "one_hot": pin_one_hot_columns(o)}


def test_pins_hold(qref):
    r = run_pins(qref)
    assert all(r.values()), r


def test_all_eights_give_zero(qref):
    O, I, gs = 4, 256, 64
    wb = np.full((O, I // 2), 0x88, np.uint8)
    s = np.full((O, I // gs), 0.01, np.float32)
    x = np.random.default_rng(0).standard_normal(I).astype(np.float32)
    y = qref.i4g_gemv(wb, s, x, O, I, gs)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("O,I,gs,S", [(64, 6144, 64, 1), (48, 2048, 64, 4), (33, 200, 64, 2),
                                      (33, 201, 64, 3), (16, 64, 64, 1), (16, 40, 64, 1),
                                      (24, 512, 128, 1), (9, 300, 16, 2)])
def test_shape_matrix_brute_force(qref, O, I, gs, S):
    assert pin_brute_force(qref, O=O, I=I, gs=gs, S=S, seed=O + I)


@pytest.mark.parametrize("I", [512, 201])
def test_outlier_activation_in_group0(qref, I):
    d = W.gen_i4g(20, I, 64, seed=11)
    d["x"][0, 3] = 50.0
    yref = d["x"][0].astype(np.float64) @ dense_from_draws(d).T
    y = qref.i4g_gemv(d["w"], d["scales"], d["x"], 20, I, 64)[0]
    assert np.allclose(y, yref, rtol=1e-6, atol=1e-6)


def test_row_subset_matches_full(qref):
    d = W.gen_i4g(50, 320, 64, S=2, seed=12)
    full = qref.i4g_gemv(d["w"], d["scales"], d["x"], 50, 320, 64)
    rows = [49, 0, 17, 17, 3]
    sub = qref.i4g_gemv(d["w"], d["scales"], d["x"], 50, 320, 64, rows=rows)
    assert np.array_equal(sub, full[:, rows])


def test_thread_count_does_not_change_results(qref):
    d = W.gen_i4g(300, 1024, 64, seed=13)
    qref.set_threads(1)
    a = qref.i4g_gemv(d["w"], d["scales"], d["x"], 300, 1024, 64)
    qref.set_threads(4)
    b = qref.i4g_gemv(d["w"], d["scales"], d["x"], 300, 1024, 64)
    qref.set_threads(1)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("n", [1, 2, 3])
def test_planted_i4g_mistakes_are_caught(n, mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(n, mutant_dir))
    r = run_pins(m)
    assert not all(r.values()), r
