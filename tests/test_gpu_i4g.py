"""Grouped-int4 GEMV on the GPU against the CPU oracle.

Shapes follow colibri PR #457, section 5 (I a multiple of gs, I = 200 / 201,
I <= gs, S = 1..4, an activation forced to 50.0 in group 0) plus the
workload shapes O=256 x I=512 and O=12288 x I=6144 at gs = 64 and 128.
Decoded weights must match bit for bit (the decode-only export, and one-hot
activations through the streaming GEMV itself); y to relative L2 <= 1e-5 and
every element to |dy| / sum_i |w_i x_i| <= 1e-4.  The cases include several
vectors per call, infinities, a twelve-decade dynamic range, and outliers on
a column whose weights are all zero (the staged fixed point is then not
precise enough and the kernel multiplies per element in f32).  Canary zones
around y catch stray writes.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import (assert_bits_equal, assert_guard_intact, assert_y_close, dev, guarded, host,
                      magnitude, torch_cuda)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


@pytest.mark.parametrize("O,I,gs", [(256, 512, 64), (37, 201, 64), (64, 6144, 128), (5, 40, 64),
                                    (130, 300, 16), (1, 1, 2)])
def test_dequant_bit_exact(q, qref, O, I, gs):
    d = W.gen_i4g(O, I, gs, seed=O + I)
    got = host(q.dequant_i4g(dev(d["w"]), dev(d["scales"]), I, gs))
    assert_bits_equal(got, qref.i4g_dequant(d["w"], d["scales"], O, I, gs))


@pytest.mark.parametrize("O,I,gs,S", [
    (256, 512, 64, 1),        # small workload
    (12288, 6144, 64, 1),     # resident-projection workload, gs 64
    (12288, 6144, 128, 1),    # same shape, gs 128
    (2048, 6144, 64, 4), (6144, 2048, 64, 1), (333, 2048, 64, 3),
    (77, 200, 64, 2), (77, 201, 64, 1), (9, 64, 64, 1), (9, 40, 64, 4),
    (50, 512, 64, 8), (100, 1024, 96, 2), (31, 4096, 256, 1), (3, 96, 32, 1),
    (1, 32, 32, 1), (1, 1, 2, 1),
    # tiles the launcher picks by rows on the busiest CU: two rows per lane
    # group (16384 x 512), one row (20000 x 1024, ragged)
    (16384, 512, 64, 1), (20000, 1024, 64, 1),
    # few rows of long rows: 64 lanes per row, a ring of four sweeps
    (2048, 14336, 64, 1), (1000, 8192, 128, 1), (4096, 6144, 64, 1),
    # several vectors: 16-wave workgroups; S > 4 runs as groups of streaming launches
    (12288, 6144, 64, 2), (4000, 6144, 64, 4), (300, 1024, 64, 6), (65, 6144, 64, 7),
    # four vectors, scale groups of one, two and three 64-column blocks, ragged
    # row blocks
    (1000, 6144, 128, 4), (96, 4096, 192, 4), (17, 64, 64, 4), (12288, 6144, 64, 4),
])
def test_gemv_matches_oracle(q, qref, O, I, gs, S):
    d = W.gen_i4g(O, I, gs, S=S, seed=7 * O + I)
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    mag = magnitude(qref.i4g_dequant(d["w"], d["scales"], O, I, gs), d["x"])
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs), mag=mag)


@pytest.mark.parametrize("S,big", [(1, 1e3), (1, 1e4), (4, 1e4), (2, 3e5)])
def test_outlier_on_zero_weight_column(q, qref, S, big):
    # an activation 1e3..3e5 times its chunk neighbours on a column whose
    # weights are all zero (nibble 8): the outlier contributes nothing, so y
    # rests on the neighbours, which a fixed point sharing the outlier's
    # exponent would carry to about 2^-21 * big only
    O, I, gs = 512, 6144, 64
    d = W.gen_i4g(O, I, gs, S=S, seed=int(big) + S)
    col = 130
    b = d["w"][:, col // 2]
    d["w"][:, col // 2] = (b & 0xF0) | 0x08 if col % 2 == 0 else (b & 0x0F) | 0x80
    d["x"][:, col] = big
    Wd = qref.i4g_dequant(d["w"], d["scales"], O, I, gs)
    assert np.all(Wd[:, col] == 0.0)
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs),
                   mag=magnitude(Wd, d["x"]))


@pytest.mark.parametrize("O,I,gs,S", [(256, 2048, 64, 1), (300, 6144, 128, 1), (96, 4096, 64, 4)])
def test_one_hot_columns_bit_exact(q, qref, O, I, gs, S):
    # x = e_j (1.0) through the streaming GEMV: the fixed point of 1.0 is
    # exact, so y is the decoded column j, (q - 8) * s with one rounding
    import torch
    d = W.gen_i4g(O, I, gs, seed=O + 3)
    Wd = qref.i4g_dequant(d["w"], d["scales"], O, I, gs)
    wt, st = dev(d["w"]), dev(d["scales"])
    cols = [0, 1, 7, 8, 31, 32, 33, 63, 64, gs - 1, gs, I // 2 + 5, I - 2, I - 1]
    for c0 in range(0, len(cols), S):
        cs = cols[c0:c0 + S]
        x = torch.zeros((len(cs), I), device="cuda")
        for t, j in enumerate(cs):
            x[t, j] = 1.0
        y = host(q.i4g(wt, st, x, gs))
        for t, j in enumerate(cs):
            assert_bits_equal(y[t], Wd[:, j])


@pytest.mark.parametrize("I", [512, 201])
def test_outlier_activation(q, qref, I):
    d = W.gen_i4g(64, I, 64, seed=3)
    d["x"][0, 5] = 50.0
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], 64, I, 64),
                   mag=magnitude(qref.i4g_dequant(d["w"], d["scales"], 64, I, 64), d["x"]))


def test_magnitude_relative_error(q, qref):
    # per-element |dy| / sum_i |w_i x_i| <= 1e-4 (colibri PR #457, section 5)
    O, I, gs = 512, 2048, 64
    d = W.gen_i4g(O, I, gs, seed=21)
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))[0]
    ref = qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs)[0]
    mag = np.abs(qref.i4g_dequant(d["w"], d["scales"], O, I, gs).astype(np.float64)) @ \
        np.abs(d["x"][0].astype(np.float64))
    assert np.max(np.abs(y - ref) / mag) <= 1e-4


def test_nan_activation_poisons_all_rows(q):
    d = W.gen_i4g(40, 256, 64, seed=4)
    d["x"][0, 100] = np.nan
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    assert np.isnan(y).all()


@pytest.mark.parametrize("O,I,S", [(300, 512, 1), (12288, 6144, 1), (200, 6144, 2),
                                   (200, 6144, 4)])
def test_infinite_activations_propagate(q, qref, O, I, S):
    # an infinity makes its rows +-inf, or NaN where a zero weight meets it or
    # two infinities of opposite sign meet, exactly as in the plain definition
    d = W.gen_i4g(O, I, 64, S=S, seed=O + S)
    d["x"][0, 37] = np.inf
    d["x"][S - 1, I - 3] = -np.inf
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    ref = qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, 64)
    assert np.isinf(ref).any() and np.isnan(ref).any()
    assert_y_close(y, ref)


@pytest.mark.parametrize("O,I,S", [(512, 6144, 1), (256, 2048, 2), (256, 2048, 4)])
def test_wide_dynamic_range_activations(q, qref, O, I, S):
    # magnitudes spread over twelve decades, zeros, subnormals and one chunk
    # holding a value 1e4 times its neighbours
    d = W.gen_i4g(O, I, 64, S=S, seed=3 * O + S)
    rng = np.random.default_rng(99)
    x = d["x"] * (10.0 ** rng.uniform(-6, 6, size=d["x"].shape)).astype(np.float32)
    x[:, 64:96] = 0.0
    x[:, 96:100] = np.float32(1e-40)
    x[:, 130] = 1e4 * np.abs(x[:, 131]).max() + 1.0
    d["x"] = x.astype(np.float32)
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, 64),
                   mag=magnitude(qref.i4g_dequant(d["w"], d["scales"], O, I, 64), d["x"]))


def test_zero_activations_give_zero(q):
    d = W.gen_i4g(128, 2048, 64, seed=8)
    d["x"][:] = 0.0
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    assert np.all(y == 0.0)


def test_misaligned_weights_take_general_path(q, qref):
    import torch
    O, I, gs = 20, 512, 64
    d = W.gen_i4g(O, I, gs, seed=5)
    buf = torch.zeros(d["w"].size + 8, dtype=torch.uint8, device="cuda")
    buf[8:] = dev(d["w"].reshape(-1))
    w_off = buf[8:]  # 8-byte offset: not 16-byte aligned
    y = torch.empty((1, O), dtype=torch.float32, device="cuda")
    x = dev(d["x"])
    s = dev(d["scales"])
    st = q.qgemv_i4g(w_off.data_ptr(), s.data_ptr(), x.data_ptr(), y.data_ptr(), 1, I, O, gs,
                     torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert_y_close(host(y), qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))


@pytest.mark.parametrize("O,I,gs,S", [(37, 512, 64, 1), (300, 6144, 64, 4), (20, 201, 64, 2)])
def test_canaries_around_y(q, qref, O, I, gs, S):
    import torch
    d = W.gen_i4g(O, I, gs, S=S, seed=O + S)
    yv, buf, fill = guarded(torch, S * O, torch.float32)
    # inputs held in locals: a temporary's memory could be reused before the launch
    wt, sc, xt = dev(d["w"]), dev(d["scales"]), dev(d["x"])
    st = q.qgemv_i4g(wt.data_ptr(), sc.data_ptr(), xt.data_ptr(), yv.data_ptr(), S, I, O, gs,
                     torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert_guard_intact(buf, S * O, fill)
    assert_y_close(host(yv).reshape(S, O), qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))


def test_output_rows_outside_o_untouched(q):
    import torch
    d = W.gen_i4g(37, 512, 64, S=2, seed=6)
    y = torch.full((2, 37 + 64), 7.0, device="cuda")
    # write through the raw ABI into a wider buffer: rows >= O must stay 7.0
    wt, sc, xt = dev(d["w"]), dev(d["scales"]), dev(d["x"])
    st = q.qgemv_i4g(wt.data_ptr(), sc.data_ptr(), xt.data_ptr(), y.data_ptr(), 2, 512, 37, 64,
                     torch.cuda.current_stream().cuda_stream)
    assert st == 0
    flat = host(y).reshape(-1)
    assert np.all(flat[2 * 37:] == 7.0)


@pytest.mark.parametrize("O,I,S", [(2048, 2176, 1), (700, 4352, 1), (4096, 11008, 1),
                                   (300, 18944, 1), (5000, 3584, 1), (1000, 2560, 2),
                                   (513, 11008, 4)])
def test_odd_row_widths(q, qref, O, I, S):
    # rows whose chunk count no wide lane width divides (64 or 32 lanes per
    # row with idle lanes in the last sweep)
    d = W.gen_i4g(O, I, 64, S=S, seed=O + I)
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    rows = np.arange(0, O, 7) if O * I > (1 << 22) else np.arange(O)
    wr = np.ascontiguousarray(d["w"].reshape(O, -1)[rows])
    sr = np.ascontiguousarray(d["scales"].reshape(O, -1)[rows])
    ref = qref.i4g_gemv(wr, sr, d["x"], len(rows), I, 64)
    mag = magnitude(qref.i4g_dequant(wr, sr, len(rows), I, 64), d["x"])
    assert_y_close(y[:, rows], ref, mag=mag)
