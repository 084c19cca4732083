"""MQ4-v2 GEMV and the FWHT-256 rotation on the GPU against the CPU oracle.

hipfire "MQ4 V2" page: sections 2 and 4 (layout, w = q*scale + zero, the half
chosen by weight index) and section 1e (a discriminating fixture).  The
rotation is the orthonormal Sylvester FWHT-256 with signs applied first
(the reading stated in the oracle); the GPU does radix-2 butterflies in f32,
so x_rot is compared with a tolerance: relative L2 <= 1e-6 per call (eight
rounding stages of 2^-24).  y: relative L2 <= 1e-5 and every element within
1e-4 of sum_i |w_i x_i|.  The streaming kernel forms sum_i w_i x_i as
scale * sum (q - 8) x + (8 scale + zero) * sum x, which rounds 8 scale + zero
once more than the definition's q * scale + zero; one-hot activations show
each recovered weight within that bound.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import (assert_bits_equal, assert_guard_intact, assert_y_close, dev, guarded, host,
                      magnitude, rel_l2, torch_cuda)
from test_oracle_mq4v2 import handbuilt_fixture

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


def test_handbuilt_fixture_decodes_exactly(q, qref):
    w, checks = handbuilt_fixture()
    got = host(q.dequant_mq4v2(dev(w.reshape(1, -1)), 512))[0]
    assert_bits_equal(got, qref.mq4v2_dequant(w, 1, 512)[0])
    for i, v in checks:
        assert got[i] == v


@pytest.mark.parametrize("O,I", [(9, 768), (64, 8192), (3, 256)])
def test_dequant_bit_exact(q, qref, O, I):
    d = W.gen_mq4v2(O, I, seed=O)
    got = host(q.dequant_mq4v2(dev(d["w"].reshape(O, -1)), I))
    assert_bits_equal(got, qref.mq4v2_dequant(d["w"], O, I))


@pytest.mark.parametrize("O,I,S", [
    (8192, 8192, 1),          # workload shape (GEMV on the rotated x)
    (256, 512, 1), (300, 1024, 2), (77, 256, 3), (1000, 4096, 4), (33, 2304, 1),
    (5, 768, 8), (1, 256, 1),
    # one vector on 14-, 12- and 8-wave tiles (ragged row counts included)
    (7000, 8192, 1), (5000, 5120, 1), (4096, 8192, 1), (2000, 7168, 1),
    # short rows: lanes per row narrowed so that a row takes two sweeps
    (3000, 1024, 1), (5000, 2048, 1), (700, 512, 1),
    # row widths no wide lane count divides: 64 or 32 lanes with idle lanes
    (500, 11008, 1), (300, 18944, 1), (1000, 3584, 2), (600, 2560, 1), (200, 4352, 4),
])
def test_gemv_matches_oracle(q, qref, O, I, S):
    d = W.gen_mq4v2(O, I, S=S, seed=O + 7)
    y = host(q.mq4v2(dev(d["w"].reshape(O, -1)), dev(d["x"])))
    mag = magnitude(qref.mq4v2_dequant(d["w"], O, I), d["x"])
    assert_y_close(y, qref.mq4v2_gemv(d["w"], d["x"], O, I), mag=mag)


def _zero_half(d, g, h):
    """Sets every row's header of group g, half h to scale 0, zero 0 (all its
    128 weights decode to 0)."""
    d["w"][:, g, 4 * h:4 * h + 4] = 0


def _unrotate(x_rot, signs, I):
    """x whose FWHT-256 pre-rotation is x_rot (the transform is its own
    inverse up to the signs): x = signs * (H256 x_rot) / 16, in f64."""
    from scipy.linalg import hadamard
    H = hadamard(256).astype(np.float64)
    xr = np.asarray(x_rot, np.float64).reshape(-1, I // 256, 256)
    return (np.einsum("ij,sbj->sbi", H, xr).reshape(-1, I) / 16.0) * signs.astype(np.float64)


@pytest.mark.parametrize("S,big,rot", [(1, 1e3, False), (1, 1e4, False), (2, 1e4, False),
                                       (1, 1e4, True), (2, 3e4, True)])
def test_outlier_on_zero_weight_column(q, qref, S, big, rot):
    # an activation big times its neighbours where every row's weights are
    # zero: y rests on the neighbours, which a fixed point sharing the
    # outlier's exponent would carry to about 2^-21 * big only
    O, I = 512, 4096
    d = W.gen_mq4v2(O, I, S=S, seed=int(big) + S)
    _zero_half(d, 3, 0)
    col = 3 * 256 + 40
    w = dev(d["w"].reshape(O, -1))
    Wd = qref.mq4v2_dequant(d["w"], O, I)
    assert np.all(Wd[:, col] == 0.0)
    if rot:
        xr = qref.fwht256(d["x"], d["signs"], I)
        xr[:, col] = big
        x = _unrotate(xr, d["signs"], I).astype(np.float32)
        xd, sg = dev(x), dev(d["signs"])
        y = host(q.mq4v2_rot(w, xd, sg))
        # the reference GEMV takes the rotation the GPU computed (qgemv_fwht256,
        # bit-identical to the fused one): an f32 rotation of a block this
        # large carries its own rounding, which the FWHT tests bound
        xr = host(q.fwht256(xd, sg))
    else:
        xr = d["x"].copy()
        xr[:, col] = big
        y = host(q.mq4v2(w, dev(xr)))
    assert np.abs(xr[:, col]).min() > 0.5 * big
    assert_y_close(y, qref.mq4v2_gemv(d["w"], xr, O, I), mag=magnitude(Wd, xr))


def test_one_hot_columns_within_two_roundings(q, qref):
    # x = e_j: y[o] = scale * (q - 8) + (8 scale + zero), rounded twice; the
    # definition rounds q * scale + zero once
    import torch
    O, I = 256, 2048
    d = W.gen_mq4v2(O, I, seed=17)
    Wd = qref.mq4v2_dequant(d["w"], O, I).astype(np.float64)
    w = dev(d["w"].reshape(O, -1))
    G = I // 256
    sc = d["sc16"].astype(np.float64)   # [O][G][2]
    zp = d["zp16"].astype(np.float64)
    for j in [0, 1, 31, 32, 127, 128, 129, 255, 256, 1000, I - 1]:
        x = torch.zeros((1, I), device="cuda")
        x[0, j] = 1.0
        got = host(q.mq4v2(w, x))[0].astype(np.float64)
        g, h = j // 256, (j % 256) // 128
        off = 8.0 * sc[:, g, h] + zp[:, g, h]
        bound = 2.0 ** -24 * (np.abs(off) + np.abs(Wd[:, j])) * 1.0000001
        assert np.all(np.abs(got - Wd[:, j]) <= bound), f"column {j}"


@pytest.mark.parametrize("rot", [False, True])
def test_canaries_around_y(q, qref, rot):
    import torch
    O, I, S = 300, 2048, 2
    d = W.gen_mq4v2(O, I, S=S, seed=31)
    yv, buf, fill = guarded(torch, S * O, torch.float32)
    w, x, sg = dev(d["w"].reshape(O, -1)), dev(d["x"]), dev(d["signs"])
    sp = torch.cuda.current_stream().cuda_stream
    if rot:
        st = q.qgemv_mq4v2_rot(w.data_ptr(), x.data_ptr(), sg.data_ptr(), yv.data_ptr(), S, I, O,
                               sp)
        xr = qref.fwht256(d["x"], d["signs"], I)
    else:
        st = q.qgemv_mq4v2(w.data_ptr(), x.data_ptr(), yv.data_ptr(), S, I, O, sp)
        xr = d["x"]
    assert st == 0
    assert_guard_intact(buf, S * O, fill)
    assert_y_close(host(yv).reshape(S, O), qref.mq4v2_gemv(d["w"], xr, O, I))


def test_fwht_canaries(q):
    import torch
    S, I = 3, 512
    x = dev(np.random.default_rng(5).standard_normal((S, I)).astype(np.float32))
    sg = dev(W.gen_fwht_signs(I))
    pad = 256
    yv, buf, fill = guarded(torch, S * I, torch.float32, pad=pad)
    st = q.qgemv_fwht256(x.data_ptr(), sg.data_ptr(), yv.data_ptr(), S, I,
                         torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert_guard_intact(buf, S * I, fill, pad=pad)


@pytest.mark.parametrize("O,I,S", [(256, 512, 1), (8192, 8192, 1), (300, 2048, 2)])
def test_infinite_activations_propagate(q, qref, O, I, S):
    # infinities give +-inf rows (NaN where two of opposite sign meet), as in
    # the plain definition
    d = W.gen_mq4v2(O, I, S=S, seed=O + S)
    d["x"][0, 37] = np.inf
    d["x"][S - 1, I - 3] = -np.inf
    y = host(q.mq4v2(dev(d["w"].reshape(O, -1)), dev(d["x"])))
    ref = qref.mq4v2_gemv(d["w"], d["x"], O, I)
    assert np.isinf(ref).any()
    assert_y_close(y, ref)


def test_nan_activation_poisons_all_rows(q):
    d = W.gen_mq4v2(40, 512, seed=4)
    d["x"][0, 300] = np.nan
    y = host(q.mq4v2(dev(d["w"].reshape(40, -1)), dev(d["x"])))
    assert np.isnan(y).all()


@pytest.mark.parametrize("O,I,S", [(512, 8192, 1), (256, 2048, 2)])
def test_wide_dynamic_range_activations(q, qref, O, I, S):
    # magnitudes over twelve decades, a zero chunk, subnormals and a value
    # 1e4 times its chunk neighbours
    d = W.gen_mq4v2(O, I, S=S, seed=5 * O + S)
    rng = np.random.default_rng(98)
    x = d["x"] * (10.0 ** rng.uniform(-6, 6, size=d["x"].shape)).astype(np.float32)
    x[:, 64:96] = 0.0
    x[:, 96:100] = np.float32(1e-40)
    x[:, 130] = 1e4 * np.abs(x[:, 131]).max() + 1.0
    d["x"] = x.astype(np.float32)
    y = host(q.mq4v2(dev(d["w"].reshape(O, -1)), dev(d["x"])))
    assert_y_close(y, qref.mq4v2_gemv(d["w"], d["x"], O, I),
                   mag=magnitude(qref.mq4v2_dequant(d["w"], O, I), d["x"]))


def test_unaligned_rows_take_general_path(q, qref):
    import torch
    O, I = 12, 512
    d = W.gen_mq4v2(O, I, seed=2)
    buf = torch.zeros(d["w"].size + 4, dtype=torch.uint8, device="cuda")
    buf[4:] = dev(d["w"].reshape(-1))
    x = dev(d["x"])
    y = torch.empty((1, O), device="cuda")
    st = q.qgemv_mq4v2(buf[4:].data_ptr(), x.data_ptr(), y.data_ptr(), 1, I, O,
                       torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert_y_close(host(y), qref.mq4v2_gemv(d["w"], d["x"], O, I))


@pytest.mark.parametrize("S,I", [(1, 8192), (3, 512), (8, 256)])
def test_fwht_matches_oracle(q, qref, S, I):
    rng = np.random.default_rng(S + I)
    x = rng.standard_normal((S, I)).astype(np.float32)
    sg = W.gen_fwht_signs(I)
    got = host(q.fwht256(dev(x), dev(sg)))
    ref = qref.fwht256(x, sg, I)
    assert rel_l2(got, ref) <= 1e-6
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.abs(ref).max()


def test_fwht_in_place(q, qref):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 512)).astype(np.float32)
    sg = W.gen_fwht_signs(512)
    xd = dev(x)
    q.fwht256(xd, dev(sg), out=xd)
    assert rel_l2(host(xd), qref.fwht256(x, sg, 512)) <= 1e-6


def test_rotate_then_gemv_end_to_end(q, qref):
    """The MQ4 workload path: x -> FWHT-256 rotation -> MQ4-v2 GEMV."""
    O, I = 2048, 8192
    d = W.gen_mq4v2(O, I, seed=0)
    xr = q.fwht256(dev(d["x"]), dev(d["signs"]))
    y = host(q.mq4v2(dev(d["w"].reshape(O, -1)), xr))
    ref = qref.mq4v2_gemv(d["w"], qref.fwht256(d["x"], d["signs"], I), O, I)
    assert_y_close(y, ref)


def _two_launch(q, w, x, signs):
    xr = q.fwht256(x, signs)
    return q.mq4v2(w, xr)


@pytest.mark.parametrize("O,I,S", [(8192, 8192, 1), (256, 512, 1), (300, 1024, 2),
                                   (77, 256, 3), (1000, 4096, 4), (33, 2304, 1), (5, 768, 6),
                                   (7000, 8192, 1), (5000, 5120, 1), (3000, 1024, 1),
                                   # two staged items per thread
                                   (1500, 16384, 1), (2000, 7168, 1), (600, 12288, 2),
                                   # odd row widths (64 or 32 lanes, idle lanes)
                                   (500, 11008, 1), (900, 3584, 1), (300, 4352, 2),
                                   # many rows: one-row tiles kept to one
                                   # workgroup per CU
                                   (18944, 3584, 1)])
def test_fused_rotation_matches_two_launches_bitwise(q, qref, O, I, S):
    # one launch == qgemv_fwht256 then qgemv_mq4v2, to the bit; and the oracle
    d = W.gen_mq4v2(O, I, S=S, seed=O + 11)
    w, x, sg = dev(d["w"].reshape(O, -1)), dev(d["x"]), dev(d["signs"])
    fused = host(q.mq4v2_rot(w, x, sg))
    two = host(_two_launch(q, w, x, sg))
    assert np.array_equal(fused.view(np.uint32), two.view(np.uint32))
    if O * I <= 1 << 22:
        ref = qref.mq4v2_gemv(d["w"], qref.fwht256(d["x"], d["signs"], I), O, I)
    else:
        rows = np.arange(0, O, 97)
        ref = qref.mq4v2_gemv(d["w"], qref.fwht256(d["x"], d["signs"], I), O, I, rows=rows)
        fused = fused[:, rows]
    assert_y_close(fused, ref)


def test_fused_rotation_non_finite_activations(q):
    # an infinity and a NaN in x: the same NaN / inf pattern and values as the
    # two-launch path
    O, I, S = 200, 2048, 2
    d = W.gen_mq4v2(O, I, S=S, seed=3)
    d["x"][0, 700] = np.inf
    d["x"][1, 5] = np.nan
    w, x, sg = dev(d["w"].reshape(O, -1)), dev(d["x"]), dev(d["signs"])
    fused = host(q.mq4v2_rot(w, x, sg))
    two = host(_two_launch(q, w, x, sg))
    assert np.array_equal(np.isnan(fused), np.isnan(two))
    ok = ~np.isnan(two)
    assert np.array_equal(fused[ok].view(np.uint32), two[ok].view(np.uint32))


def test_fused_rotation_refuses_large_i(q):
    import torch
    O, I = 4, 65536
    d = W.gen_mq4v2(O, I, seed=1)
    y = torch.empty((1, O), device="cuda")
    st = q.qgemv_mq4v2_rot(dev(d["w"]).data_ptr(), dev(d["x"]).data_ptr(),
                           dev(d["signs"]).data_ptr(), y.data_ptr(), 1, I, O,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 2
