"""fp8-e4m3 GEMV with UE8M0 block scales on the GPU against the CPU oracle.

colibri PR #528 "fmt=7: fp8-e4m3-b128 passthrough weight format", section
"Design" (the same 128x128 block geometry with one power-of-two scale byte
per block, dtype F8_E8M0; decode 2^(e - 127), 255 = NaN as the oracle reads
it).  Decoded weights must match bit for bit; y to relative L2 <= 1e-5; and
y equals the f32-scale kernel fed with the decoded scales bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bits_equal, assert_y_close, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


def e8m0_f32(se):
    e = se.astype(np.uint32)
    v = (e << 23).view(np.float32).copy()
    v[e == 0] = np.float32(2.0 ** -127)
    v[e == 255] = np.nan
    return v


@pytest.mark.parametrize("O,I", [(130, 200), (129, 128), (128, 129), (1, 1), (384, 6144)])
def test_dequant_bit_exact(q, qref, O, I):
    d = W.gen_fp8ue8m0(O, I, seed=O + I)
    got = host(q.dequant_fp8b128_ue8m0(dev(d["w"]), dev(d["scale_e8m0"])))
    assert_bits_equal(got, qref.fp8ue8m0_dequant(d["w"], d["scale_e8m0"], O, I))


def test_dequant_extreme_scales(q, qref):
    # exponent bytes 0 (2^-127, an f32 subnormal), 254 (overflow to inf for
    # large codes) and 255 (NaN) in different blocks
    O, I = 256, 384
    d = W.gen_fp8ue8m0(O, I, seed=9)
    d["scale_e8m0"][0, 0] = 0
    d["scale_e8m0"][0, 1] = 254
    d["scale_e8m0"][1, 2] = 255
    got = host(q.dequant_fp8b128_ue8m0(dev(d["w"]), dev(d["scale_e8m0"])))
    assert_bits_equal(got, qref.fp8ue8m0_dequant(d["w"], d["scale_e8m0"], O, I))


@pytest.mark.parametrize("O,I,S", [
    (130, 200, 1), (129, 128, 2), (384, 6144, 1), (2048, 6144, 4), (300, 16384, 4),
    (77, 100, 3), (1, 1, 1), (50, 512, 8),
])
def test_gemv_matches_oracle(q, qref, O, I, S):
    d = W.gen_fp8ue8m0(O, I, S=S, seed=3 * O + I)
    y = host(q.fp8b128_ue8m0(dev(d["w"]), dev(d["scale_e8m0"]), dev(d["x"])))
    assert_y_close(y, qref.fp8ue8m0_gemv(d["w"], d["scale_e8m0"], d["x"], O, I))


def test_workload_shape_sampled_rows(q, qref):
    O, I = 7168, 16384
    d = W.gen_fp8ue8m0(O, I, seed=0)
    y = host(q.fp8b128_ue8m0(dev(d["w"]), dev(d["scale_e8m0"]), dev(d["x"])))
    rows = np.concatenate([np.arange(0, O, 61), [O - 1]])
    assert_y_close(y[:, rows], qref.fp8ue8m0_gemv(d["w"], d["scale_e8m0"], d["x"], O, I, rows=rows))


@pytest.mark.parametrize("O,I,S", [(7168, 16384, 1), (300, 16384, 2), (77, 100, 1)])
def test_equals_f32_scale_kernel_bitwise(q, O, I, S):
    d = W.gen_fp8ue8m0(O, I, S=S, seed=O)
    a = host(q.fp8b128_ue8m0(dev(d["w"]), dev(d["scale_e8m0"]), dev(d["x"])))
    b = host(q.fp8b128(dev(d["w"]), dev(e8m0_f32(d["scale_e8m0"])), dev(d["x"])))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_nan_scale_byte_poisons_its_band(q):
    O, I = 300, 512
    d = W.gen_fp8ue8m0(O, I, seed=12)
    d["scale_e8m0"][1, 3] = 255          # rows 128..255
    y = host(q.fp8b128_ue8m0(dev(d["w"]), dev(d["scale_e8m0"]), dev(d["x"])))[0]
    assert np.isnan(y[128:256]).all() and np.isfinite(y[:128]).all() and np.isfinite(y[256:]).all()
