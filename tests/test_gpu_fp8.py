"""fp8-e4m3 128x128-block GEMV on the GPU against the CPU oracle.

colibri PR #528 "fmt=7: fp8-e4m3-b128 passthrough weight format", section
"Metal validation record": all 256 codes through the GPU decoder, block
edges 130x200 / 129x128 / 128x129, 1x1, the 3x48 block-grid stride audit
(384x6144), the [2048,6144] / [6144,2048] projections at S = 1 and S = 4,
the 130x130 partial-block tensor at all 16,900 positions, NaN rows.  y:
relative L2 <= 1e-5 and every element within 1e-4 of sum_i |w_i x_i|.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bits_equal, assert_y_close, dev, host, magnitude, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


def test_all_256_codes_decode_exactly(q, qref):
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    sc = np.ones((1, 1), np.float32)
    got = host(q.dequant_fp8b128(dev(codes), dev(sc)))
    assert_bits_equal(got, qref.fp8b128_dequant(codes, sc, 2, 128))


@pytest.mark.parametrize("O,I", [(130, 130), (130, 200), (384, 6144), (1, 1), (257, 129)])
def test_dequant_bit_exact(q, qref, O, I):
    d = W.gen_fp8b128(O, I, seed=O + I)
    got = host(q.dequant_fp8b128(dev(d["w"]), dev(d["scale_inv"])))
    assert_bits_equal(got, qref.fp8b128_dequant(d["w"], d["scale_inv"], O, I))


@pytest.mark.parametrize("O,I,S", [
    (7168, 16384, 1),         # workload shape
    (2048, 6144, 1), (2048, 6144, 4), (6144, 2048, 1), (384, 6144, 3),
    (130, 200, 2), (129, 128, 1), (128, 129, 1), (1, 1, 1), (300, 2048, 2),
    (77, 16, 1), (64, 4096, 8),
    # one vector on eight-wave tiles: two rows per lane group (4096, ragged
    # 4001 rows) and one (2048 x 6144 above, ragged 2047 rows)
    (4096, 7168, 1), (4001, 4096, 1), (2047, 16384, 1),
    # short rows: lanes per row narrowed to 16 and 8 (three or more sweeps)
    (3000, 1024, 1), (1000, 512, 1), (5000, 2048, 1),
    # several vectors whose activations do not all fit the LDS: column phases
    (300, 16384, 4), (7168, 16384, 2),
])
def test_gemv_matches_oracle(q, qref, O, I, S):
    d = W.gen_fp8b128(O, I, S=S, seed=3 * O + I)
    y = host(q.fp8b128(dev(d["w"]), dev(d["scale_inv"]), dev(d["x"])))
    mag = magnitude(qref.fp8b128_dequant(d["w"], d["scale_inv"], O, I), d["x"])
    assert_y_close(y, qref.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I), mag=mag)


@pytest.mark.parametrize("I", [2048, 200])
def test_nan_code_poisons_only_its_row(q, qref, I):
    d = W.gen_fp8b128(300, I, seed=5)
    d["w"][7, 11] = 0x7F
    d["w"][260, I - 1] = 0xFF
    y = host(q.fp8b128(dev(d["w"]), dev(d["scale_inv"]), dev(d["x"])))
    assert_y_close(y, qref.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], 300, I))
    assert np.isnan(y[0, 7]) and np.isnan(y[0, 260]) and np.isfinite(np.delete(y[0], [7, 260])).all()


def test_every_column_of_a_chunk(q, qref):
    """One-hot activations read single weight columns back: covers every
    position inside the 16-column lane chunks and several 128-column blocks.
    Compared by value: a -0 weight gives +0 once summed from +0 (IEEE)."""
    import torch
    O, I = 256, 2048
    d = W.gen_fp8b128(O, I, seed=1)
    Wd = qref.fp8b128_dequant(d["w"], d["scale_inv"], O, I)
    wt, st = dev(d["w"]), dev(d["scale_inv"])
    for j in list(range(32)) + [127, 128, 129, 1023, 1024, 2047]:
        x = torch.zeros((1, I), device="cuda")
        x[0, j] = 1.0
        got = host(q.fp8b128(wt, st, x))[0]
        assert np.array_equal(got, Wd[:, j]), f"column {j}"


@pytest.mark.parametrize("O,I,S", [(700, 11008, 1), (300, 4352, 1), (1000, 2176, 1),
                                   (257, 11008, 3)])
def test_odd_row_widths(q, qref, O, I, S):
    # row widths whose chunk counts no wide lane count divides
    d = W.gen_fp8b128(O, I, S=S, seed=O + I)
    y = host(q.fp8b128(dev(d["w"]), dev(d["scale_inv"]), dev(d["x"])))
    mag = magnitude(qref.fp8b128_dequant(d["w"], d["scale_inv"], O, I), d["x"])
    assert_y_close(y, qref.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I), mag=mag)
