"""Many-token grouped-int4 product (MFMA prefill) on the GPU against the oracle.

colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV support", sections 1 and 3:
the same y = W x as the GEMV, for many tokens at once.  y to relative L2
<= 1e-5 (f32 operands and accumulation on the matrix cores).
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_y_close, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


@pytest.mark.parametrize("O,I,gs,S", [
    (256, 512, 64, 64), (300, 1024, 64, 100), (77, 2048, 128, 17), (64, 256, 32, 1),
    (1000, 4096, 64, 130), (5, 64, 64, 3),
    (200, 200, 64, 40), (31, 300, 16, 9),          # shapes the tiles do not take
])
def test_matches_oracle(q, qref, O, I, gs, S):
    d = W.gen_i4g(O, I, gs, S=S, seed=O + S)
    y = host(q.i4g_prefill(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))


def test_workload_shape_sampled_rows(q, qref):
    O, I, gs, S = 12288, 6144, 64, 256
    d = W.gen_i4g(O, I, gs, S=S, seed=3)
    y = host(q.i4g_prefill(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    rows = np.concatenate([np.arange(0, O, 251), [O - 1]])
    assert_y_close(y[:, rows], qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs, rows=rows))


def test_agrees_with_gemv(q):
    # the GEMV on the same tokens, four at a time: same values within f32 rounding
    O, I, gs, S = 512, 2048, 64, 32
    d = W.gen_i4g(O, I, gs, S=S, seed=9)
    a = host(q.i4g_prefill(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    b = np.concatenate([host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"][s:s + 4]), gs))
                        for s in range(0, S, 4)])
    assert_y_close(a, b.astype(np.float64))


def test_non_finite_activation(q, qref):
    O, I, gs, S = 100, 512, 64, 20
    d = W.gen_i4g(O, I, gs, S=S, seed=10)
    d["x"][3, 17] = np.inf
    d["x"][7, 100] = np.nan
    y = host(q.i4g_prefill(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))
