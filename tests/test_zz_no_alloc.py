"""The allocation-free routed-expert entry point against the workspace one.

qgemv_moe_topk_noalloc keeps the per-token error flags in a device array of
the library instead of a caller workspace, and shares the kernels of
qgemv_moe_topk: its y must equal qgemv_moe_topk's bit for bit (and the
oracle's within the parity bar), on two calls in a row, the second with a
smaller input, and an out-of-range id must still make its token's row NaN.
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


def _both(q, d):
    import torch
    sp = torch.cuda.current_stream().cuda_stream
    w, s = dev(d["w"]), dev(d["scales"])
    ids, gates, x = dev(d["ids"]), dev(d["gates"]), dev(d["x"])
    T, K, O = d["T"], d["K"], d["O"]
    y0 = torch.full((T, O), -3.0, device="cuda")
    y1 = torch.full((T, O), -5.0, device="cuda")
    ws = q.moe_topk_workspace(T, K, O, "cuda")
    st = q.qgemv_moe_topk(w.data_ptr(), s.data_ptr(), w[0].numel(), s[0].numel(), d["E"],
                          ids.data_ptr(), gates.data_ptr(), T, K, x.data_ptr(), y0.data_ptr(),
                          d["I"], O, d["gs"], ws.data_ptr(), ws.numel(), sp)
    assert st == 0
    st = q.qgemv_moe_topk_noalloc(w.data_ptr(), s.data_ptr(), w[0].numel(), s[0].numel(),
                                  d["E"], ids.data_ptr(), gates.data_ptr(), T, K, x.data_ptr(),
                                  y1.data_ptr(), d["I"], O, d["gs"], sp)
    assert st == 0
    return host(y0), host(y1)


def test_two_calls_match_the_workspace_entry_point(q, qref):
    big = W.gen_moe(24, 512, 2048, 64, 4, 8, seed=51)
    small = W.gen_moe(10, 200, 1024, 64, 2, 3, seed=52)
    small["ids"][1, 2] = 10   # out of range: token 1's row is NaN
    for d in (big, small):
        a, b = _both(q, d)
        assert np.array_equal(np.isnan(a), np.isnan(b))
        ok = ~np.isnan(a)
        assert np.array_equal(a[ok].view(np.uint32), b[ok].view(np.uint32))
        ref = qref.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], d["E"], d["O"],
                           d["I"], d["gs"])
        assert_y_close(b, ref)
    assert np.isnan(b[1]).all() and np.isfinite(b[0]).all()


def test_refusals_before_any_launch(q):
    f = q.qgemv_moe_topk_noalloc
    BAD = 0xDEADBEEF0
    assert f(0, BAD, 1 << 20, 1 << 20, 4, BAD, BAD, 1, 1, BAD, BAD, 64, 8, 64, 0) == 1
    assert f(BAD, BAD, 1 << 20, 1 << 20, 4, BAD, BAD, 9, 1, BAD, BAD, 64, 8, 64, 0) == 2
    assert f(BAD, BAD, 1 << 20, 1 << 20, 4, BAD, BAD, 1, 1, BAD, BAD, 64, 8, 63, 0) == 3
    assert f(BAD, BAD, 1, 1, 4, BAD, BAD, 1, 1, BAD, BAD, 64, 8, 64, 0) == 6
