"""Canary zones around every output of the remaining C-ABI entry points.

Each output is placed inside a larger device buffer whose head and tail
hold a known pattern (inputs are held in locals for the whole call: the
memory of a temporary tensor could be handed to the next allocation); after the call the pattern must be intact and the
output must still match the oracle.  (The grouped-int4, MQ4-v2, FWHT and
routed-expert entry points have theirs next to their parity tests.)
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import (assert_bits_equal, assert_guard_intact, assert_y_close, dev, guarded, host,
                      torch_cuda)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


def _sp():
    import torch
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("ue8m0", [False, True])
@pytest.mark.parametrize("O,I,S", [(300, 2048, 1), (130, 200, 3), (200, 16384, 4)])
def test_fp8_y(q, qref, ue8m0, O, I, S):
    import torch
    d = (W.gen_fp8ue8m0 if ue8m0 else W.gen_fp8b128)(O, I, S=S, seed=O + S)
    key = "scale_e8m0" if ue8m0 else "scale_inv"
    yv, buf, fill = guarded(torch, S * O, torch.float32)
    fn = q.qgemv_fp8b128_ue8m0 if ue8m0 else q.qgemv_fp8b128
    wt, sc, xt = dev(d["w"]), dev(d[key]), dev(d["x"])
    st = fn(wt.data_ptr(), sc.data_ptr(), xt.data_ptr(), yv.data_ptr(), S, I, O, _sp())
    assert st == 0
    assert_guard_intact(buf, S * O, fill)
    ref = (qref.fp8ue8m0_gemv if ue8m0 else qref.fp8b128_gemv)(d["w"], d[key], d["x"], O, I)
    assert_y_close(host(yv).reshape(S, O), ref)


@pytest.mark.parametrize("fmt", ["v1", "c"])
def test_mq4_family_y(q, qref, fmt):
    import torch
    O, I, S = 260, 2048, 2
    d = (W.gen_mq4v1 if fmt == "v1" else W.gen_mq4c)(O, I, S=S, seed=7)
    yv, buf, fill = guarded(torch, S * O, torch.float32)
    fn = q.qgemv_mq4v1 if fmt == "v1" else q.qgemv_mq4c
    wt, xt = dev(d["w"].reshape(O, -1)), dev(d["x"])
    st = fn(wt.data_ptr(), xt.data_ptr(), yv.data_ptr(), S, I, O, _sp())
    assert st == 0
    assert_guard_intact(buf, S * O, fill)
    ref = (qref.mq4v1_gemv if fmt == "v1" else qref.mq4c_gemv)(d["w"], d["x"], O, I)
    assert_y_close(host(yv).reshape(S, O), ref)


@pytest.mark.parametrize("O,I,gs,S", [(300, 1024, 64, 100), (31, 300, 16, 9)])
def test_prefill_y(q, qref, O, I, gs, S):
    import torch
    d = W.gen_i4g(O, I, gs, S=S, seed=O + S)
    yv, buf, fill = guarded(torch, S * O, torch.float32)
    wt, sc, xt = dev(d["w"]), dev(d["scales"]), dev(d["x"])
    st = q.qgemv_i4g_prefill(wt.data_ptr(), sc.data_ptr(), xt.data_ptr(), yv.data_ptr(), S, I, O,
                             gs, _sp())
    assert st == 0
    assert_guard_intact(buf, S * O, fill)
    assert_y_close(host(yv).reshape(S, O),
                   qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))


def test_router_ids_and_gates(q, qref):
    import torch
    T, E, K = 33, 77, 5
    lg = np.random.default_rng(3).standard_normal((T, E)).astype(np.float32)
    idv, ibuf, ifill = guarded(torch, T * K, torch.int32)
    gv, gbuf, gfill = guarded(torch, T * K, torch.float32)
    lgd = dev(lg)
    st = q.qgemv_router_topk(lgd.data_ptr(), T, E, E, K, idv.data_ptr(), gv.data_ptr(), _sp())
    assert st == 0
    assert_guard_intact(ibuf, T * K, ifill)
    assert_guard_intact(gbuf, T * K, gfill)
    rid, rg = qref.router_topk(lg, E, K)
    assert np.array_equal(host(idv).reshape(T, K), rid)
    assert np.allclose(host(gv).reshape(T, K), rg, rtol=2e-6, atol=0)


def test_dequant_outputs(q, qref):
    import torch
    # grouped int4, odd I and a partial group
    O, I, gs = 37, 201, 64
    d = W.gen_i4g(O, I, gs, seed=1)
    Wv, buf, fill = guarded(torch, O * I, torch.float32)
    wt, sc = dev(d["w"]), dev(d["scales"])
    assert q.qgemv_dequant_i4g(wt.data_ptr(), sc.data_ptr(), Wv.data_ptr(), I, O, gs, _sp()) == 0
    assert_guard_intact(buf, O * I, fill)
    assert_bits_equal(host(Wv).reshape(O, I), qref.i4g_dequant(d["w"], d["scales"], O, I, gs))
    # fp8, both scale kinds, partial blocks
    O, I = 130, 200
    for ue8m0 in (False, True):
        d = (W.gen_fp8ue8m0 if ue8m0 else W.gen_fp8b128)(O, I, seed=2)
        key = "scale_e8m0" if ue8m0 else "scale_inv"
        fn = q.qgemv_dequant_fp8b128_ue8m0 if ue8m0 else q.qgemv_dequant_fp8b128
        Wv, buf, fill = guarded(torch, O * I, torch.float32)
        wt, sc = dev(d["w"]), dev(d[key])
        assert fn(wt.data_ptr(), sc.data_ptr(), Wv.data_ptr(), I, O, _sp()) == 0
        assert_guard_intact(buf, O * I, fill)
        ref = (qref.fp8ue8m0_dequant if ue8m0 else qref.fp8b128_dequant)(d["w"], d[key], O, I)
        assert_bits_equal(host(Wv).reshape(O, I), ref)
    # the three MQ4 header formats
    O, I = 9, 768
    for gen, fn, rf in ((W.gen_mq4v2, q.qgemv_dequant_mq4v2, qref.mq4v2_dequant),
                        (W.gen_mq4v1, q.qgemv_dequant_mq4v1, qref.mq4v1_dequant),
                        (W.gen_mq4c, q.qgemv_dequant_mq4c, qref.mq4c_dequant)):
        d = gen(O, I, seed=3)
        Wv, buf, fill = guarded(torch, O * I, torch.float32)
        wt = dev(d["w"].reshape(O, -1))
        assert fn(wt.data_ptr(), Wv.data_ptr(), I, O, _sp()) == 0
        assert_guard_intact(buf, O * I, fill)
        assert_bits_equal(host(Wv).reshape(O, I), rf(d["w"], O, I))


def test_encoder_output(q, qref):
    import torch
    O, I = 5, 768
    Wt = W.gen_rotated_weights(O, I, seed=4)
    n = O * (I // 256) * 136
    ov, buf, fill = guarded(torch, n, torch.uint8)
    Wd = dev(Wt)
    assert q.qgemv_mq4v2_encode(Wd.data_ptr(), ov.data_ptr(), I, O, _sp()) == 0
    assert_guard_intact(buf, n, fill)
    assert np.array_equal(host(ov).reshape(O, -1), qref.mq4v2_encode(Wt, O, I).reshape(O, -1))
