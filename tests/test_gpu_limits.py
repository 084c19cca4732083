"""Longest rows the streaming kernels stage, and the first lengths past them.

A streaming launch stages each activation vector of the call in LDS, whose
size per workgroup bounds the row length (and, for several vectors, how
many vectors share one launch).  These cases sit at those bounds on both
sides: the last length that streams, the first that takes the general
kernel, more launches or (fp8) several column phases, each against the
oracle to the same bar as every other GEMV test (relative L2 1e-5), plus
the fused rotation's largest accepted length and its first refusal.  colibri PR #457 "metal: grouped-int4
(fmt=4) GEMV support", sections 1 and 3 (i4g); the fp8 block-scale and
MQ4-v2 layouts as in the format-specific tests.
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


# grouped int4 stages 100 B per 32 columns and vector: one vector of 49152
# columns (153.6 KiB) streams, 65536 takes the general kernel; two vectors of
# 32768 columns take one launch each, four of 16384 two launches of two
@pytest.mark.parametrize("O,I,S", [(40, 49152, 1), (40, 65536, 1), (33, 32768, 2),
                                   (33, 16384, 4)])
def test_i4g_long_rows(q, qref, O, I, S):
    d = W.gen_i4g(O, I, 64, S=S, seed=I + S)
    y = host(q.i4g(dev(d["w"]), dev(d["scales"]), dev(d["x"]), 64))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, 64))


# fp8 stages 4 B per column and vector: 36864 columns stream in one phase,
# 40960 (160 KiB plus padding) in two column phases, as do three or four
# vectors of 16384; 100000 columns take three phases of one vector
@pytest.mark.parametrize("O,I,S", [(130, 36864, 1), (130, 40960, 1), (130, 16384, 3),
                                   (200, 16384, 4), (65, 100000, 1), (129, 49152, 2)])
def test_fp8_long_rows(q, qref, O, I, S):
    d = W.gen_fp8b128(O, I, S=S, seed=I + S)
    y = host(q.fp8b128(dev(d["w"]), dev(d["scale_inv"]), dev(d["x"])))
    assert_y_close(y, qref.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I))


# MQ4-v2 on rotated activations stages 104 B per 32 columns: 49152 columns
# stream, 65536 take the general kernel (any vector stands for x_rot here)
@pytest.mark.parametrize("O,I", [(40, 49152), (40, 65536)])
def test_mq4v2_long_rows(q, qref, O, I):
    d = W.gen_mq4v2(O, I, seed=I)
    y = host(q.mq4v2(dev(d["w"].reshape(O, -1)), dev(d["x"])))
    assert_y_close(y, qref.mq4v2_gemv(d["w"], d["x"], O, I))


def test_mq4v2_rot_longest_accepted_row(q, qref):
    # the fused rotation keeps x_rot as f32 for its fallback: 40960 columns
    # (160 KiB) is the longest it takes
    O, I = 24, 40960
    d = W.gen_mq4v2(O, I, seed=5)
    y = host(q.mq4v2_rot(dev(d["w"].reshape(O, -1)), dev(d["x"]), dev(d["signs"])))
    assert_y_close(y, qref.mq4v2_gemv(d["w"], qref.fwht256(d["x"], d["signs"], I), O, I))


def test_mq4v2_rot_refuses_one_block_more(q):
    O, I = 8, 40960 + 256
    d = W.gen_mq4v2(O, I, seed=6)
    with pytest.raises(q.QgemvError):
        q.mq4v2_rot(dev(d["w"].reshape(O, -1)), dev(d["x"]), dev(d["signs"]))


def test_prefill_long_rows(q, qref):
    O, I, gs, S = 70, 49152, 64, 70
    d = W.gen_i4g(O, I, gs, S=S, seed=11)
    y = host(q.i4g_prefill(dev(d["w"]), dev(d["scales"]), dev(d["x"]), gs))
    assert_y_close(y, qref.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))


# routed experts stage one token (100 B per 32 columns) plus the partials:
# 32768 columns stream, 65536 take the general kernel
@pytest.mark.parametrize("I", [32768, 65536])
def test_moe_long_rows(q, qref, I):
    d = W.gen_moe(6, 48, I, 64, 2, 3, seed=I)
    ws = q.moe_topk_workspace(d["T"], d["K"], d["O"], "cuda")
    y = host(q.moe_topk(dev(d["w"]), dev(d["scales"]), dev(d["ids"]), dev(d["gates"]),
                        dev(d["x"]), d["gs"], workspace=ws))
    assert q.moe_topk_error(ws) == 0
    ref = qref.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], d["E"], d["O"], d["I"],
                       d["gs"])
    assert_y_close(y, ref)
