"""Routed-expert GEMV on the GPU against the CPU oracle.

y[t] = sum_k gates[t][k] * W_{ids[t][k]} x[t] over grouped-int4 experts
(regolith audit, section 2.2; colibri PR #457, section 4).  Includes the
workload shape (256 experts of 2048x7168, gs 64, 4 tokens, top-8) checked on
every row, duplicate ids, experts shared by every token (each streamed once
for all of them), K = E = 64, more tokens than one launch stages, shapes
smaller than one tile, out-of-range ids (NaN row plus the error flag, which
each call resets), one-hot activations recovering decoded weights bit for
bit, an outlier on a column whose weights are all zero, canaries around y and
the workspace, bitwise repeatability under the dynamic unit hand-out, and the
general kernel (odd I, gs not a multiple of 32).  y: relative L2 <= 1e-5 and
every element within 1e-4 of sum_k |g_k| sum_i |w_i x_i|.
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


def run(q, d):
    ws = q.moe_topk_workspace(d["T"], d["K"], d["O"], "cuda")
    y = q.moe_topk(dev(d["w"]), dev(d["scales"]), dev(d["ids"]), dev(d["gates"]), dev(d["x"]),
                   d["gs"], workspace=ws)
    return host(y), q.moe_topk_error(ws)


def oracle_y(qref, d, rows=None):
    return qref.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], d["E"], d["O"],
                        d["I"], d["gs"], rows=rows)


def moe_magnitude(qref, d):
    """sum_k |g[t][k]| sum_i |W_e[o][i] x[t][i]| (e = ids[t][k], valid ids) as f64 [T][O]."""
    T, O, I, gs = d["T"], d["O"], d["I"], d["gs"]
    mag = np.zeros((T, O))
    dec = {}
    for t in range(T):
        for k in range(d["K"]):
            e = int(d["ids"][t, k])
            if not 0 <= e < d["E"]:
                continue
            if e not in dec:
                dec[e] = np.abs(qref.i4g_dequant(d["w"][e], d["scales"][e], O, I, gs)
                                .astype(np.float64))
            mag[t] += abs(float(d["gates"][t, k])) * (dec[e] @ np.abs(d["x"][t].astype(np.float64)))
    return mag


@pytest.mark.parametrize("E,O,I,gs,T,K", [
    (16, 256, 512, 64, 4, 8), (32, 300, 1024, 64, 2, 4), (8, 77, 7168, 64, 4, 2),
    (12, 40, 256, 128, 1, 1), (64, 512, 2048, 32, 8, 8), (6, 100, 2048, 64, 3, 6),
    # short rows: 16 and 32 lanes per row instead of 64 (two- and four-sweep units)
    (8, 7168, 2048, 64, 4, 8), (12, 768, 2048, 64, 4, 8),
    # expert rows no wide lane count divides (1408, 2560 and 11008 columns)
    (16, 500, 1408, 64, 4, 8), (10, 300, 2560, 64, 2, 4), (6, 200, 11008, 64, 2, 2),
])
def test_matches_oracle(q, qref, E, O, I, gs, T, K):
    d = W.gen_moe(E, O, I, gs, T, K, seed=E + O)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d), mag=moe_magnitude(qref, d))


def test_workload_shape_every_row(q, qref):
    d = W.gen_moe(256, 2048, 7168, 64, 4, 8, seed=0)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d), mag=moe_magnitude(qref, d))


@pytest.mark.parametrize("E,O,I,T,K", [(40, 200, 7168, 8, 8), (24, 300, 2048, 8, 8),
                                       (30, 100, 7168, 6, 3)])
def test_many_tokens(q, qref, E, O, I, T, K):
    # eight tokens of 7168 columns exceed what one launch stages: token groups
    d = W.gen_moe(E, O, I, 64, T, K, seed=T + O)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d), mag=moe_magnitude(qref, d))


def test_one_hot_columns_bit_exact(q, qref):
    # K = 1, gate 1, x[t] = e_j: y[t] is column j of the selected expert,
    # (q - 8) * s with one rounding, through the streaming kernel
    E, O, I, gs, T = 6, 128, 2048, 64, 4
    d = W.gen_moe(E, O, I, gs, T, 1, seed=41)
    d["ids"][:, 0] = [3, 1, 3, 5]
    d["gates"][:] = 1.0
    cols = [0, 1, 33, 64, 1025, I - 1]
    for c0 in range(0, len(cols), T):
        cs = cols[c0:c0 + T] + [cols[0]] * (T - len(cols[c0:c0 + T]))
        d["x"][:] = 0.0
        for t, j in enumerate(cs):
            d["x"][t, j] = 1.0
        y, err = run(q, d)
        assert err == 0
        for t, j in enumerate(cs):
            e = int(d["ids"][t, 0])
            Wd = qref.i4g_dequant(d["w"][e], d["scales"][e], O, I, gs)
            assert_bits_equal(y[t], Wd[:, j])


@pytest.mark.parametrize("big", [1e3, 1e4])
def test_outlier_on_zero_weight_column(q, qref, big):
    # an activation big times its neighbours in one token, on a column whose
    # weights are zero in every expert: that token's rows rest on the
    # neighbours (per-element path); the other tokens keep the fast path
    E, O, I, gs, T, K = 12, 256, 7168, 64, 4, 4
    d = W.gen_moe(E, O, I, gs, T, K, seed=int(big))
    col = 130
    b = d["w"][:, :, col // 2]
    d["w"][:, :, col // 2] = (b & 0xF0) | 0x08
    d["x"][2, col] = big
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d), mag=moe_magnitude(qref, d))


def test_canaries_around_y_and_workspace(q, qref):
    import torch
    d = W.gen_moe(16, 200, 1024, 64, 3, 4, seed=43)
    T, K, O = d["T"], d["K"], d["O"]
    n_ws = q.qgemv_moe_topk_workspace(T, K, O)
    wsv, wsbuf, wsfill = guarded(torch, n_ws, torch.uint8)
    yv, ybuf, yfill = guarded(torch, T * O, torch.float32)
    w, s = dev(d["w"]), dev(d["scales"])
    ids, gates, x = dev(d["ids"]), dev(d["gates"]), dev(d["x"])
    st = q.qgemv_moe_topk(w.data_ptr(), s.data_ptr(), w[0].numel(), s[0].numel(), d["E"],
                          ids.data_ptr(), gates.data_ptr(), T, K, x.data_ptr(), yv.data_ptr(),
                          d["I"], O, d["gs"], wsv.data_ptr(), n_ws,
                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert_guard_intact(ybuf, T * O, yfill)
    assert_guard_intact(wsbuf, n_ws, wsfill)
    assert_y_close(host(yv).reshape(T, O), oracle_y(qref, d))


def test_duplicate_ids_count_per_occurrence(q, qref):
    d = W.gen_moe(10, 64, 512, 64, 3, 4, seed=9)
    d["ids"][1] = [5, 5, 2, 5]
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d))


def test_out_of_range_id(q, qref):
    d = W.gen_moe(10, 64, 512, 64, 3, 4, seed=10)
    d["ids"][2, 1] = 10
    y, err = run(q, d)
    assert err == 1
    assert np.isnan(y[2]).all() and np.isfinite(y[:2]).all()
    assert_y_close(y[:2], oracle_y(qref, d)[:2])


@pytest.mark.parametrize("E,O,I,gs,T,K", [(50, 50, 201, 64, 2, 40), (5, 30, 300, 16, 2, 3)])
def test_general_kernel(q, qref, E, O, I, gs, T, K):
    d = W.gen_moe(E, O, I, gs, T, K, seed=O)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d))


def test_experts_shared_by_every_token(q, qref):
    # every token selects the same experts (in its own order): each token's
    # workgroups stream them for that token
    d = W.gen_moe(20, 128, 1024, 64, 4, 6, seed=21)
    rng = np.random.default_rng(21)
    for t in range(1, 4):
        d["ids"][t] = rng.permutation(d["ids"][0])
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d))


def test_every_expert_selected(q, qref):
    # K = 64 = E: one token selects all experts
    d = W.gen_moe(64, 96, 512, 64, 1, 64, seed=22)
    d["ids"][0] = np.random.default_rng(22).permutation(64).astype(np.int32)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d))


def test_tiny_shapes(q, qref):
    # fewer rows than one wave tile, one lane chunk per row
    d = W.gen_moe(4, 3, 32, 32, 2, 2, seed=23)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d))


def test_token_with_only_bad_ids(q, qref):
    d = W.gen_moe(10, 64, 512, 64, 3, 4, seed=24)
    d["ids"][0] = [-1, 10, 11, 99]
    y, err = run(q, d)
    assert err == 1
    assert np.isnan(y[0]).all() and np.isfinite(y[1:]).all()
    assert_y_close(y[1:], oracle_y(qref, d)[1:])


def test_error_flag_is_per_call(q, qref):
    # a flagged call followed by clean calls on the same workspace, including
    # one with fewer tokens than the flagged one
    ws = q.moe_topk_workspace(8, 4, 64, "cuda")
    bad = W.gen_moe(10, 64, 512, 64, 8, 4, seed=25)
    bad["ids"][7, 3] = 12
    good = W.gen_moe(10, 64, 512, 64, 2, 4, seed=26)

    def call(d):
        y = q.moe_topk(dev(d["w"]), dev(d["scales"]), dev(d["ids"]), dev(d["gates"]),
                       dev(d["x"]), d["gs"], workspace=ws)
        return host(y), q.moe_topk_error(ws)

    assert call(bad)[1] == 1
    y, err = call(good)
    assert err == 0
    assert_y_close(y, oracle_y(qref, good))


def test_infinite_activation_in_one_token(q, qref):
    # the token with an infinity gets the plain definition's +-inf / NaN rows;
    # the other tokens are unaffected
    d = W.gen_moe(12, 256, 2048, 64, 3, 4, seed=28)
    d["x"][1, 100] = np.inf
    y, err = run(q, d)
    assert err == 0
    ref = oracle_y(qref, d)
    assert np.isinf(ref[1]).any()
    assert_y_close(y, ref)


@pytest.mark.parametrize("T", [1, 4])
def test_wide_dynamic_range_activations(q, qref, T):
    d = W.gen_moe(16, 256, 7168, 64, T, 4, seed=29 + T)
    rng = np.random.default_rng(97)
    x = d["x"] * (10.0 ** rng.uniform(-6, 6, size=d["x"].shape)).astype(np.float32)
    x[:, 64:96] = 0.0
    x[:, 130] = 1e4 * np.abs(x[:, 131]).max() + 1.0
    d["x"] = x.astype(np.float32)
    y, err = run(q, d)
    assert err == 0
    assert_y_close(y, oracle_y(qref, d), mag=moe_magnitude(qref, d))


def test_repeated_calls_are_bitwise_identical(q):
    # units are handed out dynamically; the result must not depend on which
    # wave computed which unit
    d = W.gen_moe(32, 512, 2048, 64, 4, 8, seed=27)
    a, _ = run(q, d)
    for _ in range(3):
        b, _ = run(q, d)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
