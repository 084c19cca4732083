"""Router top-k on the GPU against the CPU oracle, and the router feeding the
routed-expert GEMV end to end.

regolith audit "phase 0 + phase 2 m5 air validation", sections 2.1 and 2.2
(masked columns past the expert count, gates renormalised over the picks).
The picked ids must match exactly (both sides compare the same f32 logits);
the gates to 2e-6 relative (an f32 exponential and sum against f64).
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


@pytest.mark.parametrize("T,E,ld,K", [(4, 256, 512, 8), (100, 1024, 1024, 64), (1, 1, 1, 1),
                                      (33, 77, 80, 5), (7, 64, 64, 64), (2048, 256, 256, 8)])
def test_matches_oracle(q, qref, T, E, ld, K):
    lg = np.random.default_rng(T + E).standard_normal((T, ld)).astype(np.float32) * 3
    lg[:, E:] = 1e30
    ids, g = q.router_topk(dev(lg), E, K)
    rid, rg = qref.router_topk(lg, E, K)
    assert np.array_equal(host(ids), rid)
    assert np.allclose(host(g), rg, rtol=2e-6, atol=0)


def test_ties_and_quantised_logits(q, qref):
    # logits on a coarse grid: many exact ties, broken by the lower index
    T, E, K = 64, 256, 8
    lg = np.round(np.random.default_rng(5).standard_normal((T, E)) * 2).astype(np.float32)
    lg[0] = 0.0
    ids, g = q.router_topk(dev(lg), E, K)
    rid, rg = qref.router_topk(lg, E, K)
    assert np.array_equal(host(ids), rid)
    assert list(rid[0]) == list(range(8))
    assert np.allclose(host(g), rg, rtol=2e-6, atol=0)


def test_router_feeds_routed_experts(q, qref):
    # router on the GPU -> routed-expert GEMV on the GPU, against the oracle's
    # router -> the oracle's routed-expert GEMV
    E, O, I, gs, T, K = 64, 256, 2048, 64, 4, 8
    d = W.gen_moe(E, O, I, gs, T, K, seed=40)
    lg = np.random.default_rng(41).standard_normal((T, 96)).astype(np.float32)
    ids, g = q.router_topk(dev(lg), E, K)
    ws = q.moe_topk_workspace(T, K, O, "cuda")
    y = q.moe_topk(dev(d["w"]), dev(d["scales"]), ids, g, dev(d["x"]), gs, workspace=ws)
    rid, rg = qref.router_topk(lg, E, K)
    ref = qref.moe_i4g(d["w"], d["scales"], rid, rg, d["x"], E, O, I, gs)
    assert q.moe_topk_error(ws) == 0
    assert_y_close(host(y), ref)
