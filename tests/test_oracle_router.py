"""Pins for the router top-k oracle.

regolith audit "phase 0 + phase 2 m5 air validation", section 2.1 (columns at
or past n_expert are masked out of the softmax; the logits row stride may be
larger than n_expert) and section 2.2 (the gates are the picked experts'
probabilities renormalised over the picked set).  Ties rank by the lower
expert index (the reading the oracle states).
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


@pytest.fixture(scope="module")
def o():
    return oracle.load()


def pin_against_library(o, T=16, E=256, ld=512, K=8, seed=0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, ld)).astype(np.float32)
    lg[:, E:] = 1e30                          # masked columns must not matter
    ids, g = o.router_topk(lg, E, K)
    ref_ids = np.argsort(-lg[:, :E], axis=1, kind="stable")[:, :K]
    full = softmax(lg[:, :E].astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ref_ids, axis=1)
    ref_g = sel / sel.sum(1, keepdims=True)
    return np.array_equal(ids, ref_ids) and np.allclose(g, ref_g, rtol=1e-6, atol=0)


def pin_ties(o):
    lg = np.zeros((2, 64), np.float32)
    lg[1, [3, 9, 40]] = 2.0
    ids, g = o.router_topk(lg, 64, 5)
    return (list(ids[0]) == [0, 1, 2, 3, 4] and np.allclose(g[0], 0.2)
            and list(ids[1]) == [3, 9, 40, 0, 1])


def pin_all_experts(o, T=3, E=64, seed=1):
    lg = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    ids, g = o.router_topk(lg, E, E)
    full = softmax(lg.astype(np.float64), axis=1)
    return np.allclose(g, np.take_along_axis(full, ids, axis=1), rtol=1e-6) and \
        np.allclose(g.sum(1), 1.0, atol=1e-6)


def run_pins(o):
    return {"library": pin_against_library(o), "ties": pin_ties(o), "all": pin_all_experts(o)}


def test_pins_hold(o):
    r = run_pins(o)
    assert all(r.values()), r


def test_planted_router_mistake_is_caught(mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(14, mutant_dir))
    assert m.mutation == 14
    r = run_pins(m)
    assert not all(r.values()), r
