"""Pins for the FWHT-256 rotation oracle and the routed-expert oracle.

FWHT: hipfire "MQ4 V2" page, section 1 (weights are FWHT-256 rotated with
per-element signs before quantising; MQ denotes the rotated line).  Reading
where the page is silent: orthonormal 1/16 scaling, signs applied before the
transform, Sylvester (natural) ordering -- pinned here against SciPy's
Hadamard matrix, the identity H.e0 = (1/16) 1, the involution H.H = I and
norm preservation.

Routed experts: regolith audit "phase 0 + phase 2 m5 air validation",
section 2.2 (gates are the selection probabilities renormalised over the
selected experts) with grouped-int4 experts (colibri PR #457, section 4).
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads as W
from conftest import unpack_nibbles


def pin_scipy_hadamard(o, S=2, I=512, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((S, I)).astype(np.float32)
    sg = W.gen_fwht_signs(I)
    H = scipy.linalg.hadamard(256).astype(np.float64)
    ref = np.concatenate([(H @ (sg[b * 256:(b + 1) * 256] * x[:, b * 256:(b + 1) * 256].astype(np.float64)).T).T
                          for b in range(I // 256)], axis=1) / 16.0
    got = o.fwht256(x, sg, I)
    return np.allclose(got, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def pin_unit_vector(o):
    x = np.zeros(256, np.float32)
    x[0] = 1.0
    got = o.fwht256(x, np.ones(256, np.int8), 256)[0]
    return bool(np.all(got == np.float32(1.0 / 16.0)))


def pin_involution_and_norm(o, seed=1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(768).astype(np.float32)
    ones = np.ones(768, np.int8)
    y = o.fwht256(x, ones, 768)[0]
    z = o.fwht256(y, ones, 768)[0]
    ok_norm = all(abs(np.linalg.norm(y[b:b + 256].astype(np.float64)) -
                      np.linalg.norm(x[b:b + 256].astype(np.float64))) < 1e-5
                  for b in range(0, 768, 256))
    return bool(np.allclose(z, x, atol=2e-6) and ok_norm)


def pin_signs_first(o, seed=2):
    # H.(s.x) differs from s.(H.x); with s = -1 on one element only the former
    # changes every output.
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(256).astype(np.float32)
    s = np.ones(256, np.int8)
    s[5] = -1
    a = o.fwht256(x, s, 256)[0].astype(np.float64)
    b = o.fwht256(x, np.ones(256, np.int8), 256)[0].astype(np.float64)
    H = scipy.linalg.hadamard(256)
    return bool(np.allclose(a - b, -2.0 * x[5] * H[:, 5] / 16.0, atol=1e-6))


def fwht_pins(o):
    return {"scipy": pin_scipy_hadamard(o), "e0": pin_unit_vector(o),
            "inv": pin_involution_and_norm(o), "signs": pin_signs_first(o)}


def test_fwht_pins_hold(qref):
    r = fwht_pins(qref)
    assert all(r.values()), r


def test_planted_fwht_mistake_is_caught(mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(9, mutant_dir))
    r = fwht_pins(m)
    assert not all(r.values()), r


# --------------------------------------------------------------------------
def moe_dense_ref(d):
    E, O, I, gs = d["E"], d["O"], d["I"], d["gs"]
    T, K = d["ids"].shape
    y = np.zeros((T, O))
    for t in range(T):
        for k in range(K):
            e = d["ids"][t, k]
            q = unpack_nibbles(d["w"][e], I)
            s = np.repeat(d["scales"][e].astype(np.float64), gs, axis=1)[:, :I]
            y[t] += float(d["gates"][t, k]) * (((q - 8) * s) @ d["x"][t].astype(np.float64))
    return y


def small_moe(seed=0, E=12, O=40, I=256, gs=64, T=4, K=3):
    return W.gen_moe(E, O, I, gs, T, K, seed=seed)


def pin_moe_brute(o):
    d = small_moe()
    y = o.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], d["E"], d["O"], d["I"], d["gs"])
    ref = moe_dense_ref(d)
    return np.allclose(y, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def pin_moe_single_expert(o):
    d = small_moe(seed=1, K=1)
    d["gates"][:] = 1.0
    y = o.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], d["E"], d["O"], d["I"], d["gs"])
    ok = True
    for t in range(d["T"]):
        e = d["ids"][t, 0]
        yt = o.i4g_gemv(d["w"][e], d["scales"][e], d["x"][t], d["O"], d["I"], d["gs"])[0]
        ok &= np.array_equal(y[t], yt)
    return bool(ok)


def moe_pins(o):
    return {"brute": pin_moe_brute(o), "single": pin_moe_single_expert(o)}


def test_moe_pins_hold(qref):
    r = moe_pins(qref)
    assert all(r.values()), r


def test_moe_permutation_invariance(qref):
    d = small_moe(seed=2, K=4)
    args = (d["E"], d["O"], d["I"], d["gs"])
    y0 = qref.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], *args)
    p = np.array([2, 0, 3, 1])
    y1 = qref.moe_i4g(d["w"], d["scales"], d["ids"][:, p], d["gates"][:, p], d["x"], *args)
    assert np.allclose(y0, y1, rtol=1e-6, atol=1e-7)


def test_moe_out_of_range_id_gives_nan_row(qref):
    d = small_moe(seed=3)
    d["ids"][1, 2] = d["E"]
    y = qref.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], d["E"], d["O"], d["I"], d["gs"])
    assert np.isnan(y[1]).all() and np.isfinite(np.delete(y, 1, axis=0)).all()


def test_moe_routing_recipe():
    ids, gates = W.gen_moe_routing(256, 4, 8, seed=0)
    assert ids.shape == (4, 8) and all(len(set(r)) == 8 for r in ids.tolist())
    assert ids.min() >= 0 and ids.max() < 256
    assert np.allclose(gates.sum(axis=1), 1.0, atol=1e-6) and (gates > 0).all()


def test_planted_moe_mistake_is_caught(mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(10, mutant_dir))
    r = moe_pins(m)
    assert not all(r.values()), r
