"""Pins for the MQ4-v2 oracle (hipfire "MQ4 V2" page).

Section 2 (136 B per 256 weights, little-endian, payload at bytes 8..135),
section 3 (degenerate constant half: scale 0, the decoder reproduces the zero
exactly), section 4 (w = q * scale[h] + zero[h]; h comes from the weight's
index, weights >= 128 use the second header dword) and section 1e (a
discriminating fixture catches a wrong payload offset or stride).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from conftest import golden_lines, unpack_nibbles


def handbuilt_fixture():
    """Bytes built straight from the page's layout statement (not workloads)."""
    groups, checks = [], []
    for p in golden_lines("mq4v2_handbuilt.txt"):
        if p[0] == "group":
            groups.append(p)
        elif p[0] == "check":
            checks.append((int(p[1]), float(p[2])))
    row = bytearray()
    for p in groups:
        sc0, zp0, sc1, zp1 = (int(h, 16) for h in p[2:6])
        hdr0 = sc0 | (zp0 << 16)
        hdr1 = sc1 | (zp1 << 16)
        row += hdr0.to_bytes(4, "little") + hdr1.to_bytes(4, "little")
        q = [(j % 16) if p[6] == "up" else 15 - (j % 16) for j in range(256)]
        row += bytes(q[2 * k] | (q[2 * k + 1] << 4) for k in range(128))
    return np.frombuffer(bytes(row), np.uint8).copy(), checks


def pin_handbuilt(o):
    w, checks = handbuilt_fixture()
    if w.size != 2 * 136:
        return False
    Wd = o.mq4v2_dequant(w, 1, 512)[0]
    return all(Wd[i] == v for i, v in checks)


def dense_from_draws(d):
    O, I = d["O"], d["I"]
    G = I // 256
    q = unpack_nibbles(d["w"][:, :, 8:], 256)                      # [O][G][256]
    half = (np.arange(256) >= 128).astype(int)
    sc = d["sc16"].astype(np.float64)[:, :, half]
    zp = d["zp16"].astype(np.float64)[:, :, half]
    return (q * sc + zp).reshape(O, G * 256)


def pin_dequant_draws(o, O=9, I=768, seed=2):
    d = W.gen_mq4v2(O, I, seed=seed)
    return np.array_equal(o.mq4v2_dequant(d["w"], O, I).view(np.uint32),
                          dense_from_draws(d).astype(np.float32).view(np.uint32))


def pin_brute_force(o, O=17, I=1024, S=2, seed=3):
    d = W.gen_mq4v2(O, I, S=S, seed=seed)
    yref = d["x"].astype(np.float64) @ dense_from_draws(d).T
    y = o.mq4v2_gemv(d["w"], d["x"], O, I)
    return np.allclose(y, yref, rtol=1e-6, atol=1e-6 * np.abs(yref).max())


def run_pins(o):
    return {"handbuilt": pin_handbuilt(o), "dequant": pin_dequant_draws(o),
            "brute": pin_brute_force(o)}


def test_pins_hold(qref):
    r = run_pins(qref)
    assert all(r.values()), r


def test_byte_geometry():
    d = W.gen_mq4v2(3, 512)
    assert d["w"].nbytes == 3 * (512 // 256) * 136
    hb, _ = handbuilt_fixture()
    # the generator places headers the way the hand-built fixture does
    assert np.array_equal(d["w"][0, 0, 0:2].view("<f2")[0], d["sc16"][0, 0, 0])
    assert np.array_equal(d["w"][0, 0, 6:8].view("<f2")[0], d["zp16"][0, 0, 1])


def test_degenerate_half_reproduces_zero(qref):
    w, _ = handbuilt_fixture()
    w = w.copy()
    w[0:2] = [0, 0]            # group 0 half 0 scale = +0.0
    Wd = qref.mq4v2_dequant(w, 1, 512)[0]
    assert np.all(Wd[:128] == -2.0)


@pytest.mark.parametrize("n", [7, 8])
def test_planted_mq4_mistakes_are_caught(n, mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(n, mutant_dir))
    r = run_pins(m)
    assert not all(r.values()), r
