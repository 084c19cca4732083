"""Pins for the MQ4 family around v2 in the oracle.

hipfire "MQ4 V2": section 1b (MQ4C pad, qt=45: fp16 header at +0, 136-byte
geometry of v1), section 1e (v1 reads two f32 fields; all three keep the 128
payload bytes at [8..136); equal half headers make v2 numerically identical
to v1 on the same nibbles), section 3 (the encoder: min/max per 128-weight
half, step = (hi - lo)/15 in f32, fp16 header, codes chosen against the
round-tripped header, constant half -> scale 0), section 4 (w = q*scale + zero).
"""
import numpy as np
import pytest

import oracle
import workloads as W


@pytest.fixture(scope="module")
def o():
    return oracle.load()


def unpack_q(w, O, I):
    pay = w.reshape(O, I // 256, 136)[:, :, 8:]
    q = np.empty((O, I // 256, 256), np.int64)
    q[:, :, 0::2] = pay & 0xF
    q[:, :, 1::2] = pay >> 4
    return q.reshape(O, I)


# -- decoders ------------------------------------------------------------------
def pin_v1_brute(o, O=9, I=768, S=2, seed=1):
    d = W.gen_mq4v1(O, I, S=S, seed=seed)
    q = unpack_q(d["w"], O, I)
    sc = np.repeat(d["sc"].astype(np.float64), 256, 1)
    zp = np.repeat(d["zp"].astype(np.float64), 256, 1)
    dense = q * sc + zp
    ok = np.array_equal(o.mq4v1_dequant(d["w"], O, I).view(np.uint32),
                        dense.astype(np.float32).view(np.uint32))
    y = o.mq4v1_gemv(d["w"], d["x"], O, I)
    yref = d["x"].astype(np.float64) @ dense.T
    return ok and np.allclose(y, yref, rtol=1e-6, atol=1e-7 * np.abs(yref).max())


def pin_c_brute(o, O=9, I=768, S=2, seed=2):
    d = W.gen_mq4c(O, I, S=S, seed=seed)
    q = unpack_q(d["w"], O, I)
    sc = np.repeat(d["sc16"].astype(np.float64), 256, 1)
    zp = np.repeat(d["zp16"].astype(np.float64), 256, 1)
    dense = q * sc + zp
    ok = np.array_equal(o.mq4c_dequant(d["w"], O, I).view(np.uint32),
                        dense.astype(np.float32).view(np.uint32))
    y = o.mq4c_gemv(d["w"], d["x"], O, I)
    yref = d["x"].astype(np.float64) @ dense.T
    return ok and np.allclose(y, yref, rtol=1e-6, atol=1e-7 * np.abs(yref).max())


def pin_c_pad_ignored(o, O=4, I=512, seed=3):
    d = W.gen_mq4c(O, I, seed=seed)
    w2 = d["w"].copy()
    w2[:, :, 4:8] = 0xA5
    return np.array_equal(o.mq4c_dequant(d["w"], O, I), o.mq4c_dequant(w2, O, I))


def v2_with_equal_halves(O, I, seed):
    d = W.gen_mq4v2(O, I, seed=seed)
    w = d["w"].reshape(O, I // 256, 136).copy()
    w[:, :, 4:8] = w[:, :, 0:4]             # half 1 header := half 0 header
    return d, w


def pin_v2_equals_v1_and_c(o, O=7, I=1024, seed=4):
    # equal half headers: v2 == v1 (f32 header = the fp16 values) == MQ4C
    d, w2 = v2_with_equal_halves(O, I, seed)
    hdr = w2[:, :, 0:4].copy().view("<u2").reshape(O, I // 256, 2)
    sc = hdr[:, :, 0].view(np.float16).astype(np.float32)
    zp = hdr[:, :, 1].view(np.float16).astype(np.float32)
    w1 = w2.copy()
    w1[:, :, 0:4] = sc.astype("<f4").view(np.uint8).reshape(O, I // 256, 4)
    w1[:, :, 4:8] = zp.astype("<f4").view(np.uint8).reshape(O, I // 256, 4)
    wc = w2.copy()
    wc[:, :, 4:8] = 0
    a = o.mq4v2_dequant(w2, O, I)
    b = o.mq4v1_dequant(w1, O, I)
    c = o.mq4c_dequant(wc, O, I)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32)) and \
        np.array_equal(a.view(np.uint32), c.view(np.uint32))


def pin_v1_fixture(o):
    # one group: scale 0.25, zero -1.5 as f32, payload nibble j = j mod 16
    w = np.zeros((1, 136), np.uint8)
    w[0, 0:4] = np.array([0.25], "<f4").view(np.uint8)
    w[0, 4:8] = np.array([-1.5], "<f4").view(np.uint8)
    j = np.arange(256)
    q = j % 16
    w[0, 8:] = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)
    got = o.mq4v1_dequant(w, 1, 256)[0]
    return np.array_equal(got, (q * 0.25 - 1.5).astype(np.float32))


# -- encoder -------------------------------------------------------------------
def decode_v2(o, w, O, I):
    return o.mq4v2_dequant(w, O, I)


def pin_encoder_exact_grid(o):
    # a half on an fp16-exact grid lo + k*step: codes k, exact reconstruction
    O, I = 2, 256
    Wt = np.zeros((O, I), np.float32)
    k = np.arange(128) % 16
    k[0], k[1] = 0, 15                      # both extremes present
    Wt[0, :128] = -0.5 + k * 2.0 ** -6
    Wt[0, 128:] = 0.25 + (15 - k) * 2.0 ** -8
    Wt[1, :128] = 0.125                     # constant half: scale 0, q 0
    Wt[1, 128:] = -3.0 + k * 2.0 ** -2
    enc = o.mq4v2_encode(Wt, O, I)
    ok = np.array_equal(decode_v2(o, enc, O, I), Wt)
    hd = enc[1, 0:4].view("<u2")
    ok &= hd[0] == 0 and hd[1] == np.float16(0.125).view(np.uint16)
    ok &= np.all(unpack_q(enc, O, I)[1, :128] == 0)
    ok &= np.array_equal(unpack_q(enc, O, I)[0, :128], k)
    return bool(ok)


def pin_encoder_codes_minimize_error(o, O=16, I=1024, seed=5):
    # every code is the nearest of the 16 levels of its stored header
    Wt = W.gen_rotated_weights(O, I, seed=seed)
    enc = o.mq4v2_encode(Wt, O, I)
    q = unpack_q(enc, O, I).reshape(O, I // 256, 2, 128)
    hdr = enc.reshape(O, I // 256, 136)[:, :, 0:8].copy().view("<u2").reshape(O, I // 256, 2, 2)
    st = hdr[..., 0].view(np.float16).astype(np.float32)[..., None]
    z = hdr[..., 1].view(np.float16).astype(np.float32)[..., None]
    w = Wt.reshape(O, I // 256, 2, 128)
    levels = np.arange(16, dtype=np.float32)[:, None, None, None, None] * st + z
    err = np.abs(w[None] - levels)
    best = err.min(axis=0)
    chosen = np.take_along_axis(err, q[None], axis=0)[0]
    # rint in f32 may pick either neighbour within an f32 rounding of a tie
    return bool(np.all(chosen <= best + 4e-7 * np.abs(st)))


def pin_encoder_halves_and_headers(o, O=8, I=512, seed=6):
    # header h describes exactly the min / max of half h (up to fp16 rounding)
    Wt = W.gen_rotated_weights(O, I, seed=seed)
    enc = o.mq4v2_encode(Wt, O, I)
    hdr = enc.reshape(O, I // 256, 136)[:, :, 0:8].copy().view("<u2").reshape(O, I // 256, 2, 2)
    w = Wt.reshape(O, I // 256, 2, 128).astype(np.float64)
    lo, hi = w.min(-1), w.max(-1)
    z = hdr[..., 1].view(np.float16).astype(np.float64)
    st = hdr[..., 0].view(np.float16).astype(np.float64)
    ok_z = np.all(np.abs(z - lo) <= 2.0 ** -11 * np.abs(lo) + 1e-12)
    ok_s = np.all(np.abs(st - (hi - lo) / 15) <= 2.0 ** -11 * (hi - lo) / 15 + 1e-12)
    return bool(ok_z and ok_s)


def run_pins(o):
    return {"v1_brute": pin_v1_brute(o), "c_brute": pin_c_brute(o), "c_pad": pin_c_pad_ignored(o),
            "v2_eq": pin_v2_equals_v1_and_c(o), "v1_fixture": pin_v1_fixture(o),
            "enc_grid": pin_encoder_exact_grid(o), "enc_min": pin_encoder_codes_minimize_error(o),
            "enc_hdr": pin_encoder_halves_and_headers(o)}


def test_pins_hold(o):
    r = run_pins(o)
    assert all(r.values()), r


def test_f16_rounding_matches_numpy(o):
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 6, 20000)).astype(np.float32)
    v = np.concatenate([v, np.array([0.0, -0.0, 65504, 65519.99, 65520, 6e-8, 2.98e-8,
                                     np.inf, -np.inf], np.float32)])
    got = np.array([o.f32_to_f16(float(f)) for f in v], np.uint16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("n", [12, 13])
def test_planted_mq4_family_mistakes_are_caught(n, mutant_dir):
    m = oracle.Oracle(oracle.build_mutant(n, mutant_dir))
    assert m.mutation == n
    r = run_pins(m)
    assert not all(r.values()), r
