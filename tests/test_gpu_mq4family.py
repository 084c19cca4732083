"""MQ4 v1, MQ4C pad and the MQ4-v2 encoder on the GPU against the CPU oracle.

hipfire "MQ4 V2": sections 1b / 1e (v1's two f32 header fields, MQ4C's one
fp16 pair plus zero pad, the shared 136-byte geometry; equal half headers make
v2 identical to v1) and section 3 (the encoder).  Decoded weights and encoded
bytes must match bit for bit; y to relative L2 <= 1e-5.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bits_equal, assert_y_close, dev, host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    torch_cuda()
    import quantized_weight_decode_amd as q
    return q


GEN = {"v1": W.gen_mq4v1, "c": W.gen_mq4c}


def gemv(q, fmt, w, x):
    return q.mq4v1(w, x) if fmt == "v1" else q.mq4c(w, x)


def ref_gemv(qref, fmt, w, x, O, I, rows=None):
    return (qref.mq4v1_gemv if fmt == "v1" else qref.mq4c_gemv)(w, x, O, I, rows=rows)


@pytest.mark.parametrize("fmt", ["v1", "c"])
@pytest.mark.parametrize("O,I", [(9, 768), (64, 8192), (3, 256)])
def test_dequant_bit_exact(q, qref, fmt, O, I):
    d = GEN[fmt](O, I, seed=O + I)
    f = q.dequant_mq4v1 if fmt == "v1" else q.dequant_mq4c
    got = host(f(dev(d["w"].reshape(O, -1)), I))
    want = (qref.mq4v1_dequant if fmt == "v1" else qref.mq4c_dequant)(d["w"], O, I)
    assert_bits_equal(got, want)


@pytest.mark.parametrize("fmt", ["v1", "c"])
@pytest.mark.parametrize("O,I,S", [(256, 512, 1), (300, 1024, 2), (77, 256, 3), (1000, 4096, 4),
                                   (33, 2304, 1), (5, 768, 8), (1, 256, 1)])
def test_gemv_matches_oracle(q, qref, fmt, O, I, S):
    d = GEN[fmt](O, I, S=S, seed=O + 5)
    y = host(gemv(q, fmt, dev(d["w"].reshape(O, -1)), dev(d["x"])))
    assert_y_close(y, ref_gemv(qref, fmt, d["w"], d["x"], O, I))


@pytest.mark.parametrize("fmt", ["v1", "c"])
def test_workload_shape_sampled_rows(q, qref, fmt):
    O, I = 8192, 8192
    d = GEN[fmt](O, I, seed=0)
    y = host(gemv(q, fmt, dev(d["w"].reshape(O, -1)), dev(d["x"])))
    rows = np.concatenate([np.arange(0, O, 89), [O - 1]])
    assert_y_close(y[:, rows], ref_gemv(qref, fmt, d["w"], d["x"], O, I, rows=rows))


def test_equal_halves_v2_v1_c_bitwise(q):
    # v2 with both halves' headers equal == v1 with those values as f32 ==
    # MQ4C with that pair and a zero pad, on the same nibbles
    O, I = 512, 4096
    d = W.gen_mq4v2(O, I, S=2, seed=31)
    G = I // 256
    w2 = d["w"].reshape(O, G, 136).copy()
    w2[:, :, 4:8] = w2[:, :, 0:4]
    hdr = w2[:, :, 0:4].copy().view("<u2").reshape(O, G, 2)
    w1 = w2.copy()
    w1[:, :, 0:4] = hdr[:, :, 0].view(np.float16).astype("<f4").view(np.uint8).reshape(O, G, 4)
    w1[:, :, 4:8] = hdr[:, :, 1].view(np.float16).astype("<f4").view(np.uint8).reshape(O, G, 4)
    wc = w2.copy()
    wc[:, :, 4:8] = 0
    x = dev(d["x"])
    a = host(q.mq4v2(dev(w2.reshape(O, -1)), x))
    b = host(q.mq4v1(dev(w1.reshape(O, -1)), x))
    c = host(q.mq4c(dev(wc.reshape(O, -1)), x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_non_finite_activation(q, qref):
    O, I = 200, 2048
    d = W.gen_mq4v1(O, I, seed=8)
    d["x"][0, 300] = np.inf
    y = host(q.mq4v1(dev(d["w"].reshape(O, -1)), dev(d["x"])))
    assert_y_close(y, qref.mq4v1_gemv(d["w"], d["x"], O, I))


# -- encoder -------------------------------------------------------------------
@pytest.mark.parametrize("O,I", [(64, 8192), (7, 256), (300, 1024)])
def test_encoder_bytes_match_oracle(q, qref, O, I):
    Wt = W.gen_rotated_weights(O, I, seed=O)
    got = host(q.mq4v2_encode(dev(Wt)))
    assert np.array_equal(got, qref.mq4v2_encode(Wt, O, I))


def test_encoder_special_halves(q, qref):
    O, I = 6, 512
    Wt = W.gen_rotated_weights(O, I, seed=3)
    k = np.arange(128) % 16
    Wt[0, :128] = 0.0625                         # constant half
    Wt[0, 128:256] = -0.5 + k * 2.0 ** -6        # fp16-exact grid
    Wt[1, :128] = 1.0 + np.arange(128) * 1e-10   # step below fp16's range
    Wt[2, :128] = np.abs(Wt[2, :128])
    Wt[2, 5] = -0.0                              # -0 minimum
    Wt[3, 256:384] = -0.0                        # constant -0 half
    Wt[4, :128] = 60000.0 + k * 100.0            # large values
    Wt[5, 128:256] = np.float32(1e-7) * k        # fp16-subnormal step and zero
    Wt = Wt.astype(np.float32)
    got = host(q.mq4v2_encode(dev(Wt)))
    want = qref.mq4v2_encode(Wt, O, I)
    bad = [(r, int(np.argmax(got[r] != want[r]))) for r in range(O) if not np.array_equal(got[r], want[r])]
    assert not bad, f"rows (first differing byte): {bad}"


def test_encode_decode_round_trip(q, qref):
    O, I = 128, 4096
    Wt = W.gen_rotated_weights(O, I, seed=11)
    enc = q.mq4v2_encode(dev(Wt))
    dec = host(q.dequant_mq4v2(enc, I))
    assert_bits_equal(dec, qref.mq4v2_dequant(host(enc), O, I))
    # every weight within half a step (plus the fp16 header rounding) of its value
    hdr = host(enc).reshape(O, I // 256, 136)[:, :, 0:8].copy().view("<u2").reshape(O, I // 256, 2, 2)
    st = hdr[..., 0].view(np.float16).astype(np.float64)
    w = Wt.reshape(O, I // 256, 2, 128).astype(np.float64)
    lo, hi = w.min(-1), w.max(-1)
    z = hdr[..., 1].view(np.float16).astype(np.float64)
    bound = np.maximum(st / 2, 15 * np.abs(st - (hi - lo) / 15) + np.abs(z - lo)) + 1e-9
    err = np.abs(dec.reshape(O, I // 256, 2, 128) - w).max(-1)
    assert np.all(err <= bound)
