"""Seeded synthetic inputs for the quantized-weight GEMV workloads.

This module only draws random numbers and lays them out in the byte formats the
kernels read.  It holds none of the method's arithmetic (no decode, no dot
products): both the CPU oracle and the GPU path receive exactly these arrays.

Formats (byte layouts as the pages define them):

* grouped int4 ("fmt=4", colibri PR #457 "metal: grouped-int4 (fmt=4) GEMV
  support", sections 1 and 3): row-major ``u8[O][(I+1)//2]``, two unsigned
  nibbles per byte (even column in the low nibble), one f32 scale per
  ``gs`` columns, ``f32[O][ceil(I/gs)]``.  A byte drawn uniformly from 0..255
  is exactly two independent nibbles drawn uniformly from 0..15.
* fp8-e4m3 with 128x128 f32 block scales ("fmt=7", colibri PR #528
  "fmt=7: fp8-e4m3-b128 passthrough weight format", section "Design"):
  ``u8[O][I]`` raw E4M3-FN codes, ``f32[ceil(O/128)][ceil(I/128)]``.
* MQ4-v2 (hipfire "MQ4 V2" page, sections 2 and 4): 136 bytes per 256
  weights; bytes 0..3 hold the fp16 scale and fp16 zero of weights 0..127,
  bytes 4..7 those of weights 128..255, bytes 8..135 the 128 payload bytes.
  MQ4 v1 (sections 1b, 1e) keeps the geometry with an f32 scale at byte 0 and
  an f32 zero at byte 4 for all 256 weights; MQ4C pad one fp16 pair at byte 0
  and a zero pad at bytes 4..7.

Random numbers are drawn with ``numpy.random.default_rng(seed)`` in the order
each function lists; the recipes follow the workload descriptions (uniform
nibbles, uniform scales, N(0,1) activations, ...).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "i4g_rowbytes", "i4g_ngroups", "fp8_nblocks",
    "random_bytes", "gen_i4g", "gen_fp8b128", "gen_fp8ue8m0", "gen_mq4v2", "gen_mq4v1",
    "gen_mq4c", "gen_rotated_weights", "gen_fwht_signs",
    "gen_moe", "gen_moe_routing", "E4M3_NON_NAN_CODES",
    "WORKLOADS",
]


def i4g_rowbytes(I: int) -> int:
    """Packed bytes per row of a grouped-int4 matrix: two columns per byte."""
    return (I + 1) // 2


def i4g_ngroups(I: int, gs: int) -> int:
    """Scale groups per row: ceil(I / gs)."""
    return (I + gs - 1) // gs


def fp8_nblocks(O: int, I: int) -> tuple[int, int]:
    """Number of 128x128 scale blocks along O and along I."""
    return (O + 127) // 128, (I + 127) // 128


# The 254 E4M3-FN codes that are not NaN (0x7F and 0xFF are the only NaNs).
E4M3_NON_NAN_CODES = np.array(
    [c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform bytes 0..255 of the given shape (fast path through rng.bytes)."""
    n = int(np.prod(shape)) if len(shape) else 1
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def _uniform_f32(rng, lo, hi, shape):
    return (lo + (hi - lo) * rng.random(shape, dtype=np.float64)).astype(np.float32)


def gen_i4g(O: int, I: int, gs: int, S: int = 1, seed: int = 0,
            scale_lo: float = 0.002, scale_hi: float = 0.02) -> dict:
    """Grouped-int4 GEMV inputs.

    Draw order: packed weight bytes u8[O][(I+1)//2] (each nibble U{0..15}),
    scales U[scale_lo, scale_hi] as f32[O][ceil(I/gs)], x ~ N(0,1) f32[S][I].
    For odd I the high nibble of each row's last byte is drawn but unused.
    """
    rng = np.random.default_rng(seed)
    w = random_bytes(rng, (O, i4g_rowbytes(I)))
    scales = _uniform_f32(rng, scale_lo, scale_hi, (O, i4g_ngroups(I, gs)))
    x = rng.standard_normal((S, I), dtype=np.float32)
    return {"fmt": "i4g", "O": O, "I": I, "gs": gs, "S": S,
            "w": w, "scales": scales, "x": x}


def gen_fp8b128(O: int, I: int, S: int = 1, seed: int = 0,
                s_lo: float = 1e-4, s_hi: float = 1e-2) -> dict:
    """fp8-e4m3 block-scaled GEMV inputs.

    Draw order: weight codes uniform over the 254 non-NaN E4M3-FN codes,
    u8[O][I]; block scales exp(U[ln s_lo, ln s_hi]) as
    f32[ceil(O/128)][ceil(I/128)]; x ~ N(0,1) f32[S][I].
    """
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E4M3_NON_NAN_CODES.size, (O, I), dtype=np.uint8)
    w = E4M3_NON_NAN_CODES[idx]
    nbo, nbi = fp8_nblocks(O, I)
    scale = np.exp(rng.uniform(math.log(s_lo), math.log(s_hi), (nbo, nbi))).astype(np.float32)
    x = rng.standard_normal((S, I), dtype=np.float32)
    return {"fmt": "fp8b128", "O": O, "I": I, "S": S,
            "w": w, "scale_inv": scale, "x": x}


def gen_fp8ue8m0(O: int, I: int, S: int = 1, seed: int = 0,
                 e_lo: int = 114, e_hi: int = 120) -> dict:
    """fp8-e4m3 GEMV inputs with UE8M0 (power-of-two) 128x128 block scales.

    Draw order: weight codes as gen_fp8b128, u8[O][I]; block scale exponent
    bytes uniform over [e_lo, e_hi] (2^-13 .. 2^-7, the powers of two inside
    the f32-scale range 1e-4 .. 1e-2) as u8[ceil(O/128)][ceil(I/128)];
    x ~ N(0,1) f32[S][I].
    """
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E4M3_NON_NAN_CODES.size, (O, I), dtype=np.uint8)
    w = E4M3_NON_NAN_CODES[idx]
    nbo, nbi = fp8_nblocks(O, I)
    se = rng.integers(e_lo, e_hi + 1, (nbo, nbi)).astype(np.uint8)
    x = rng.standard_normal((S, I), dtype=np.float32)
    return {"fmt": "fp8ue8m0", "O": O, "I": I, "S": S, "w": w, "scale_e8m0": se, "x": x}


def gen_fwht_signs(I: int, seed: int = 42) -> np.ndarray:
    """Per-element +-1 rotation signs, int8[I], from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 2, I).astype(np.int8) * 2 - 1).astype(np.int8)


def gen_mq4v2(O: int, I: int, S: int = 1, seed: int = 0, sign_seed: int = 42,
              sc_lo: float = 1e-3, sc_hi: float = 1e-2,
              zp_lo: float = -0.08, zp_hi: float = 0.0) -> dict:
    """MQ4-v2 GEMV inputs (I must be a multiple of 256).

    Draw order: fp16 scales U[sc_lo, sc_hi] per (row, group, half),
    fp16 zeros U[zp_lo, zp_hi] per (row, group, half), payload bytes
    u8[O][I/256][128] (each nibble U{0..15}), x ~ N(0,1) f32[S][I]; the
    rotation signs come from their own generator seeded with sign_seed.
    fp16 values are the round-to-nearest-even conversion of the f64 draws.

    Returns the packed 136-byte groups plus the unpacked header halves
    (``sc16``/``zp16`` as float16 [O][G][2]) and ``signs``.
    """
    if I % 256:
        raise ValueError("MQ4-v2 needs I % 256 == 0")
    G = I // 256
    rng = np.random.default_rng(seed)
    sc16 = rng.uniform(sc_lo, sc_hi, (O, G, 2)).astype(np.float16)
    zp16 = rng.uniform(zp_lo, zp_hi, (O, G, 2)).astype(np.float16)
    payload = random_bytes(rng, (O, G, 128))
    x = rng.standard_normal((S, I), dtype=np.float32)
    w = np.empty((O, G, 136), dtype=np.uint8)
    # header dword h (h = 0 for weights 0..127, 1 for 128..255) sits at byte
    # 4h: its low 16 bits are the fp16 scale, its high 16 bits the fp16 zero.
    def le16(a):  # fp16 values -> their two little-endian bytes
        return np.ascontiguousarray(a).view(np.uint16).astype("<u2").view(np.uint8).reshape(O, G, 2)
    w[:, :, 0:2] = le16(sc16[:, :, 0])
    w[:, :, 2:4] = le16(zp16[:, :, 0])
    w[:, :, 4:6] = le16(sc16[:, :, 1])
    w[:, :, 6:8] = le16(zp16[:, :, 1])
    w[:, :, 8:136] = payload
    return {"fmt": "mq4v2", "O": O, "I": I, "S": S, "w": w,
            "sc16": sc16, "zp16": zp16, "x": x,
            "signs": gen_fwht_signs(I, sign_seed)}


def gen_mq4v1(O: int, I: int, S: int = 1, seed: int = 0, sign_seed: int = 42,
              sc_lo: float = 1e-3, sc_hi: float = 1e-2,
              zp_lo: float = -0.08, zp_hi: float = 0.0) -> dict:
    """MQ4 v1 (qt=13) GEMV inputs: one f32 scale and f32 zero per 256 weights.

    Draw order: f32 scales U[sc_lo, sc_hi] per (row, group), f32 zeros
    U[zp_lo, zp_hi] per (row, group), payload bytes u8[O][I/256][128], x ~
    N(0,1) f32[S][I].  Bytes 0..3 of a group hold the scale, 4..7 the zero
    (little-endian f32), 8..135 the payload.
    """
    if I % 256:
        raise ValueError("MQ4 needs I % 256 == 0")
    G = I // 256
    rng = np.random.default_rng(seed)
    sc = rng.uniform(sc_lo, sc_hi, (O, G)).astype(np.float32)
    zp = rng.uniform(zp_lo, zp_hi, (O, G)).astype(np.float32)
    payload = random_bytes(rng, (O, G, 128))
    x = rng.standard_normal((S, I), dtype=np.float32)
    w = np.empty((O, G, 136), dtype=np.uint8)
    w[:, :, 0:4] = np.ascontiguousarray(sc).astype("<f4").view(np.uint8).reshape(O, G, 4)
    w[:, :, 4:8] = np.ascontiguousarray(zp).astype("<f4").view(np.uint8).reshape(O, G, 4)
    w[:, :, 8:136] = payload
    return {"fmt": "mq4v1", "O": O, "I": I, "S": S, "w": w, "sc": sc, "zp": zp, "x": x,
            "signs": gen_fwht_signs(I, sign_seed)}


def gen_mq4c(O: int, I: int, S: int = 1, seed: int = 0, sign_seed: int = 42,
             sc_lo: float = 1e-3, sc_hi: float = 1e-2,
             zp_lo: float = -0.08, zp_hi: float = 0.0) -> dict:
    """MQ4C pad (qt=45) GEMV inputs: one fp16 scale/zero pair per 256 weights.

    Draw order: fp16 scales and zeros as gen_mq4v2 but per (row, group),
    payload bytes, x.  Bytes 0..1 hold the fp16 scale, 2..3 the fp16 zero,
    4..7 the zero pad, 8..135 the payload.
    """
    if I % 256:
        raise ValueError("MQ4 needs I % 256 == 0")
    G = I // 256
    rng = np.random.default_rng(seed)
    sc16 = rng.uniform(sc_lo, sc_hi, (O, G)).astype(np.float16)
    zp16 = rng.uniform(zp_lo, zp_hi, (O, G)).astype(np.float16)
    payload = random_bytes(rng, (O, G, 128))
    x = rng.standard_normal((S, I), dtype=np.float32)
    w = np.zeros((O, G, 136), dtype=np.uint8)
    w[:, :, 0:2] = np.ascontiguousarray(sc16).astype("<f2").view(np.uint8).reshape(O, G, 2)
    w[:, :, 2:4] = np.ascontiguousarray(zp16).astype("<f2").view(np.uint8).reshape(O, G, 2)
    w[:, :, 8:136] = payload
    return {"fmt": "mq4c", "O": O, "I": I, "S": S, "w": w, "sc16": sc16, "zp16": zp16,
            "x": x, "signs": gen_fwht_signs(I, sign_seed)}


def gen_rotated_weights(O: int, I: int, seed: int = 0, sigma: float = 0.02) -> np.ndarray:
    """Dense f32 weights [O][I] ~ N(0, sigma^2), standing in for weights already
    in the rotated space (the input of the MQ4-v2 encoder)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((O, I)) * sigma).astype(np.float32)


def gen_moe_routing(E: int, T: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-K expert ids per token (uniform, without replacement) and gates.

    ids int32[T][K]; gates f32[T][K] = softmax over each token's K logits
    drawn N(0,1) (the gate weights are normalised over the selected experts).
    """
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    logits = rng.standard_normal((T, K))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    gates = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, gates


def gen_moe_routings_disjoint(E: int, T: int, K: int, n: int, first: tuple,
                              seed: int = 1000) -> list:
    """n routings for timing: routing 0 is ``first`` (ids, gates); routing r
    draws each token's K experts uniformly without replacement from the
    experts routing r - 1 did not select (and, for the last one, not routing 0
    either, so a cycle through them never repeats an expert between calls).
    Gates as in gen_moe_routing.  Returns a list of (ids, gates)."""
    out = [first]
    used0 = set(np.unique(first[0]).tolist())
    for r in range(1, n):
        rng = np.random.default_rng(seed + r)
        banned = set(np.unique(out[-1][0]).tolist())
        if r == n - 1:
            banned |= used0
        allowed = np.array([e for e in range(E) if e not in banned], dtype=np.int64)
        if allowed.size < K:
            raise ValueError("too few experts left to draw a disjoint routing")
        ids = np.stack([rng.choice(allowed, K, replace=False) for _ in range(T)]).astype(np.int32)
        logits = rng.standard_normal((T, K))
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        out.append((ids, (e / e.sum(axis=1, keepdims=True)).astype(np.float32)))
    return out


def gen_moe(E: int, O: int, I: int, gs: int, T: int, K: int, seed: int = 0,
            routing_seed: int | None = None) -> dict:
    """Routed-expert inputs: E grouped-int4 experts of shape [O x I].

    Draw order: expert weight bytes u8[E][O][(I+1)//2], expert scales
    U[0.002, 0.02] f32[E][O][ceil(I/gs)], x ~ N(0,1) f32[T][I]; routing
    (ids, gates) from ``gen_moe_routing`` with ``routing_seed`` (default:
    seed + 1).
    """
    rng = np.random.default_rng(seed)
    w = random_bytes(rng, (E, O, i4g_rowbytes(I)))
    scales = _uniform_f32(rng, 0.002, 0.02, (E, O, i4g_ngroups(I, gs)))
    x = rng.standard_normal((T, I), dtype=np.float32)
    ids, gates = gen_moe_routing(E, T, K, seed + 1 if routing_seed is None else routing_seed)
    return {"fmt": "moe_i4g", "E": E, "O": O, "I": I, "gs": gs, "T": T, "K": K,
            "w": w, "scales": scales, "x": x, "ids": ids, "gates": gates}


# The five workload shapes (plus the gs=128 variant of the resident
# projection), named by what they are.
WORKLOADS = {
    "i4g_O256_I512_gs64": dict(fn="i4g", O=256, I=512, gs=64),
    "i4g_O12288_I6144_gs64": dict(fn="i4g", O=12288, I=6144, gs=64),
    "i4g_O12288_I6144_gs128": dict(fn="i4g", O=12288, I=6144, gs=128),
    "fp8b128_O7168_I16384": dict(fn="fp8b128", O=7168, I=16384),
    "mq4v2_O8192_I8192": dict(fn="mq4v2", O=8192, I=8192),
    "moe_E256_O2048_I7168_gs64_T4_K8": dict(fn="moe", E=256, O=2048, I=7168, gs=64, T=4, K=8),
}
