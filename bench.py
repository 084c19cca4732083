#!/usr/bin/env python3
"""Batch-1 quantized-weight GEMV benchmark on one MI355X.

The default run measures every workload in one process and prints one JSON
line.  Its headline (`value`, `ms_per_step`, `roofline`) is the largest
batch-1 dense GEMV, fp8-e4m3 with 128x128 block scales at 7168 x 16384
(117.6 MB per call); a step is one qgemv_fp8b128 call.  The key `configs`
holds every workload (the headline's included), each with its time per
launch, algorithmic bytes, roofline fraction, the plain-read ceiling of the
same bytes, HBM traffic from the committed counter profiles and the CPU
oracle's rate; `host` records the machine and the build.

Workloads (one launch per step each):
  i4g_O256_I512_gs64           grouped int4, the small parity shape
  i4g_O12288_I6144_gs64        grouped int4 at the resident-projection shape
  i4g_O12288_I6144_gs128       the same with groups of 128
  fp8b128_O7168_I16384         fp8-e4m3, f32 scale per 128x128 block (headline)
  mq4v2_O8192_I8192            MQ4-v2 GEMV on activations already rotated
  mq4v2rot_O8192_I8192         MQ4-v2 with the FWHT-256 rotation fused in
  moe_E256_O2048_I7168_gs64_T4_K8  routed experts: 4 tokens, top-8 of 256
`--case NAME` runs one of these (or a multi-vector / other-format variant)
alone.

Dense steps rotate through distinct weight copies totalling over 1 GiB, and
the routed-expert step cycles through 16 routings in which each call's
experts are disjoint from the previous call's, so calls stream their weights
from HBM rather than the 256 MB last-level cache.  All inputs are resident in
HBM before timing.  Each workload is warmed up for a fixed time (the GPU
reaches steady clocks only after some milliseconds of load) on top of
--warmup steps; then the headline times exactly --steps steps between two HIP
events on the launch stream, and every workload is timed in three
interleaved runs of max(--steps, 100) launches (median reported).

`--copy-calibrate BYTES` instead times a plain device-to-device copy of known
size (used to scale the HBM traffic counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFS = 157.3   # dense f32 matrix-core peak
DENSE_27B = 27e9   # weights of the dense decode fixture the tok/s figure is scaled to
ROTATE_BYTES = 1 << 30
WARM_SECONDS = 0.25   # per workload, before its --warmup steps
RUNS = 3
METRIC = "achieved HBM GB/s (% of MI355X peak) + equiv decode tok/s, batch-1 qGEMV"
HEADLINE = "fp8b128_O7168_I16384"
SUITE = ["i4g_O256_I512_gs64", "i4g_O12288_I6144_gs64", "i4g_O12288_I6144_gs128",
         "fp8b128_O7168_I16384", "mq4v2_O8192_I8192", "mq4v2rot_O8192_I8192",
         "moe_E256_O2048_I7168_gs64_T4_K8"]
DTYPE_4BIT = ("f32 accumulate; x as a 22-bit shared-exponent fixed point per 32 columns, "
              "exact integer nibble x digit products")


def n_copies(bytes_per_copy):
    return max(2, int(np.ceil(ROTATE_BYTES / bytes_per_copy)))


def _check(rel, what):
    if not rel <= 1e-5:
        raise SystemExit(f"bench: {what}: GPU result disagrees with the oracle (rel L2 {rel:.3e})")


def _rel(got, ref):
    return float(np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref))


class Case:
    """A workload: device inputs, one step (one launch), parity, CPU sample."""
    name = ""
    kernel = ""            # name fragment of the step's kernel
    fmt_desc = ""
    dtype = "f32"
    bound = "hbm"
    S = 1
    ceiling_pattern = 0    # plain-read pattern of the same bytes (1: MQ4 groups)

    def step(self, i):
        raise NotImplementedError

    def bytes_for(self, first, k):
        return self.alg_bytes * k

    def ceiling_bytes(self):
        return int(self.alg_bytes) // 16 * 16

    def cpu_call(self, rows):
        """The oracle on output rows `rows` (None: all); returns its bytes of work."""
        raise NotImplementedError


class I4G(Case):
    kernel = "i4g_gemv_stream"
    dtype = DTYPE_4BIT

    def __init__(self, O, I, gs, torch, q, o, S=1):
        import workloads as W
        self.name = f"i4g_O{O}_I{I}_gs{gs}" + (f"_S{S}" if S > 1 else "")
        self.fmt_desc = ("grouped int4, f32 scale per group"
                         + (f", {S} vectors per call" if S > 1 else ""))
        self.O, self.I, self.gs, self.S = O, I, gs, S
        rb, ng = (I + 1) // 2, (I + gs - 1) // gs
        self.weight_bytes = O * rb + O * ng * 4
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4)
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = W.gen_i4g(O, I, gs, S=S, seed=0)
        self.n = n_copies(self.weight_bytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        # copy 0 is the seeded workload; the others are drawn with the same laws
        # (one batched tensor each, so the copies cost a few launches)
        wall = torch.randint(0, 256, (self.n - 1, *d["w"].shape), dtype=torch.uint8, device=dev,
                             generator=g)
        sall = 0.002 + 0.018 * torch.rand((self.n - 1, *d["scales"].shape), device=dev,
                                          generator=g)
        self.ws = [torch.from_numpy(d["w"]).to(dev)] + list(wall.unbind(0))
        self.ss = [torch.from_numpy(d["scales"]).to(dev)] + list(sall.unbind(0))
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [(w.data_ptr(), s.data_ptr()) for w, s in zip(self.ws, self.ss)]
        self.d, self.o = d, o
        self.step(0)
        self.rel = _rel(self.y.cpu().numpy(), o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))
        _check(self.rel, self.name)

    def step(self, i):
        wp, spp = self.ptrs[i % self.n]
        st = self.q.qgemv_i4g(wp, spp, self.x.data_ptr(), self.y.data_ptr(), self.S, self.I,
                              self.O, self.gs, self.sp)
        if st:
            raise SystemExit(f"qgemv_i4g: {self.q.strerror(st)}")

    def cpu_call(self, rows):
        d = self.d
        self.o.i4g_gemv(d["w"], d["scales"], d["x"], self.O, self.I, self.gs, rows=rows)
        return self.alg_bytes * (1.0 if rows is None else len(rows) / self.O)


class Prefill(Case):
    """Many tokens through one grouped-int4 matrix: a dense contraction on MFMA."""
    kernel = "i4g_gemm_mfma"
    bound = "mfma"

    def __init__(self, O, I, gs, S, torch, q, o):
        import workloads as W
        self.name = f"i4g_prefill_O{O}_I{I}_gs{gs}_S{S}"
        self.fmt_desc = f"grouped int4, f32 scale per group, {S} tokens (f32 MFMA)"
        self.O, self.I, self.gs, self.S = O, I, gs, S
        rb, ng = (I + 1) // 2, (I + gs - 1) // gs
        self.weight_bytes = O * rb + O * ng * 4
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4)
        self.alg_flops = 2.0 * S * O * I
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = W.gen_i4g(O, I, gs, S=S, seed=0)
        self.n = 1
        self.w = torch.from_numpy(d["w"]).to(dev)
        self.s = torch.from_numpy(d["scales"]).to(dev)
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.d, self.o = d, o
        self.step(0)
        rows = np.arange(0, O, 97)
        self.rel = _rel(self.y.cpu().numpy()[:, rows],
                        o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs, rows=rows))
        _check(self.rel, self.name)

    def step(self, i):
        st = self.q.qgemv_i4g_prefill(self.w.data_ptr(), self.s.data_ptr(), self.x.data_ptr(),
                                      self.y.data_ptr(), self.S, self.I, self.O, self.gs, self.sp)
        if st:
            raise SystemExit(f"qgemv_i4g_prefill: {self.q.strerror(st)}")

    def cpu_call(self, rows):
        d = self.d
        self.o.i4g_gemv(d["w"], d["scales"], d["x"], self.O, self.I, self.gs, rows=rows)
        return self.alg_bytes * (1.0 if rows is None else len(rows) / self.O)


class FP8(Case):
    kernel = "fp8_gemv_stream"

    def __init__(self, O, I, torch, q, o, S=1, ue8m0=False):
        import workloads as W
        self.ue8m0 = ue8m0
        self.name = (f"fp8ue8m0_O{O}_I{I}" if ue8m0 else f"fp8b128_O{O}_I{I}") + \
            (f"_S{S}" if S > 1 else "")
        self.fmt_desc = ("fp8 e4m3, " + ("UE8M0 scale byte" if ue8m0 else "f32 scale")
                         + " per 128x128 block" + (f", {S} vectors per call" if S > 1 else ""))
        self.O, self.I, self.S = O, I, S
        nbo, nbi = W.fp8_nblocks(O, I)
        self.weight_bytes = O * I + nbo * nbi * (1 if ue8m0 else 4)
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4)
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = (W.gen_fp8ue8m0 if ue8m0 else W.gen_fp8b128)(O, I, S=S, seed=0)
        skey = "scale_e8m0" if ue8m0 else "scale_inv"
        self.n = n_copies(self.weight_bytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        # uniform over the 254 non-NaN codes: v in 0..253 -> v + (v >= 0x7F)
        v = torch.randint(0, 254, (self.n - 1, O, I), dtype=torch.uint8, device=dev, generator=g)
        v += (v >= 0x7F).to(torch.uint8)
        if ue8m0:
            sall = torch.randint(114, 121, (self.n - 1, nbo, nbi), dtype=torch.uint8, device=dev,
                                 generator=g)
        else:
            sall = torch.exp(np.log(1e-4) + (np.log(1e-2) - np.log(1e-4)) *
                             torch.rand((self.n - 1, nbo, nbi), device=dev, generator=g))
        self.ws = [torch.from_numpy(d["w"]).to(dev)] + list(v.unbind(0))
        self.ss = [torch.from_numpy(d[skey]).to(dev)] + list(sall.unbind(0))
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [(w.data_ptr(), s.data_ptr()) for w, s in zip(self.ws, self.ss)]
        self.d, self.o, self.skey = d, o, skey
        self.step(0)
        self.rel = _rel(self.y.cpu().numpy(), self._ref(None))
        _check(self.rel, self.name)

    def _ref(self, rows):
        d = self.d
        fn = self.o.fp8ue8m0_gemv if self.ue8m0 else self.o.fp8b128_gemv
        return fn(d["w"], d[self.skey], d["x"], self.O, self.I, rows=rows)

    def step(self, i):
        wp, spp = self.ptrs[i % self.n]
        fn = self.q.qgemv_fp8b128_ue8m0 if self.ue8m0 else self.q.qgemv_fp8b128
        st = fn(wp, spp, self.x.data_ptr(), self.y.data_ptr(), self.S, self.I, self.O, self.sp)
        if st:
            raise SystemExit(f"fp8 GEMV: {self.q.strerror(st)}")

    def cpu_call(self, rows):
        self._ref(rows)
        return self.alg_bytes * (1.0 if rows is None else len(rows) / self.O)


class MQ4(Case):
    """MQ4 GEMV.  rot=False: qgemv_mq4v2 (or v1 / MQ4C) on activations rotated
    beforehand (outside the timed region), the GEMV alone; rot=True:
    qgemv_mq4v2_rot, the rotation fused into the GEMV's staging."""
    kernel = "mq4v2_gemv_stream"
    dtype = DTYPE_4BIT
    ceiling_pattern = 1

    FORMATS = {
        "v2": ("mq4v2", "MQ4-v2 136 B / 256 weights (fp16 scale+zero per 128)"),
        "v1": ("mq4v1", "MQ4 v1 136 B / 256 weights (f32 scale+zero per 256)"),
        "c": ("mq4c", "MQ4C pad 136 B / 256 weights (fp16 scale+zero per 256)"),
    }

    def __init__(self, O, I, torch, q, o, S=1, fmt="v2", rot=False):
        import workloads as W
        self.fmt, self.rot = fmt, rot
        tag, desc = self.FORMATS[fmt]
        self.name = f"{tag}{'rot' if rot else ''}_O{O}_I{I}" + (f"_S{S}" if S > 1 else "")
        self.fmt_desc = (desc + (", FWHT-256 rotation of x fused in" if rot else
                                 ", activations FWHT-256 rotated beforehand")
                         + (f", {S} vectors per call" if S > 1 else ""))
        self.O, self.I, self.S = O, I, S
        self.weight_bytes = O * (I // 256) * 136
        # GEMV alone: weights, x_rot in, y out; fused: weights, x, signs in, y out
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4) + (I if rot else 0)
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = {"v2": W.gen_mq4v2, "v1": W.gen_mq4v1, "c": W.gen_mq4c}[fmt](O, I, S=S, seed=0)
        self.n = n_copies(self.weight_bytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        w0 = torch.from_numpy(d["w"].reshape(O, -1)).to(dev)
        # the other copies: fresh payload, headers from copy 0 with their rows
        # re-paired at random (same value ranges)
        G = I // 256
        wall = torch.empty((self.n - 1, O, G, 136), dtype=torch.uint8, device=dev)
        wall[..., 8:] = torch.randint(0, 256, (self.n - 1, O, G, 128), dtype=torch.uint8,
                                      device=dev, generator=g)
        perm = torch.randint(0, O, (self.n - 1, O), device=dev, generator=g)
        wall[..., :8] = w0.view(O, G, 136)[perm, :, :8]
        self.ws = [w0] + [c.view(O, G * 136) for c in wall.unbind(0)]
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.signs = torch.from_numpy(d["signs"]).to(dev)
        self.xr = torch.empty_like(self.x)
        st = q.qgemv_fwht256(self.x.data_ptr(), self.signs.data_ptr(), self.xr.data_ptr(), S, I,
                             torch.cuda.current_stream().cuda_stream)
        if st:
            raise SystemExit(f"qgemv_fwht256: {q.strerror(st)}")
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [w.data_ptr() for w in self.ws]
        self.d, self.o = d, o
        self.ref_fn = {"v2": o.mq4v2_gemv, "v1": o.mq4v1_gemv, "c": o.mq4c_gemv}[fmt]
        self.xrot_ref = o.fwht256(d["x"], d["signs"], I)
        self.step(0)
        self.rel = _rel(self.y.cpu().numpy(), self.ref_fn(d["w"], self.xrot_ref, O, I))
        _check(self.rel, self.name)

    def step(self, i):
        q = self.q
        if self.rot:
            st = q.qgemv_mq4v2_rot(self.ptrs[i % self.n], self.x.data_ptr(),
                                   self.signs.data_ptr(), self.y.data_ptr(), self.S, self.I,
                                   self.O, self.sp)
        else:
            gemv = {"v2": q.qgemv_mq4v2, "v1": q.qgemv_mq4v1, "c": q.qgemv_mq4c}[self.fmt]
            st = gemv(self.ptrs[i % self.n], self.xr.data_ptr(), self.y.data_ptr(), self.S,
                      self.I, self.O, self.sp)
        if st:
            raise SystemExit(f"mq4 step: {q.strerror(st)}")

    def ceiling_bytes(self):
        return self.weight_bytes

    def cpu_call(self, rows):
        d = self.d
        xr = self.o.fwht256(d["x"], d["signs"], self.I) if self.rot else self.xrot_ref
        self.ref_fn(d["w"], xr, self.O, self.I, rows=rows)
        return self.alg_bytes * (1.0 if rows is None else len(rows) / self.O)


class MoE(Case):
    kernel = "moe_i4g_stream"
    dtype = DTYPE_4BIT
    N_ROUTINGS = 16

    def __init__(self, E, O, I, gs, T, K, torch, q, o):
        import workloads as W
        self.name = f"moe_E{E}_O{O}_I{I}_gs{gs}_T{T}_K{K}"
        self.fmt_desc = "routed grouped-int4 experts, gate-weighted top-k sum"
        self.E, self.O, self.I, self.gs, self.T, self.K = E, O, I, gs, T, K
        self.S = T
        rb, ng = (I + 1) // 2, (I + gs - 1) // gs
        self.expert_bytes = O * rb + O * ng * 4
        self.bytes_per_weight = self.expert_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = W.gen_moe(E, O, I, gs, T, K, seed=0)
        self.w = torch.from_numpy(d["w"]).to(dev)
        self.s = torch.from_numpy(d["scales"]).to(dev)
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((T, O), dtype=torch.float32, device=dev)
        self.ws_buf = q.moe_topk_workspace(T, K, O, dev)
        routings = W.gen_moe_routings_disjoint(E, T, K, self.N_ROUTINGS, (d["ids"], d["gates"]))
        self.routings = [(torch.from_numpy(i).to(dev), torch.from_numpy(g).to(dev))
                         for i, g in routings]
        self.uniq = [len(np.unique(i)) for i, _ in routings]
        small = T * I * 4 + T * O * 4 + T * K * 8
        self.alg_bytes_per_routing = [u * self.expert_bytes + small for u in self.uniq]
        self.alg_bytes = float(np.mean(self.alg_bytes_per_routing))
        self.weight_bytes = float(np.mean(self.uniq)) * self.expert_bytes
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.d, self.o = d, o
        self.step(0)
        ref = o.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], E, O, I, gs)
        self.rel = _rel(self.y.cpu().numpy(), ref)
        _check(self.rel, self.name)

    def step(self, i):
        ids, gates = self.routings[i % self.N_ROUTINGS]
        st = self.q.qgemv_moe_topk(self.w.data_ptr(), self.s.data_ptr(), self.w[0].numel(),
                                   self.s[0].numel(), self.E, ids.data_ptr(), gates.data_ptr(),
                                   self.T, self.K, self.x.data_ptr(), self.y.data_ptr(), self.I,
                                   self.O, self.gs, self.ws_buf.data_ptr(), self.ws_buf.numel(),
                                   self.sp)
        if st:
            raise SystemExit(f"qgemv_moe_topk: {self.q.strerror(st)}")

    def bytes_for(self, first, k):
        n = self.N_ROUTINGS
        return sum(self.alg_bytes_per_routing[(first + i) % n] for i in range(k))

    def cpu_call(self, rows):
        d = self.d
        self.o.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], self.E, self.O,
                       self.I, self.gs, rows=rows)
        return self.alg_bytes_per_routing[0] * (1.0 if rows is None else len(rows) / self.O)


class ReadCeiling(Case):
    """The plain-read reference of a byte count (libqgemv_ceiling.so) as a case
    of its own, for profiling: `read_<bytes>` contiguous, `read_<bytes>_mq4` in
    the MQ4 group pattern; the tile is the fastest of the swept shapes."""
    kernel = "read_stream"
    dtype = "u8 (no arithmetic)"

    def __init__(self, name, torch):
        parts = name.split("_")
        nbytes, pattern = int(parts[1]), 1 if name.endswith("_mq4") else 0
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        self.cl = Ceiling(torch, load_ceiling_lib(), nbytes, pattern, cus)
        self.cl.pick(torch)
        self.name = name
        self.fmt_desc = f"plain streaming read, tile {self.cl.v}"
        self.O = 1
        self.alg_bytes = self.weight_bytes = self.cl.nbytes
        self.bytes_per_weight = 1.0
        self.ceiling_pattern = pattern
        self.rel = 0.0

    def step(self, i):
        self.cl.step(i)


def build_case(name, torch, q, o):
    if name.startswith("read_"):
        return ReadCeiling(name, torch)
    table = {
        "i4g_O256_I512_gs64": lambda: I4G(256, 512, 64, torch, q, o),
        "i4g_O12288_I6144_gs64": lambda: I4G(12288, 6144, 64, torch, q, o),
        "i4g_O12288_I6144_gs128": lambda: I4G(12288, 6144, 128, torch, q, o),
        "fp8b128_O7168_I16384": lambda: FP8(7168, 16384, torch, q, o),
        "mq4v2_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o),
        "mq4v2rot_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o, rot=True),
        "moe_E256_O2048_I7168_gs64_T4_K8": lambda: MoE(256, 2048, 7168, 64, 4, 8, torch, q, o),
        "i4g_O12288_I6144_gs64_S2": lambda: I4G(12288, 6144, 64, torch, q, o, S=2),
        "i4g_O12288_I6144_gs64_S4": lambda: I4G(12288, 6144, 64, torch, q, o, S=4),
        "fp8b128_O7168_I16384_S2": lambda: FP8(7168, 16384, torch, q, o, S=2),
        "fp8b128_O7168_I16384_S4": lambda: FP8(7168, 16384, torch, q, o, S=4),
        "mq4v2rot_O8192_I8192_S2": lambda: MQ4(8192, 8192, torch, q, o, S=2, rot=True),
        "mq4v2_O8192_I8192_S4": lambda: MQ4(8192, 8192, torch, q, o, S=4),
        "fp8ue8m0_O7168_I16384": lambda: FP8(7168, 16384, torch, q, o, ue8m0=True),
        "mq4v1_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o, fmt="v1"),
        "mq4c_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o, fmt="c"),
        "i4g_prefill_O12288_I6144_gs64_S256": lambda: Prefill(12288, 6144, 64, 256, torch, q, o),
        "i4g_prefill_O12288_I6144_gs64_S2048": lambda: Prefill(12288, 6144, 64, 2048, torch, q,
                                                               o),
    }
    return table[name]()


CASE_NAMES = SUITE + [n for n in [
    "i4g_O12288_I6144_gs64_S2", "i4g_O12288_I6144_gs64_S4", "fp8b128_O7168_I16384_S2",
    "fp8b128_O7168_I16384_S4", "mq4v2rot_O8192_I8192_S2", "mq4v2_O8192_I8192_S4",
    "fp8ue8m0_O7168_I16384", "mq4v1_O8192_I8192", "mq4c_O8192_I8192",
    "i4g_prefill_O12288_I6144_gs64_S256", "i4g_prefill_O12288_I6144_gs64_S2048"]] + [
    # plain-read references of the suite's byte counts (profiling)
    "read_42541056", "read_40181760", "read_117563392", "read_35651584_mq4",
    "read_250681344"]


KERNEL_SOURCES = {
    "i4g_gemv_stream": "csrc/i4g.hip",
    "fp8_gemv_stream": "csrc/fp8b128.hip",
    "mq4v2_gemv_stream": "csrc/mq4v2.hip",
    "moe_i4g_stream": "csrc/moe.hip",
    "i4g_gemm_mfma": "csrc/prefill.hip",
    "read_stream": "bench_csrc/ceiling.hip",
}


def kernel_digest(kernel):
    """sha256 over the sources that define `kernel` (its file and, for the
    library's kernels, the shared device and launch headers)."""
    pkg = os.path.join(ROOT, "quantized_weight_decode_amd")
    files = [KERNEL_SOURCES[kernel]]
    if files[0].startswith("csrc/"):
        files += ["csrc/qg_device.h", "csrc/qg_launch.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def profile_record(kernel, workload):
    """From the committed profile summary of this kernel on this workload: the traced
    average duration (us) and the calibrated HBM bytes per launch.  Each is None when
    the summary is absent or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None, None
    digest = traffic = avg = None
    import re
    with open(path) as fh:
        for line in fh:
            if line.startswith("source digest: sha256:"):
                digest = line.split(":", 2)[2].strip()
            elif line.startswith("traffic per dispatch"):
                traffic = int(line.rsplit(":", 1)[1].split()[0])
            m = re.match(r"^\| `[^`]+` \| (\d+) \| ([0-9.]+) \|", line)
            if m and avg is None:
                avg = float(m.group(2))
    if digest != kernel_digest(kernel):
        return None, None
    return avg, traffic


def profiled_traffic(kernel, workload):
    return profile_record(kernel, workload)[1]


def timed(torch, fn, first, k):
    """ms for k steps fn(first), ..., fn(first + k - 1) between two HIP events
    recorded on the launch stream (torch's current stream, which every step
    passes to the library)."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(k):
        fn(first + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def warm(torch, fn, seconds, start=0):
    """Runs steps for at least `seconds` of wall time; returns the next step index."""
    i = start
    t0 = time.perf_counter()
    while True:
        for _ in range(32):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


# ---------------------------------------------------------------------------
# Plain-read ceiling (libqgemv_ceiling.so, benchmark only)
# ---------------------------------------------------------------------------
class Ceiling:
    """Best plain streaming read of `nbytes` (pattern 0: contiguous 16-byte
    chunks; 1: the MQ4 136-byte group pattern) over a sweep of tile shapes and
    of the load policy (non-temporal hint or cached), rotating through copies
    totalling over 1 GiB."""
    # (waves per workgroup, loads in flight per lane, workgroups per CU; 0: one-shot,
    #  cached loads)
    VARIANTS = [(wpb, u, wpc, ca) for ca in (False, True)
                for wpb, u, wpc in
                [(wpb, u, wpc) for wpb in (4, 8, 16) for u in (2, 4, 8) for wpc in (1, 2)
                 if wpb * wpc <= 16] + [(wpb, u, 0) for wpb in (4, 8, 16) for u in (1, 2, 4)]]
    OUT_LEN = 1 << 20

    def __init__(self, torch, lib, nbytes, pattern, cus):
        self.lib, self.pattern = lib, pattern
        unit = 136 if pattern else 16
        self.nbytes = nbytes // unit * unit
        stride = (self.nbytes + 4095) // 4096 * 4096
        self.n = n_copies(stride)
        dev = torch.device("cuda:0")
        self.buf = torch.randint(0, 256, (self.n * stride,), dtype=torch.uint8, device=dev)
        self.ptrs = [self.buf.data_ptr() + i * stride for i in range(self.n)]
        self.out = torch.empty(self.OUT_LEN, dtype=torch.int32, device=dev)
        self.sp = torch.cuda.current_stream().cuda_stream
        self.cus = cus
        self.v = self.VARIANTS[0]
        self.name = f"read_{self.nbytes}" + ("_mq4" if pattern else "")

    def step(self, i):
        wpb, u, wpc, ca = self.v
        st = self.lib.qgemv_ceiling_read(self.ptrs[i % self.n], self.nbytes,
                                         self.pattern | (2 if ca else 0), wpb,
                                         u, self.cus * wpc, self.out.data_ptr(), self.OUT_LEN,
                                         self.sp)
        if st:
            raise SystemExit(f"qgemv_ceiling_read: status {st}")

    def pick(self, torch):
        best = None
        for v in self.VARIANTS:
            self.v = v
            warm(torch, self.step, 0.02)
            ms = min(timed(torch, self.step, 0, 40) for _ in range(2))
            if best is None or ms < best[0]:
                best = (ms, v)
        self.v = best[1]
        return self.v


def load_ceiling_lib():
    import ctypes as C
    path = os.path.join(ROOT, "quantized_weight_decode_amd", "libqgemv_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built: run quantized_weight_decode_amd.build")
    L = C.CDLL(path)
    L.qgemv_ceiling_read.restype = C.c_int
    L.qgemv_ceiling_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_int, C.c_int,
                                     C.c_void_p, C.c_size_t, C.c_void_p]
    return L


# ---------------------------------------------------------------------------
# CPU baseline (the oracle as it stands)
# ---------------------------------------------------------------------------
def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_rate(case, threads, budget_s):
    """Oracle throughput (algorithmic GB/s) on `threads` host threads over about
    budget_s seconds; a row subset of the workload when a whole call would not
    fit the budget several times."""
    import oracle
    o = oracle.load()
    o.set_threads(threads)
    try:
        rows = None
        O = case.O
        t0 = time.perf_counter()
        probe = np.arange(0, O, max(1, O // 64))
        case.cpu_call(probe)
        per_row = (time.perf_counter() - t0) / len(probe)
        if per_row * O > budget_s / 4:
            nr = max(1, min(O, int(budget_s / 8 / max(per_row, 1e-9))))
            rows = np.linspace(0, O - 1, nr).astype(np.int64)
        case.cpu_call(rows)  # warm-up
        n, done = 0, 0.0
        t0 = time.perf_counter()
        while True:
            done += case.cpu_call(rows)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    finally:
        o.set_threads(1)
    part = "whole calls" if rows is None else f"calls on {len(rows)} of {O} output rows"
    return {"value": round(done / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} {part} of {case.name} in {el:.2f} s ({el / n * 1e3:.2f} ms each), "
                      f"f64 accumulate"}


# ---------------------------------------------------------------------------
# Host record
# ---------------------------------------------------------------------------
SOURCE_GLOBS = ["bench.py", "include/*.h", "quantized_weight_decode_amd/*.py",
                "quantized_weight_decode_amd/csrc/*", "quantized_weight_decode_amd/bench_csrc/*",
                "workloads/*.py", "oracle/qref.c", "oracle/*.py"]


def sources_digest():
    """sha256 over the sources that decide what a run computes and times (path and
    bytes of each, in sorted order): the record's link to a checkout where the
    git metadata is not present (recompute with --sources-digest)."""
    import glob
    h = hashlib.sha256()
    paths = sorted({p for g in SOURCE_GLOBS for p in glob.glob(os.path.join(ROOT, g))
                    if os.path.isfile(p)})
    for p in paths:
        h.update(os.path.relpath(p, ROOT).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def host_record(torch):
    def read(path):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            return None
    cpu = None
    txt = read("/proc/cpuinfo") or ""
    for line in txt.splitlines():
        if line.startswith("model name"):
            cpu = line.split(":", 1)[1].strip()
            break
    sha = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        if r.returncode == 0:
            sha = r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass

    def digest(path):
        try:
            with open(path, "rb") as f:
                return hashlib.sha256(f.read()).hexdigest()
        except OSError:
            return None
    lib = os.path.join(ROOT, "quantized_weight_decode_amd", "libqgemv.so")
    props = torch.cuda.get_device_properties(0)
    return {
        "cmdline": " ".join([os.path.basename(sys.executable)] + sys.argv),
        "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": cpu,
        "gpu": props.name, "gpu_arch": getattr(props, "gcnArchName", None),
        "cus": props.multi_processor_count,
        "rocm": read("/opt/rocm/.info/version"), "torch": torch.__version__,
        "python": platform.python_version(), "git_sha": sha,
        "sources_sha256": sources_digest(),
        "libqgemv_sha256": digest(lib),
        "env": {k: os.environ[k] for k in ("HIP_VISIBLE_DEVICES", "ROCR_VISIBLE_DEVICES",
                                           "GPU_MAX_HW_QUEUES", "HSA_XNACK")
                if k in os.environ},
    }


def roofline(case, us, alg_bytes):
    gbs = alg_bytes / (us * 1e-6) / 1e9
    r = {"bound": "hbm", "kernel": case.kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "us_per_launch": round(us, 3),
         "alg_bytes_per_launch": round(alg_bytes)}
    avg, traffic = profile_record(case.kernel, case.name)
    r["traffic"] = traffic
    if traffic and avg:
        # counter view: calibrated HBM bytes over the traced kernel duration
        r["counter_gbs"] = round(traffic / (avg * 1e-6) / 1e9, 1)
        r["profile_avg_us"] = avg
        r["traffic_over_alg"] = round(traffic / alg_bytes, 4)
    if case.bound == "mfma":
        tf = case.alg_flops / (us * 1e-6) / 1e12
        r.update({"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F32_PEAK_TFS,
                  "unit": "TFLOP/s", "frac": round(tf / MFMA_F32_PEAK_TFS, 4),
                  "alg_flops_per_launch": case.alg_flops})
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--case", default=None, choices=CASE_NAMES,
                    help="run one workload alone (default: the whole suite)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the plain-read ceilings")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only time a plain device copy of BYTES bytes")
    ap.add_argument("--sources-digest", action="store_true",
                    help="print the sources digest a record carries, and exit")
    args = ap.parse_args()
    if args.sources_digest:
        print(sources_digest())
        return

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported (across GPUs "
              f"the dense GEMVs would split by output rows and the routed experts by expert, "
              f"each GPU running these kernels on its share)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibrate:
        copy_calibrate(torch, args.copy_calibrate, args.steps)
        return

    import oracle
    import quantized_weight_decode_amd as q

    o = oracle.load()
    names = [args.case] if args.case else SUITE
    headline = args.case or HEADLINE
    cases = {}
    for n in names:
        cases[n] = build_case(n, torch, q, o)
        print(f"bench: built {n} (parity rel L2 {cases[n].rel:.2e})", file=sys.stderr,
              flush=True)

    # headline: time-based warm-up, --warmup steps, then exactly --steps steps
    hc = cases[headline]
    nxt = warm(torch, hc.step, WARM_SECONDS)
    for i in range(args.warmup):
        hc.step(nxt + i)
    first = nxt + args.warmup
    ms = timed(torch, hc.step, first, args.steps)
    ms_step = ms / args.steps
    step_bytes = hc.bytes_for(first, args.steps) / args.steps
    us_head = ms_step * 1e3
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    wgbs = hc.weight_bytes / (ms_step * 1e-3) / 1e9
    nexti = {headline: first + args.steps}

    # every workload: warm-up, then RUNS interleaved runs of max(--steps, 100) launches
    k = max(args.steps, 100)
    runs = {n: [] for n in names}
    for n in names:
        nexti[n] = warm(torch, cases[n].step, WARM_SECONDS, nexti.get(n, 0))
    for _ in range(RUNS):
        for n in names:
            ms_r = timed(torch, cases[n].step, nexti[n], k)
            runs[n].append((ms_r * 1e3 / k, cases[n].bytes_for(nexti[n], k) / k))
            nexti[n] += k

    # plain-read ceilings of the same bytes
    ceilings = {}
    if not args.no_ceiling:
        lib = load_ceiling_lib()
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        for n in names:
            c = cases[n]
            key = (c.ceiling_bytes(), c.ceiling_pattern)
            if key not in ceilings:
                cl = Ceiling(torch, lib, key[0], key[1], cus)
                v = cl.pick(torch)
                warm(torch, cl.step, WARM_SECONDS)
                us = sorted(timed(torch, cl.step, j * k, k) * 1e3 / k for j in range(RUNS))
                ceilings[key] = {"name": cl.name, "bytes": cl.nbytes, "us": round(us[1], 3),
                                 "gbs": round(cl.nbytes / (us[1] * 1e-6) / 1e9, 1),
                                 "frac": round(cl.nbytes / (us[1] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                               4),
                                 "tile": {"waves_per_wg": v[0], "loads_in_flight": v[1],
                                          "mapping": "slab" if v[2] else "one-shot",
                                          "wgs_per_cu": v[2] or None,
                                          "loads": "cached" if v[3] else "non-temporal"}}
                del cl
                torch.cuda.empty_cache()

    threads = host_threads()
    others = {}
    for n in names:
        c = cases[n]
        rr = sorted(runs[n])
        us_med, bytes_med = rr[len(rr) // 2]
        ent = {"format": c.fmt_desc, "dtype": c.dtype, "vectors": c.S,
               "us_per_launch": {"median": round(us_med, 3), "min": round(rr[0][0], 3),
                                 "max": round(rr[-1][0], 3), "runs": RUNS, "launches": k},
               "alg_bytes_per_launch": round(bytes_med),
               "roofline": roofline(c, us_med, bytes_med),
               "weights_gbs": round(c.weight_bytes / (us_med * 1e-6) / 1e9, 1),
               "equiv_decode_tok_s": round(c.weight_bytes / (us_med * 1e-6) /
                                           (DENSE_27B * c.bytes_per_weight), 1),
               "parity_rel_l2": c.rel}
        key = (c.ceiling_bytes(), c.ceiling_pattern)
        if key in ceilings:
            ce = ceilings[key]
            ent["ceiling"] = dict(ce)
            # the workload's time against a plain read of its bytes
            ent["frac_of_ceiling"] = round(ce["us"] / us_med, 4)
        if isinstance(c, MoE):
            ent["distinct_experts_per_routing"] = c.uniq
            ent["tokens_per_s"] = round(c.T / (us_med * 1e-6), 1)
        if not args.no_cpu and not isinstance(c, ReadCeiling):
            budget = 2.5
            ent["cpu_baseline"] = {"all_threads": cpu_rate(c, threads, budget),
                                   "one_thread": cpu_rate(c, 1, budget)}
        others[n] = ent
        print(f"bench: {n}: {us_med:.3f} us/launch, "
              f"{ent['roofline']['frac']:.3f} of peak", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": hc.dtype, "data": "synthetic",
        "config": {"workload": hc.name, "batch": hc.S, "format": hc.fmt_desc,
                   "alg_bytes_per_step": round(step_bytes)},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "weights_gbs": round(wgbs, 1),
        "equiv_decode_tok_s": round(wgbs * 1e9 / (DENSE_27B * hc.bytes_per_weight), 1),
        "roofline": roofline(hc, us_head, step_bytes),
        "parity_rel_l2": hc.rel,
    }
    if not args.no_cpu and not isinstance(hc, ReadCeiling):
        # the headline workload's oracle on all host threads over a longer sample
        out["cpu_baseline"] = cpu_rate(hc, threads, 10.0)
    out["configs"] = others
    out["host"] = host_record(torch)
    print(json.dumps(out), flush=True)


def copy_calibrate(torch, nbytes, steps):
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    ms = timed(torch, lambda i: b.copy_(a), 0, steps)
    print(json.dumps({"copy_calibrate_bytes": nbytes, "steps": steps,
                      "ms_per_copy": ms / steps,
                      "GBs_read_plus_write": 2 * nbytes / (ms / steps * 1e-3) / 1e9}), flush=True)


if __name__ == "__main__":
    main()
