#!/usr/bin/env python3
"""Batch-1 quantized-weight GEMV benchmark on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:

  i4g_O12288_I6144_gs64 (default), i4g_O12288_I6144_gs128:
      one qgemv_i4g call (grouped int4, one activation vector)
  i4g_O12288_I6144_gs64_S2, _S4, fp8b128_O7168_I16384_S2, _S4,
  mq4v2_O8192_I8192_S2, _S4:
      the same step on 2 or 4 activation vectors per call (multi-token decode)
  fp8b128_O7168_I16384:
      one qgemv_fp8b128 call
  mq4v1_O8192_I8192, mq4c_O8192_I8192:
      qgemv_fwht256 then qgemv_mq4v1 / qgemv_mq4c (MQ4 v1 and the MQ4C pad
      form on the same shape)
  fp8ue8m0_O7168_I16384:
      one qgemv_fp8b128_ue8m0 call (the same weights with power-of-two
      UE8M0 block scale bytes)
  mq4v2_O8192_I8192:
      one qgemv_mq4v2_rot call (the FWHT-256 rotation of x fused into the
      GEMV; the same result as qgemv_fwht256 followed by qgemv_mq4v2), also
      for _S2; the _S4 step calls qgemv_fwht256 then qgemv_mq4v2
  moe_E256_O2048_I7168_gs64_T4_K8:
      one qgemv_moe_topk call (4 tokens, top-8 of 256 experts)
  i4g_prefill_O12288_I6144_gs64_S256, _S2048:
      one qgemv_i4g_prefill call (256 or 2048 prompt tokens through the
      grouped-int4 matrix on f32 MFMA; its roofline is the matrix cores')

Dense steps rotate through distinct weight copies totalling over 1 GiB, and
the routed-expert step cycles through 16 seeded routings over one resident
2.1 GB expert stack, so calls stream their weights from HBM rather than the
256 MB last-level cache.  All inputs are resident in HBM before timing.

Prints one JSON line.  `value` is the algorithmic bytes of K steps divided by
the time between two HIP events bracketing them on the launch stream;
`roofline.achieved` is the same for the step's kernel launches (one launch
per vector group, except the rotation launch of the multi-vector MQ4 steps).
`--copy-calibrate` instead runs a plain device-to-device copy of known size
(used to scale the HBM traffic counters).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFS = 157.3   # dense f32 matrix-core peak
DENSE_27B = 27e9   # weights of the dense decode fixture the tok/s figure is scaled to
ROTATE_BYTES = 1 << 30
METRIC = "achieved HBM GB/s (% of MI355X peak) + equiv decode tok/s, batch-1 qGEMV"


def n_copies(bytes_per_copy):
    return max(2, int(np.ceil(ROTATE_BYTES / bytes_per_copy)))


class Case:
    """A workload: builds device inputs, runs one step, checks parity."""
    name = ""
    kernel = ""            # name fragment of the dominant kernel
    fmt_desc = ""

    def step(self, i):
        raise NotImplementedError


def _check(rel, what):
    if not rel <= 1e-5:
        raise SystemExit(f"bench: {what}: GPU result disagrees with the oracle (rel L2 {rel:.3e})")


def _rel(got, ref):
    return float(np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref))


class I4G(Case):
    kernel = "i4g_gemv_stream"

    def __init__(self, O, I, gs, torch, q, o, S=1):
        import workloads as W
        self.name = f"i4g_O{O}_I{I}_gs{gs}" + (f"_S{S}" if S > 1 else "")
        # four vectors in whole 64-column blocks run on the int8 matrix cores
        if S == 4 and I % 64 == 0 and gs % 64 == 0:
            self.kernel = "i4g_gemv_mv"
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
        self.ws = [torch.from_numpy(d["w"]).to(dev)]
        self.ss = [torch.from_numpy(d["scales"]).to(dev)]
        for _ in range(1, self.n):
            self.ws.append(torch.randint(0, 256, d["w"].shape, dtype=torch.uint8, device=dev,
                                         generator=g))
            self.ss.append(0.002 + 0.018 * torch.rand(d["scales"].shape, device=dev, generator=g))
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [(w.data_ptr(), s.data_ptr()) for w, s in zip(self.ws, self.ss)]
        self.step(0)
        self.rel = _rel(self.y.cpu().numpy(), o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs))
        _check(self.rel, self.name)
        self.cpu = lambda: o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs)

    def step(self, i):
        wp, spp = self.ptrs[i % self.n]
        st = self.q.qgemv_i4g(wp, spp, self.x.data_ptr(), self.y.data_ptr(), self.S, self.I,
                              self.O, self.gs, self.sp)
        if st:
            raise SystemExit(f"qgemv_i4g: {self.q.strerror(st)}")


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
        self.step(0)
        rows = np.arange(0, O, 97)
        self.rel = _rel(self.y.cpu().numpy()[:, rows],
                        o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs, rows=rows))
        _check(self.rel, self.name)
        self.cpu_frac = len(rows) / O
        self.cpu = lambda: o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs, rows=rows)

    def step(self, i):
        st = self.q.qgemv_i4g_prefill(self.w.data_ptr(), self.s.data_ptr(), self.x.data_ptr(),
                                      self.y.data_ptr(), self.S, self.I, self.O, self.gs, self.sp)
        if st:
            raise SystemExit(f"qgemv_i4g_prefill: {self.q.strerror(st)}")


class FP8(Case):
    kernel = "fp8_gemv_stream"

    def __init__(self, O, I, torch, q, o, S=1):
        import workloads as W
        self.name = f"fp8b128_O{O}_I{I}" + (f"_S{S}" if S > 1 else "")
        self.fmt_desc = ("fp8 e4m3, f32 scale per 128x128 block"
                         + (f", {S} vectors per call" if S > 1 else ""))
        self.O, self.I, self.S = O, I, S
        nbo, nbi = W.fp8_nblocks(O, I)
        self.weight_bytes = O * I + nbo * nbi * 4
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4)
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = W.gen_fp8b128(O, I, S=S, seed=0)
        self.n = n_copies(self.weight_bytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        self.ws = [torch.from_numpy(d["w"]).to(dev)]
        self.ss = [torch.from_numpy(d["scale_inv"]).to(dev)]
        for _ in range(1, self.n):
            # uniform over the 254 non-NaN codes: v in 0..253 -> v + (v >= 0x7F)
            v = torch.randint(0, 254, (O, I), dtype=torch.uint8, device=dev, generator=g)
            self.ws.append(v + (v >= 0x7F).to(torch.uint8))
            self.ss.append(torch.exp(np.log(1e-4) + (np.log(1e-2) - np.log(1e-4)) *
                                     torch.rand((nbo, nbi), device=dev, generator=g)))
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [(w.data_ptr(), s.data_ptr()) for w, s in zip(self.ws, self.ss)]
        self.step(0)
        self.rel = _rel(self.y.cpu().numpy(), o.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I))
        _check(self.rel, self.name)
        self.cpu = lambda: o.fp8b128_gemv(d["w"], d["scale_inv"], d["x"], O, I)

    def step(self, i):
        wp, spp = self.ptrs[i % self.n]
        st = self.q.qgemv_fp8b128(wp, spp, self.x.data_ptr(), self.y.data_ptr(), self.S, self.I,
                                  self.O, self.sp)
        if st:
            raise SystemExit(f"qgemv_fp8b128: {self.q.strerror(st)}")


class FP8E8(Case):
    """fp8-e4m3 with UE8M0 (one power-of-two byte per 128x128 block) scales."""
    kernel = "fp8_gemv_stream"

    def __init__(self, O, I, torch, q, o, S=1):
        import workloads as W
        self.name = f"fp8ue8m0_O{O}_I{I}" + (f"_S{S}" if S > 1 else "")
        self.fmt_desc = ("fp8 e4m3, UE8M0 scale byte per 128x128 block"
                         + (f", {S} vectors per call" if S > 1 else ""))
        self.O, self.I, self.S = O, I, S
        nbo, nbi = W.fp8_nblocks(O, I)
        self.weight_bytes = O * I + nbo * nbi
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4)
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = W.gen_fp8ue8m0(O, I, S=S, seed=0)
        self.n = n_copies(self.weight_bytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        self.ws = [torch.from_numpy(d["w"]).to(dev)]
        self.ss = [torch.from_numpy(d["scale_e8m0"]).to(dev)]
        for _ in range(1, self.n):
            v = torch.randint(0, 254, (O, I), dtype=torch.uint8, device=dev, generator=g)
            self.ws.append(v + (v >= 0x7F).to(torch.uint8))
            self.ss.append(torch.randint(114, 121, (nbo, nbi), dtype=torch.uint8, device=dev,
                                         generator=g))
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [(w.data_ptr(), s.data_ptr()) for w, s in zip(self.ws, self.ss)]
        self.step(0)
        ref = o.fp8ue8m0_gemv(d["w"], d["scale_e8m0"], d["x"], O, I)
        self.rel = _rel(self.y.cpu().numpy(), ref)
        _check(self.rel, self.name)
        self.cpu = lambda: o.fp8ue8m0_gemv(d["w"], d["scale_e8m0"], d["x"], O, I)

    def step(self, i):
        wp, spp = self.ptrs[i % self.n]
        st = self.q.qgemv_fp8b128_ue8m0(wp, spp, self.x.data_ptr(), self.y.data_ptr(), self.S,
                                        self.I, self.O, self.sp)
        if st:
            raise SystemExit(f"qgemv_fp8b128_ue8m0: {self.q.strerror(st)}")


class MQ4(Case):
    kernel = "mq4v2_gemv_stream"

    FORMATS = {
        "v2": ("mq4v2", "MQ4-v2 136 B / 256 weights (fp16 scale+zero per 128)"),
        "v1": ("mq4v1", "MQ4 v1 136 B / 256 weights (f32 scale+zero per 256)"),
        "c": ("mq4c", "MQ4C pad 136 B / 256 weights (fp16 scale+zero per 256)"),
    }

    def __init__(self, O, I, torch, q, o, S=1, fmt="v2"):
        import workloads as W
        self.fmt = fmt
        tag, desc = self.FORMATS[fmt]
        self.name = f"{tag}_O{O}_I{I}" + (f"_S{S}" if S > 1 else "")
        self.fmt_desc = (desc + ", FWHT-256 rotated activations"
                         + (f", {S} vectors per call" if S > 1 else ""))
        self.O, self.I, self.S = O, I, S
        self.weight_bytes = O * (I // 256) * 136
        # up to two vectors: one fused launch (weights, x, signs in; y out),
        # the rotated activations never leave the chip.  Four: the rotation
        # kernel (x, signs in; x_rot out) then the GEMV (weights, x_rot in;
        # y out) -- every workgroup of the fused kernel rotates all S
        # vectors, which at S = 4 costs more than the extra launch
        self.alg_bytes = self.weight_bytes + S * (I * 4 + O * 4) + I
        if S > 2 or fmt != "v2":
            self.alg_bytes += S * I * 8
        self.bytes_per_weight = self.weight_bytes / (O * I)
        dev = torch.device("cuda:0")
        d = {"v2": W.gen_mq4v2, "v1": W.gen_mq4v1, "c": W.gen_mq4c}[fmt](O, I, S=S, seed=0)
        self.n = n_copies(self.weight_bytes)
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        w0 = torch.from_numpy(d["w"].reshape(O, -1)).to(dev)
        self.ws = [w0]
        for _ in range(1, self.n):
            # another draw: fresh payload, headers from copy 0 with their
            # scale/zero halves re-paired at random (same value ranges)
            w = w0.clone()
            pay = torch.randint(0, 256, (O, I // 256, 128), dtype=torch.uint8, device=dev,
                                generator=g)
            w.view(O, I // 256, 136)[:, :, 8:] = pay
            perm = torch.randperm(O, device=dev, generator=g)
            w.view(O, I // 256, 136)[:, :, :8] = w0.view(O, I // 256, 136)[perm, :, :8]
            self.ws.append(w)
        self.x = torch.from_numpy(d["x"]).to(dev)
        self.signs = torch.from_numpy(d["signs"]).to(dev)
        self.xr = torch.empty_like(self.x)
        self.y = torch.empty((S, O), dtype=torch.float32, device=dev)
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.ptrs = [w.data_ptr() for w in self.ws]
        self.step(0)
        ref_fn = {"v2": o.mq4v2_gemv, "v1": o.mq4v1_gemv, "c": o.mq4c_gemv}[fmt]
        ref = ref_fn(d["w"], o.fwht256(d["x"], d["signs"], I), O, I)
        self.rel = _rel(self.y.cpu().numpy(), ref)
        _check(self.rel, self.name)
        self.cpu = lambda: ref_fn(d["w"], o.fwht256(d["x"], d["signs"], I), O, I)

    def step(self, i):
        q = self.q
        if self.S <= 2 and self.fmt == "v2":
            st = q.qgemv_mq4v2_rot(self.ptrs[i % self.n], self.x.data_ptr(),
                                   self.signs.data_ptr(), self.y.data_ptr(), self.S, self.I,
                                   self.O, self.sp)
        else:
            st = q.qgemv_fwht256(self.x.data_ptr(), self.signs.data_ptr(), self.xr.data_ptr(),
                                 self.S, self.I, self.sp)
            gemv = {"v2": q.qgemv_mq4v2, "v1": q.qgemv_mq4v1, "c": q.qgemv_mq4c}[self.fmt]
            st = st or gemv(self.ptrs[i % self.n], self.xr.data_ptr(), self.y.data_ptr(), self.S,
                            self.I, self.O, self.sp)
        if st:
            raise SystemExit(f"mq4v2 step: {q.strerror(st)}")


class MoE(Case):
    kernel = "moe_i4g_stream"
    N_ROUTINGS = 16

    def __init__(self, E, O, I, gs, T, K, torch, q, o):
        import workloads as W
        self.name = f"moe_E{E}_O{O}_I{I}_gs{gs}_T{T}_K{K}"
        self.fmt_desc = "routed grouped-int4 experts, gate-weighted top-k sum"
        self.E, self.O, self.I, self.gs, self.T, self.K = E, O, I, gs, T, K
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
        self.routings = []
        uniq = []
        for r in range(self.N_ROUTINGS):
            ids, gates = (d["ids"], d["gates"]) if r == 0 else W.gen_moe_routing(E, T, K, 1000 + r)
            self.routings.append((torch.from_numpy(ids).to(dev), torch.from_numpy(gates).to(dev)))
            uniq.append(len(np.unique(ids)))
        self.uniq = uniq
        small = T * I * 4 + T * O * 4 + T * K * 8
        self.alg_bytes_per_routing = [u * self.expert_bytes + small for u in uniq]
        self.alg_bytes = float(np.mean(self.alg_bytes_per_routing))
        self.weight_bytes = float(np.mean(uniq)) * self.expert_bytes
        self.q, self.sp = q, torch.cuda.current_stream().cuda_stream
        self.step(0)
        rows = np.random.default_rng(0).choice(O, 64, replace=False)
        ref = o.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], E, O, I, gs, rows=rows)
        self.rel = _rel(self.y.cpu().numpy()[:, rows], ref)
        _check(self.rel, self.name)
        self.cpu_rows = rows
        self.cpu = lambda: o.moe_i4g(d["w"], d["scales"], d["ids"], d["gates"], d["x"], E, O, I,
                                     gs, rows=rows)

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


def build_case(name, torch, q, o):
    table = {
        "i4g_O12288_I6144_gs64": lambda: I4G(12288, 6144, 64, torch, q, o),
        "i4g_O12288_I6144_gs128": lambda: I4G(12288, 6144, 128, torch, q, o),
        "fp8b128_O7168_I16384": lambda: FP8(7168, 16384, torch, q, o),
        "mq4v2_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o),
        "moe_E256_O2048_I7168_gs64_T4_K8": lambda: MoE(256, 2048, 7168, 64, 4, 8, torch, q, o),
        "i4g_O256_I512_gs64": lambda: I4G(256, 512, 64, torch, q, o),
        "i4g_O12288_I6144_gs64_S2": lambda: I4G(12288, 6144, 64, torch, q, o, S=2),
        "i4g_prefill_O12288_I6144_gs64_S256": lambda: Prefill(12288, 6144, 64, 256, torch, q, o),
        "i4g_prefill_O12288_I6144_gs64_S2048": lambda: Prefill(12288, 6144, 64, 2048, torch, q,
                                                               o),
        "i4g_O12288_I6144_gs64_S4": lambda: I4G(12288, 6144, 64, torch, q, o, S=4),
        "fp8b128_O7168_I16384_S2": lambda: FP8(7168, 16384, torch, q, o, S=2),
        "fp8b128_O7168_I16384_S4": lambda: FP8(7168, 16384, torch, q, o, S=4),
        "mq4v2_O8192_I8192_S2": lambda: MQ4(8192, 8192, torch, q, o, S=2),
        "mq4v2_O8192_I8192_S4": lambda: MQ4(8192, 8192, torch, q, o, S=4),
        "fp8ue8m0_O7168_I16384": lambda: FP8E8(7168, 16384, torch, q, o),
        "mq4v1_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o, fmt="v1"),
        "mq4c_O8192_I8192": lambda: MQ4(8192, 8192, torch, q, o, fmt="c"),
    }
    return table[name]()


CASE_NAMES = ["i4g_O12288_I6144_gs64", "i4g_O12288_I6144_gs128", "fp8b128_O7168_I16384",
              "mq4v2_O8192_I8192", "moe_E256_O2048_I7168_gs64_T4_K8", "i4g_O256_I512_gs64",
              "i4g_O12288_I6144_gs64_S2", "i4g_O12288_I6144_gs64_S4",
              "fp8b128_O7168_I16384_S2", "fp8b128_O7168_I16384_S4",
              "mq4v2_O8192_I8192_S2", "mq4v2_O8192_I8192_S4", "fp8ue8m0_O7168_I16384",
              "mq4v1_O8192_I8192", "mq4c_O8192_I8192", "i4g_prefill_O12288_I6144_gs64_S256",
              "i4g_prefill_O12288_I6144_gs64_S2048"]


KERNEL_SOURCES = {
    "i4g_gemv_stream": "i4g.hip",
    "i4g_gemv_mv": "i4g.hip",
    "fp8_gemv_stream": "fp8b128.hip",
    "mq4v2_gemv_stream": "mq4v2.hip",
    "moe_i4g_stream": "moe.hip",
    "i4g_gemm_mfma": "prefill.hip",
}


def kernel_digest(kernel):
    """sha256 over the sources that define `kernel` (its file and the shared headers)."""
    import hashlib
    csrc = os.path.join(ROOT, "quantized_weight_decode_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "qg_device.h", "qg_launch.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def profiled_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary of this kernel on this
    workload, or None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    digest = traffic = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("source digest: sha256:"):
                digest = line.split(":", 2)[2].strip()
            elif line.startswith("traffic per dispatch"):
                traffic = int(line.rsplit(":", 1)[1].split()[0])
    if digest != kernel_digest(kernel):
        return None
    return traffic


def timed(torch, fn, first, k):
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(k):
        fn(first + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)  # ms


def cpu_baseline(case, budget_s=12.0):
    """The oracle as it stands, on the host's cores (OpenMP over rows)."""
    import oracle
    o = oracle.load()
    cores = min(os.cpu_count() or 1, 16)
    o.set_threads(cores)
    case.cpu()  # warm-up
    n = 0
    t0 = time.perf_counter()
    while True:
        case.cpu()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    o.set_threads(1)
    if isinstance(case, MoE):
        frac = len(case.cpu_rows) / case.O
        per_call = case.alg_bytes_per_routing[0] * frac
        sample = (f"{n} routed-expert calls restricted to {len(case.cpu_rows)} of {case.O} output "
                  f"rows (routing seed 0) in {el:.1f} s")
    else:
        frac = getattr(case, "cpu_frac", 1.0)
        per_call = case.alg_bytes * frac
        part = "full GEMVs" if frac == 1.0 else f"calls on {frac:.2%} of the output rows"
        sample = f"{n} {part} of {case.name} in {el:.1f} s ({el / n * 1e3:.1f} ms each)"
    return {"value": round(per_call * n / el / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "sample": sample + ", f64 accumulate"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    # the GPU reaches its steady clocks only after some milliseconds of load:
    # the first few hundred calls run 5-15 % slower
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--case", default="i4g_O12288_I6144_gs64", choices=CASE_NAMES)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only time a plain device copy of BYTES bytes")
    args = ap.parse_args()

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

    case = build_case(args.case, torch, q, oracle.load())
    for i in range(args.warmup):
        case.step(i)
    ms = timed(torch, case.step, args.warmup, args.steps)
    ms_step = ms / args.steps
    if isinstance(case, MoE):
        step_bytes = case.bytes_for(args.warmup, args.steps) / args.steps
    else:
        step_bytes = case.alg_bytes
    gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # the dominant kernel is the step's one launch
    kms, kbytes = ms_step, step_bytes
    kgbs = kbytes / (kms * 1e-3) / 1e9
    wgbs = case.weight_bytes / (kms * 1e-3) / 1e9

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": case.name, "batch": getattr(case, "S", 1), "format": case.fmt_desc,
                   "alg_bytes_per_step": round(step_bytes)},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "weights_gbs": round(wgbs, 1),
        "equiv_decode_tok_s": round(wgbs * 1e9 / (DENSE_27B * case.bytes_per_weight), 1),
        "roofline": {"bound": "hbm", "kernel": case.kernel, "achieved": round(kgbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "us_per_launch": round(kms * 1e3, 3), "alg_bytes_per_launch": round(kbytes),
                     "traffic": profiled_traffic(case.kernel, case.name)},
        "parity_rel_l2": case.rel,
    }
    if getattr(case, "bound", "hbm") == "mfma":
        tf = case.alg_flops / (kms * 1e-3) / 1e12
        out["roofline"].update({"bound": "mfma", "achieved": round(tf, 2),
                                "peak": MFMA_F32_PEAK_TFS, "unit": "TFLOP/s",
                                "frac": round(tf / MFMA_F32_PEAK_TFS, 4),
                                "alg_flops_per_launch": case.alg_flops})
    if isinstance(case, MoE):
        out["config"]["distinct_experts_per_routing"] = case.uniq
        out["tokens_per_s"] = round(case.T / (ms_step * 1e-3), 1)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
