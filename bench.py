#!/usr/bin/env python3
"""Batch-1 quantized-weight GEMV benchmark on one MI355X.

A step is one pass of the hot path over one batch: for the grouped-int4
resident projection (O=12288, I=6144, gs=64, one activation vector) one
qgemv_i4g call.  Steps rotate through distinct weight copies totalling over
1 GiB so that every call streams its weights from HBM, not from the 256 MB
last-level cache.  Inputs are resident in HBM before timing starts.

Prints one JSON line:
  value            algorithmic bytes moved per second (GB/s) over the timed
                   region (K steps between two events on the launch stream)
  roofline         the GEMV kernel's algorithmic bytes / its average launch
                   duration against the 8 TB/s HBM peak
  cpu_baseline     the CPU oracle on a bounded sample of the same workload
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
DENSE_27B = 27e9   # weights of the dense decode fixture the tok/s figure is scaled to


def i4g_case(O, I, gs):
    rb = (I + 1) // 2
    ng = (I + gs - 1) // gs
    wbytes = O * rb + O * ng * 4          # packed nibbles + f32 scales
    total = wbytes + I * 4 + O * 4        # + x + y
    return {"workload": f"i4g_O{O}_I{I}_gs{gs}", "fmt": "i4g", "O": O, "I": I, "gs": gs,
            "weight_bytes": wbytes, "alg_bytes": total,
            "bytes_per_weight": wbytes / (O * I)}


CASES = {
    "i4g_O12288_I6144_gs64": lambda: i4g_case(12288, 6144, 64),
    "i4g_O12288_I6144_gs128": lambda: i4g_case(12288, 6144, 128),
}


def make_copies(case, n_copies, torch, dev):
    """Copy 0 from the seeded generator (checked against the oracle); the rest
    are distinct seeded draws made on the device, same distributions."""
    import workloads as W
    O, I, gs = case["O"], case["I"], case["gs"]
    d = W.gen_i4g(O, I, gs, seed=0)
    ws = [torch.from_numpy(d["w"]).to(dev)]
    ss = [torch.from_numpy(d["scales"]).to(dev)]
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    for _ in range(1, n_copies):
        ws.append(torch.randint(0, 256, d["w"].shape, dtype=torch.uint8, device=dev, generator=g))
        ss.append((0.002 + 0.018 * torch.rand(d["scales"].shape, device=dev, generator=g)).float())
    x = torch.from_numpy(d["x"]).to(dev)
    return d, ws, ss, x


def cpu_baseline(case, d, budget_s=12.0):
    """The oracle as it stands, on all host cores (OpenMP over rows)."""
    import oracle
    o = oracle.load()
    cores = min(os.cpu_count() or 1, 16)
    o.set_threads(cores)
    O, I, gs = case["O"], case["I"], case["gs"]
    o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs)  # warm-up
    n = 0
    t0 = time.perf_counter()
    while True:
        o.i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    o.set_threads(1)
    return {"value": case["alg_bytes"] * n / el / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{n} full GEMVs of {case['workload']} in {el:.1f} s "
                      f"({el / n * 1e3:.1f} ms each, f64 accumulate)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--case", default="i4g_O12288_I6144_gs64", choices=sorted(CASES))
    ap.add_argument("--copies-gib", type=float, default=1.0,
                    help="total size of the rotated weight copies")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the row-sharded multi-GPU layout is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_weight_decode_amd as q
    import oracle

    dev = torch.device("cuda:0")
    case = CASES[args.case]()
    per_copy = case["weight_bytes"]
    n_copies = max(2, int(np.ceil(args.copies_gib * (1 << 30) / per_copy)))
    d, ws, ss, x = make_copies(case, n_copies, torch, dev)
    O, I, gs = case["O"], case["I"], case["gs"]
    y = torch.empty((1, O), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    # correctness of the timed configuration: copy 0 against the oracle
    q.i4g(ws[0], ss[0], x, gs, out=y)
    ref = oracle.load().i4g_gemv(d["w"], d["scales"], d["x"], O, I, gs)
    got = y.cpu().numpy()
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    if not rel <= 1e-5:
        raise SystemExit(f"bench: GPU result disagrees with the oracle (rel L2 {rel:.3e})")

    ptrs = [(w.data_ptr(), s.data_ptr()) for w, s in zip(ws, ss)]
    xp, yp = x.data_ptr(), y.data_ptr()

    def step(i):
        wp, spp = ptrs[i % n_copies]
        st = q.qgemv_i4g(wp, spp, xp, yp, 1, I, O, gs, sp)
        if st:
            raise SystemExit(f"qgemv_i4g failed: {q.strerror(st)}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    gbs = case["alg_bytes"] / (ms * 1e-3) / 1e9
    wgbs = case["weight_bytes"] / (ms * 1e-3) / 1e9
    out = {
        "metric": "achieved HBM GB/s (% of MI355X peak) + equiv decode tok/s, batch-1 qGEMV",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": case["workload"], "batch": 1, "format": "grouped int4, f32 scales",
                   "rotated_copies": n_copies, "alg_bytes_per_step": case["alg_bytes"]},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "weights_gbs": round(wgbs, 1),
        "equiv_decode_tok_s": round(wgbs * 1e9 / (DENSE_27B * case["bytes_per_weight"]), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "parity_rel_l2": rel,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(case, d)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
