#!/usr/bin/env python3
"""Benchmark of the pooled bidirectional selective-scan layer on one MI355X.

One step = one call of the whole layer (pool, x_proj, step size + both scans,
repeat + skip + gate) on the 2048^2 FastVim-T workload: B = 128 images of a
128 x 128 token grid, E = 384, N = 16, R = 12, fp32, pooled over columns,
inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-extras]

Besides the headline images/s it reports the per-stage kernel times, the
roofline of the dominant kernel (the streaming epilogue: x and z read once,
out written once), a plain device-copy ceiling, the unpooled layer on the same
inputs (scan over all h*w tokens) for the pooling speedup, and the fp64 CPU
oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "pooled SSM layer images/s + % HBM peak at 2048² (h=w=128) fp32, B=128"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the unpooled / copy-ceiling measurements")
    ap.add_argument("--cpu-images", type=int, default=64, help="images in the oracle's timed sample")
    return ap.parse_args()


def timed(fn, n, stream):
    """Average ms of fn() over n calls, HIP events on ``stream``."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / n


def cpu_baseline(wl, n_img):
    """fp64 oracle (as it stands) on the first n_img images of the workload."""
    import oracle
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    n_img = min(n_img, x.shape[0])
    xs, zs = x[:n_img], z[:n_img]
    t0 = time.perf_counter()
    oracle.layer(xs, zs, prm["fwd"], prm["bwd"], oracle.COLS)
    dt = time.perf_counter() - t0
    return {"value": n_img / dt, "unit": "images/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "first %d of %d images of the same seeded workload, full layer in fp64 (%.2f s wall)"
                      % (n_img, x.shape[0], dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (batch sharding across GPUs is "
              "described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import pooled_selective_state_amd as P
    from pooled_selective_state_amd import configs as C
    from pooled_selective_state_amd.inputs import draw_workload

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    P.lib()
    cfg = C.HIRES_2048
    t0 = time.perf_counter()
    wl = draw_workload(cfg)
    print("[bench] inputs drawn in %.1f s" % (time.perf_counter() - t0), file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(wl["x"]).to(dev)
    z = torch.from_numpy(wl["z"][0]).to(dev)
    prm = {d: {k: torch.from_numpy(v).to(dev) for k, v in wl["params"][0][d].items()} for d in ("fwd", "bwd")}
    stream = torch.cuda.current_stream()
    call = P.SSMCall(x, z, prm, P.POOL_COLS)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        call.run(stream)
    torch.cuda.synchronize()
    ms = timed(lambda: call.run(stream), args.steps, stream)
    torch.cuda.synchronize()
    print("[bench] layer %.3f ms/step" % ms, file=sys.stderr, flush=True)

    elems = cfg.B * cfg.h * cfg.w * cfg.E
    alg_bytes = 3 * 4 * elems  # x read once, z read once, out written once
    stages = {}
    for name, sid in (("pool", P.STAGE_POOL), ("proj", P.STAGE_PROJ), ("scan", P.STAGE_SCAN),
                      ("epilogue", P.STAGE_EPILOGUE)):
        stages[name] = timed(lambda: call.stage(sid, stream), max(3, args.steps // 2), stream)
    torch.cuda.synchronize()
    epi_ms = stages["epilogue"]
    epi_gbs = alg_bytes / (epi_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": cfg.B / (ms * 1e-3),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "h": cfg.h, "w": cfg.w, "E": cfg.E, "N": cfg.N, "R": cfg.R,
                   "pool_axis": "cols", "seed": 0},
        "tokens_per_s": cfg.B * cfg.h * cfg.w / (ms * 1e-3),
        "layer_hbm_frac": alg_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "stage_ms": stages,
        "roofline": {"bound": "hbm", "kernel": "epilogue (repeat + skip + gate)", "achieved": epi_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": epi_gbs / HBM_PEAK_GBS, "traffic": None},
    }

    if not args.no_extras:
        # Plain device copy of one input-sized buffer: a practical streaming ceiling.
        dst = torch.empty_like(x)
        cp_ms = timed(lambda: dst.copy_(x), 5, stream)
        result["copy_ceiling_GBps"] = 2 * 4 * elems / (cp_ms * 1e-3) / 1e9
        del dst
        # Unpooled layer on the same inputs: scan over all h*w tokens.
        ucall = P.SSMCall(x, z, prm, P.POOL_NONE_ROWMAJOR)
        ucall.run(stream)
        torch.cuda.synchronize()
        u_ms = timed(lambda: ucall.run(stream), 3, stream)
        u_scan = timed(lambda: ucall.stage(P.STAGE_SCAN, stream), 3, stream)
        u_proj = timed(lambda: ucall.stage(P.STAGE_PROJ, stream), 3, stream)
        torch.cuda.synchronize()
        result["unpooled"] = {"layer_ms": u_ms, "scan_ms": u_scan, "proj_ms": u_proj, "T": cfg.h * cfg.w,
                              "layer_speedup": u_ms / ms, "scan_speedup": u_scan / stages["scan"]}
        del ucall
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_images)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
