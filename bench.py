#!/usr/bin/env python3
"""Benchmark of the pooled bidirectional selective-scan layer on one MI355X.

One step = one call of the whole layer -- pool, x_proj, step sizes and both
scans, repeat + skip + gate -- on the 2048^2 FastVim-T workload: B = 128
images of a 128 x 128 token grid, E = 384, N = 16, R = 12, fp32, pooled over
columns, inputs already resident in HBM.  The layer runs as the library's
default path, one pipelined kernel launch (plus a one-block launch that resets
its counters).  Prints one JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extras] [--no-cpu-baseline]
                    [--cpu-seconds S] [--profile-run] [--profile-bwd] [--profile-small]

Reported besides images/s:
  roofline      the single-launch kernel against the 8 TB/s HBM peak, with
                algorithmic bytes (x and z read once, out written once:
                12 B per grid element) over the measured step time, and the
                HBM traffic the hardware counters recorded for it, when the
                recorded counter summary belongs to the current kernel source;
  cpu_baseline  the fp64 CPU oracle on the same host arrays, cycled over the
                batch for at least --cpu-seconds (with the extras, also the
                oracle on one thread for the small workloads and on the
                unpooled layer, extrapolated from 8 images);
  extras        the stage-kernel path and its per-stage times, the other
                pooling axis, the layer with the post-SSM LayerNorm, the layer
                with the producer Conv1D fused, the backward pass, the
                unpooled layer (scan over all h*w tokens) with the pooled /
                unpooled ratios, LBMamba's local backward scan against the
                bidirectional one, the 1024^2 two-block chain, and the small
                workloads over rotating input sets.
--profile-run times a few steps and the calibration copy only (for profiler
runs); --profile-bwd adds three backward calls of the same workload, three
more given the pooled tokens a forward call saved, and three each with the
post-SSM LayerNorm, the local backward scan, the producer Conv1D and both the
Conv1D and the LayerNorm (pooled tokens saved).  --profile-small runs only the
small workloads (tiny, short-sequence, masked), a few calls of each form.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "pooled SSM layer images/s + % HBM peak at 2048² (h=w=128) fp32, B=128"
COUNTERS = os.path.join(ROOT, "profiles", "fused_layer_pooled_2048_T_b128_counters.md")
# the sources the single-launch kernel is compiled from (the counter summary is
# only valid for the exact text it was recorded with)
KERNEL_SOURCES = ("pooled_selective_state_amd/csrc/fused.hip", "pooled_selective_state_amd/csrc/scan_core.h",
                  "pooled_selective_state_amd/csrc/fastvim_internal.h", "include/fastvim.h",
                  "pooled_selective_state_amd/build.py")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU time of the oracle sample")
    ap.add_argument("--profile-run", action="store_true", help="layer steps and calibration copy only")
    ap.add_argument("--profile-bwd", action="store_true", help="with --profile-run: also three backward calls")
    ap.add_argument("--profile-small", action="store_true",
                    help="the small workloads only, a few calls each (for counter runs); prints their times")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_sources_sha256():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the single-launch kernel from the committed
    counter summary, or None if absent or recorded for other kernel sources."""
    if not os.path.exists(COUNTERS):
        return None, "no counter summary"
    text = open(COUNTERS).read()
    m_t = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)\s*$", text, re.M)
    m_h = re.search(r"^kernel_sources_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not (m_t and m_h):
        return None, "counter summary incomplete"
    if m_h.group(1) != kernel_sources_sha256():
        return None, "counter summary recorded for other kernel sources"
    return float(m_t.group(1)), os.path.relpath(COUNTERS, ROOT)


def time_steps(fn, k, stream):
    """Run fn() k times on ``stream`` with a HIP event between calls; returns
    (mean ms over the whole region, list of per-call ms)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(k):
        fn()
        ev[i + 1].record(stream)
    ev[k].synchronize()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[k]) / k, [ev[i].elapsed_time(ev[i + 1]) for i in range(k)]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, z, prm, axis, seconds):
    """The fp64 oracle as it stands, cycled over the batch in chunks of
    images until at least ``seconds`` have passed."""
    import oracle
    B = x.shape[0]
    threads = oracle.max_threads()
    chunk = min(B, max(8, threads))
    done, b = 0, 0
    t0 = time.perf_counter()
    while True:
        e = min(B, b + chunk)
        oracle.layer(x[b:e], z[b:e], prm["fwd"], prm["bwd"], axis)
        done += e - b
        b = 0 if e == B else e
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return {"value": done / dt, "unit": "images/s", "cores": min(threads, chunk), "kind": "oracle",
            "sample": "%d images (the batch of %d cycled in chunks of %d) of the same seeded host arrays, whole "
                      "layer in fp64, %.1f s wall; CPU %s" % (done, B, chunk, dt, cpu_model())}


def oracle_timings(C, wl_big, seconds=1.0):
    """The fp64 oracle on the other workloads: one thread on the small ones
    (whole layer, the chain's two blocks in turn), and the unpooled 2048^2
    layer on 8 images with all threads, extrapolated to the batch (linear in
    B: images are independent)."""
    import oracle
    from pooled_selective_state_amd.inputs import draw_workload
    out = {}
    full = oracle.max_threads()

    def rate(fn, n_img):
        done, t0 = 0, time.perf_counter()
        while True:
            fn()
            done += n_img
            dt = time.perf_counter() - t0
            if dt >= seconds:
                return done / dt
    try:
        oracle.set_threads(1)
        for cfg, batch in ((C.TINY, None), (C.SHORT_224_S, None), (C.CHAIN_1024, 8), (C.MASKED_B, 32)):
            wl = draw_workload(cfg, batch=batch)
            x, zs, ps, idx = wl["x"], wl["z"], wl["params"], wl["idx"]
            hw = (cfg.h, cfg.w) if cfg.masked else None

            def run():
                y = x
                for k, axis in enumerate(cfg.axes):
                    y = oracle.layer(y, zs[k], ps[k]["fwd"], ps[k]["bwd"], axis, idx=idx, hw=hw).astype(np.float32)
            out[cfg.name] = {"images_per_s": rate(run, wl["B"]), "threads": 1,
                             "sample": "%d images, %s" % (wl["B"], "two blocks" if len(cfg.axes) > 1 else "one layer")}
        oracle.set_threads(full)
        sel = slice(0, 8)
        t0 = time.perf_counter()
        oracle.layer(wl_big["x"][sel], wl_big["z"][0][sel], wl_big["params"][0]["fwd"], wl_big["params"][0]["bwd"], 2)
        dt = time.perf_counter() - t0
        B = wl_big["x"].shape[0]
        out["unpooled_2048"] = {"images_per_s": 8 / dt, "threads": min(full, 8), "seconds_for_8": dt,
                                "batch_seconds_extrapolated": dt * B / 8,
                                "sample": "8 of %d images, T = 16384, extrapolated (linear in B)" % B}
    finally:
        oracle.set_threads(full)
    return out


def small_configs(P, C, torch, stream, nsets=4, calls=200):
    """Throughput of the workloads that fit in the Infinity Cache: calls
    rotate over ``nsets`` input/output sets (together well over 256 MB), so
    no call finds its inputs cached by the one before."""
    from pooled_selective_state_amd.inputs import draw_dir_params, random_mask
    res = {}
    for cfg in (C.TINY, C.SHORT_224_S, C.MASKED_B):
        g = torch.Generator(device="cuda").manual_seed(0)
        rng = np.random.default_rng(0)
        dt = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
        shape = (cfg.B, cfg.K, cfg.E) if cfg.masked else (cfg.B, cfg.h, cfg.w, cfg.E)
        prm = {d: {k: torch.from_numpy(v).cuda() for k, v in draw_dir_params(rng, cfg.E, cfg.N, cfg.R).items()}
               for d in ("fwd", "bwd")}
        sets, two = [], []
        for _ in range(nsets):
            x = torch.randn(shape, device="cuda", generator=g).to(dt)
            z = torch.randn(shape, device="cuda", generator=g).to(dt)
            idx = (torch.from_numpy(random_mask(rng, cfg.B, cfg.h, cfg.w, cfg.K)).cuda() if cfg.masked else None)
            hw = (cfg.h, cfg.w) if cfg.masked else None
            sets.append(P.SSMCall(x, z, prm, P.POOL_COLS, mask_idx=idx, hw=hw))
            # the same layer with its scan and output stages as two launches
            two.append(P.SSMCall(x, z, prm, P.POOL_COLS, mask_idx=idx, hw=hw, out=sets[-1].out,
                                 workspace=sets[-1].workspace, tuning=P.tuning_scan_out(P.SCAN_OUT_TWO)))
        for c in sets + two:
            c.run(stream)
        k = [0]

        def rotate(calls_):
            def step():
                calls_[k[0] % nsets].run(stream)
                k[0] += 1
            return step
        ms, per = time_steps(rotate(sets), calls, stream)
        ms_two, _ = time_steps(rotate(two), calls, stream)
        res[cfg.name] = {"ms": ms, "ms_median": float(np.median(per)), "images_per_s": cfg.B / (ms * 1e-3),
                         "tokens_per_s": cfg.B * cfg.tokens_per_image / (ms * 1e-3),
                         "hbm_frac": cfg.io_bytes() / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), "dtype": cfg.io_dtype,
                         "path": "stage kernels, scan and output stages in one launch",
                         "ms_scan_and_output_two_launches": ms_two}
        del sets, two
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer has no multi-GPU path in this library (images are "
              "independent, so a batch shards across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.profile_run:
        args.no_extras = args.no_cpu_baseline = True

    import torch
    import pooled_selective_state_amd as P
    from pooled_selective_state_amd import configs as C
    from pooled_selective_state_amd.inputs import draw_workload

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    P.lib()  # raises if the HIP library is not built
    if args.profile_small:
        # the tiny, short-sequence and masked workloads, each form of their
        # scan and output stages, a few calls each (counter runs)
        res = small_configs(P, C, torch, torch.cuda.current_stream(), nsets=2, calls=4)
        print(json.dumps({"profile_small": res}), flush=True)
        return
    cfg = C.HIRES_2048
    t0 = time.perf_counter()
    wl = draw_workload(cfg)
    log("inputs drawn in %.1f s" % (time.perf_counter() - t0))
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
    ms, per = time_steps(lambda: call.run(stream), args.steps, stream)
    status = int(call.export(P.EXPORT_STATUS, stream).item())
    if status:
        raise RuntimeError("single-launch kernel reported status %#x (a bounded wait gave up)" % status)
    log("layer %.4f ms/step (median %.4f, min %.4f)" % (ms, float(np.median(per)), min(per)))

    elems = cfg.B * cfg.h * cfg.w * cfg.E
    alg_bytes = 3 * 4 * elems  # x read once, z read once, out written once (fp32)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    traffic, traffic_src = recorded_traffic()

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
        "data": "synthetic (seeded N(0,1) activations, pages' parameter recipe)",
        "config": {"workload": cfg.name, "B": cfg.B, "h": cfg.h, "w": cfg.w, "E": cfg.E, "N": cfg.N, "R": cfg.R,
                   "pool_axis": "cols", "path": "single launch", "seed": 0},
        "ms_median": float(np.median(per)),
        "ms_min": float(min(per)),
        "tokens_per_s": cfg.B * cfg.h * cfg.w / (ms * 1e-3),
        "hbm_frac": achieved / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": "fused_layer_kernel (whole layer, one launch per step)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_unit": "HBM bytes per launch", "traffic_source": traffic_src,
                     "alg_bytes_per_launch": alg_bytes},
    }

    # calibration copy of one input-sized buffer (also the counter scale run)
    dst = torch.empty_like(x)
    for _ in range(2):
        P.calib_copy(dst, x, stream)
    cp_ms, _ = time_steps(lambda: P.calib_copy(dst, x, stream), 3 if args.profile_run else 5, stream)
    result["copy_ceiling"] = {"GBps": 2 * 4 * elems / (cp_ms * 1e-3) / 1e9, "bytes_read": 4 * elems,
                              "bytes_written": 4 * elems, "ms": cp_ms, "kernel": "calib_copy_kernel"}
    del dst
    log("calibration copy %.4f ms (%.0f GB/s)" % (cp_ms, result["copy_ceiling"]["GBps"]))
    if args.profile_bwd:
        dout = torch.randn(x.shape, device=dev, generator=torch.Generator(device="cuda").manual_seed(2))
        su = torch.empty((cfg.B, cfg.h, cfg.E), device=dev)
        P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, saved_u=su).run(stream)
        g_ln = torch.Generator(device="cuda").manual_seed(1)
        ln = {"weight": 1.0 + 0.1 * torch.randn(cfg.E, device=dev, generator=g_ln),
              "bias": 0.1 * torch.randn(cfg.E, device=dev, generator=g_ln), "eps": 1e-5}
        conv = {"weight": 0.5 * torch.randn(cfg.E, P.CONV_TAPS, device=dev, generator=g_ln),
                "bias": 0.1 * torch.randn(cfg.E, device=dev, generator=g_ln)}
        for kept, lnk, cv, fl in ((None, None, None, 0), (su, None, None, 0), (su, ln, None, 0),
                                  (su, None, None, P.FLAG_LOCAL_BWD), (su, None, conv, 0), (su, ln, conv, 0)):
            bcall = P.BwdCall(x, z, dout, prm, P.POOL_COLS, saved_u=kept, ln=lnk, conv=cv, flags=fl)
            for _ in range(3):
                bcall.run(stream)
            torch.cuda.synchronize()
            del bcall
        del dout, su

    if not args.no_extras:
        extras = {}
        n = max(3, args.steps // 2)
        # the same layer as stage kernels
        scall = P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, flags=P.FLAG_STAGED)
        scall.run(stream)
        st_ms, _ = time_steps(lambda: scall.run(stream), n, stream)
        stages = {}
        for name, sid in (("pool", P.STAGE_POOL), ("proj", P.STAGE_PROJ), ("scan", P.STAGE_SCAN),
                          ("epilogue", P.STAGE_EPILOGUE)):
            stages[name], _ = time_steps(lambda: scall.stage(sid, stream), n, stream)
        extras["staged"] = {"layer_ms": st_ms, "stage_ms": stages}
        # the other pooling axis (the next block's orientation)
        rcall = P.SSMCall(x, z, prm, P.POOL_ROWS, workspace=call.workspace, out=call.out)
        rcall.run(stream)
        extras["rows_layer_ms"], _ = time_steps(lambda: rcall.run(stream), n, stream)
        # the layer with the post-SSM LayerNorm before the gate (stage kernels)
        g_ln = torch.Generator(device="cuda").manual_seed(1)
        ln = {"weight": 1.0 + 0.1 * torch.randn(cfg.E, device=dev, generator=g_ln),
              "bias": 0.1 * torch.randn(cfg.E, device=dev, generator=g_ln), "eps": 1e-5}
        norm = {}
        for name, fl in (("single_launch", P.FLAG_FUSED), ("stage_kernels", P.FLAG_STAGED)):
            ncall = P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, ln=ln, flags=fl)
            ncall.run(stream)
            norm[name + "_ms"], _ = time_steps(lambda: ncall.run(stream), n, stream)
            if fl == P.FLAG_STAGED:
                norm["epilogue_ms"], _ = time_steps(lambda: ncall.stage(P.STAGE_EPILOGUE, stream), n, stream)
                norm["epilogue_GBps"] = alg_bytes / (norm["epilogue_ms"] * 1e-3) / 1e9
            del ncall
        norm["single_launch_hbm_frac"] = alg_bytes / (norm["single_launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        extras["post_norm_2048"] = norm
        # the producer Conv1D + SiLU fused into the layer (x is the conv's input; stage kernels)
        conv = {"weight": 0.5 * torch.randn(cfg.E, P.CONV_TAPS, device=dev, generator=g_ln),
                "bias": 0.1 * torch.randn(cfg.E, device=dev, generator=g_ln)}
        ccall = P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, conv=conv)
        ccall.run(stream)
        cv_ms, _ = time_steps(lambda: ccall.run(stream), n, stream)
        del ccall
        cscall = P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, conv=conv,
                           flags=P.FLAG_STAGED)
        cscall.run(stream)
        cv_st, _ = time_steps(lambda: cscall.run(stream), n, stream)
        cv_pool, _ = time_steps(lambda: cscall.stage(P.STAGE_POOL, stream), n, stream)
        cv_epi, _ = time_steps(lambda: cscall.stage(P.STAGE_EPILOGUE, stream), n, stream)
        extras["conv_producer_2048"] = {"layer_ms": cv_ms, "path": "single launch, x_conv computed on load",
                                        "layer_GBps": alg_bytes / (cv_ms * 1e-3) / 1e9,
                                        "hbm_frac": alg_bytes / (cv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "stage_kernels_ms": cv_st, "pool_ms": cv_pool, "epilogue_ms": cv_epi,
                                        "pool_GBps": 4 * elems / (cv_pool * 1e-3) / 1e9,
                                        "epilogue_GBps": alg_bytes / (cv_epi * 1e-3) / 1e9}
        del cscall
        log("conv-fused layer %.3f ms (single launch), %.3f ms (stage kernels)" % (cv_ms, cv_st))
        # the whole FastVim block in one call: the producer Conv1D (written out
        # into out first) and the post-SSM LayerNorm between the skip and the gate
        blk = {"path": "the single launch, x_conv computed on load (both axes)"}
        for name, axis in (("cols", P.POOL_COLS), ("rows", P.POOL_ROWS)):
            bk = P.SSMCall(x, z, prm, axis, workspace=call.workspace, out=call.out, conv=conv, ln=ln)
            bk.run(stream)
            f_ms, _ = time_steps(lambda: bk.run(stream), n, stream)
            blk[name] = {"forward_ms": f_ms, "images_per_s": cfg.B / (f_ms * 1e-3),
                         "alg_GBps": alg_bytes / (f_ms * 1e-3) / 1e9,
                         "hbm_frac": alg_bytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del bk
        extras["block_conv_norm_2048"] = blk
        log("conv + norm block %.3f ms (cols), %.3f ms (rows)" % (blk["cols"]["forward_ms"], blk["rows"]["forward_ms"]))
        # bf16 I/O, both axes, on the default path (the single launch)
        xb16, zb16 = x.to(torch.bfloat16), z.to(torch.bfloat16)
        b16 = {}
        for name, axis in (("cols", P.POOL_COLS), ("rows", P.POOL_ROWS)):
            bc = P.SSMCall(xb16, zb16, prm, axis)
            bc.run(stream)
            f_ms, _ = time_steps(lambda: bc.run(stream), n, stream)
            b16[name] = {"ms": f_ms, "images_per_s": cfg.B / (f_ms * 1e-3),
                         "hbm_frac": (alg_bytes // 2) / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del bc
        extras["bf16_2048"] = b16
        del xb16, zb16
        # the backward pass (gradients of sum(dout * out)) on the same inputs
        g_b = torch.Generator(device="cuda").manual_seed(2)
        dout = torch.randn(x.shape, device=dev, generator=g_b)
        bwd_bytes = 5 * 4 * elems  # x, z, dout read once, dx, dz written once (fp32)
        extras["backward_2048"] = {"alg_bytes": bwd_bytes, "path": "stage kernels, two full-resolution passes",
                                   "saved_u": "pooled tokens kept from the forward call (pass 1 reads z and dout "
                                              "only); pools_x: the backward pools x again"}
        for name, axis in (("cols", P.POOL_COLS), ("rows", P.POOL_ROWS)):
            su = torch.empty((cfg.B, cfg.h if axis == P.POOL_COLS else cfg.w, cfg.E), device=dev)
            P.SSMCall(x, z, prm, axis, workspace=call.workspace, out=call.out, saved_u=su).run(stream)
            res = {}
            for kind, kept in (("pools_x", None), ("saved_u", su)):
                bcall = P.BwdCall(x, z, dout, prm, axis, saved_u=kept)
                bcall.run(stream)
                b_ms, _ = time_steps(lambda: bcall.run(stream), n, stream)
                res[kind] = {"ms": b_ms, "images_per_s": cfg.B / (b_ms * 1e-3),
                             "GBps": bwd_bytes / (b_ms * 1e-3) / 1e9,
                             "hbm_frac": bwd_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
                del bcall
            extras["backward_2048"][name] = res
            del su
        # with the post-SSM LayerNorm: the forward stages run first, the norm's
        # adjoint in the first pass, and the second pass turns g into dx in place
        su = torch.empty((cfg.B, cfg.h, cfg.E), device=dev)
        P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, saved_u=su, ln=ln).run(stream)
        res = {}
        for kind, kept in (("pools_x", None), ("saved_u", su)):
            bcall = P.BwdCall(x, z, dout, prm, P.POOL_COLS, saved_u=kept, ln=ln)
            bcall.run(stream)
            b_ms, _ = time_steps(lambda: bcall.run(stream), n, stream)
            res[kind] = {"ms": b_ms, "images_per_s": cfg.B / (b_ms * 1e-3),
                         "GBps": bwd_bytes / (b_ms * 1e-3) / 1e9,
                         "hbm_frac": bwd_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del bcall
        extras["backward_2048"]["post_norm_cols"] = res
        # with LBMamba's local backward scan (pooled tokens saved)
        bcall = P.BwdCall(x, z, dout, prm, P.POOL_COLS, saved_u=su, flags=P.FLAG_LOCAL_BWD)
        bcall.run(stream)
        b_ms, _ = time_steps(lambda: bcall.run(stream), n, stream)
        extras["backward_2048"]["local_scan_cols"] = {"saved_u": {
            "ms": b_ms, "images_per_s": cfg.B / (b_ms * 1e-3), "GBps": bwd_bytes / (b_ms * 1e-3) / 1e9,
            "hbm_frac": bwd_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        del bcall
        # with the producer Conv1D (x is the conv's input; pooled tokens saved by a conv forward call)
        P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, saved_u=su, conv=conv).run(stream)
        bcall = P.BwdCall(x, z, dout, prm, P.POOL_COLS, saved_u=su, conv=conv)
        bcall.run(stream)
        b_ms, _ = time_steps(lambda: bcall.run(stream), n, stream)
        extras["backward_2048"]["conv_producer_cols"] = {"saved_u": {
            "ms": b_ms, "images_per_s": cfg.B / (b_ms * 1e-3), "GBps": bwd_bytes / (b_ms * 1e-3) / 1e9,
            "hbm_frac": bwd_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        del bcall
        # the whole block (Conv1D and LayerNorm), pooled tokens saved by its forward call
        P.SSMCall(x, z, prm, P.POOL_COLS, workspace=call.workspace, out=call.out, saved_u=su, conv=conv,
                  ln=ln).run(stream)
        bcall = P.BwdCall(x, z, dout, prm, P.POOL_COLS, saved_u=su, conv=conv, ln=ln)
        bcall.run(stream)
        b_ms, _ = time_steps(lambda: bcall.run(stream), n, stream)
        extras["backward_2048"]["block_conv_norm_cols"] = {"saved_u": {
            "ms": b_ms, "images_per_s": cfg.B / (b_ms * 1e-3), "GBps": bwd_bytes / (b_ms * 1e-3) / 1e9,
            "hbm_frac": bwd_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        del bcall
        # bf16 I/O (x, z, dout, dx, dz in bf16; parameters and arithmetic fp32), pooled tokens saved
        xb, zb, db = (t.to(torch.bfloat16) for t in (x, z, dout))
        P.SSMCall(xb, zb, prm, P.POOL_COLS, saved_u=su).run(stream)
        bcall = P.BwdCall(xb, zb, db, prm, P.POOL_COLS, saved_u=su)
        bcall.run(stream)
        b_ms, _ = time_steps(lambda: bcall.run(stream), n, stream)
        bf_bytes = bwd_bytes // 2
        extras["backward_2048"]["bf16_cols"] = {"saved_u": {
            "ms": b_ms, "images_per_s": cfg.B / (b_ms * 1e-3), "alg_bytes": bf_bytes,
            "GBps": bf_bytes / (b_ms * 1e-3) / 1e9, "hbm_frac": bf_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        del bcall, xb, zb, db, su, dout
        log("backward %.3f ms (cols, saved u), with the LayerNorm %.3f ms"
            % (extras["backward_2048"]["cols"]["saved_u"]["ms"], res["saved_u"]["ms"]))
        # torch's device copy, for comparison with the calibration copy
        dst = torch.empty_like(x)
        tc_ms, _ = time_steps(lambda: dst.copy_(x), 3, stream)
        extras["torch_copy_GBps"] = 2 * 4 * elems / (tc_ms * 1e-3) / 1e9
        del dst, scall, rcall
        # unpooled layer on the same inputs: a scan over all h*w tokens
        ucall = P.SSMCall(x, z, prm, P.POOL_NONE_ROWMAJOR, out=call.out)
        ucall.run(stream)
        u_ms, _ = time_steps(lambda: ucall.run(stream), 3, stream)
        u_scan, _ = time_steps(lambda: ucall.stage(P.STAGE_SCAN, stream), 3, stream)
        u_proj, _ = time_steps(lambda: ucall.stage(P.STAGE_PROJ, stream), 3, stream)
        extras["unpooled_2048"] = {"T": cfg.h * cfg.w, "layer_ms": u_ms, "scan_ms": u_scan, "proj_ms": u_proj,
                                   "layer_speedup_pooled": u_ms / ms, "scan_speedup_pooled": u_scan / stages["scan"]}
        del ucall
        # LBMamba's local backward scan in place of the global one: unpooled (T = h w) and pooled
        lb = {}
        for name, axis, reps in (("unpooled", P.POOL_NONE_ROWMAJOR, 3), ("pooled", P.POOL_COLS, n)):
            lcall = P.SSMCall(x, z, prm, axis, out=call.out, flags=P.FLAG_LOCAL_BWD)
            lcall.run(stream)
            l_ms, _ = time_steps(lambda: lcall.run(stream), reps, stream)
            l_scan, _ = time_steps(lambda: lcall.stage(P.STAGE_SCAN, stream), reps, stream)
            l_proj, _ = time_steps(lambda: lcall.stage(P.STAGE_PROJ, stream), reps, stream)
            lb[name] = {"layer_ms": l_ms, "scan_ms": l_scan, "proj_ms": l_proj}
            del lcall
        # the pooled layer's default is the single launch; its stage kernels for comparison
        lcall = P.SSMCall(x, z, prm, P.POOL_COLS, out=call.out, flags=P.FLAG_LOCAL_BWD | P.FLAG_STAGED)
        lcall.run(stream)
        lb["pooled"]["stage_kernels_ms"], _ = time_steps(lambda: lcall.run(stream), n, stream)
        lb["pooled"]["path"] = "single launch"
        lb["pooled"]["layer_vs_bidirectional"] = lb["pooled"]["layer_ms"] / ms
        del lcall
        lb["unpooled"]["scan_vs_bidirectional"] = lb["unpooled"]["scan_ms"] / u_scan
        lb["unpooled"]["layer_vs_bidirectional"] = lb["unpooled"]["layer_ms"] / u_ms
        lb["window"] = P.LOCAL_WINDOW
        extras["local_bwd_2048"] = lb
        torch.cuda.empty_cache()
        torch.cuda.empty_cache()
        log("unpooled layer %.3f ms, scan %.3f ms" % (u_ms, u_scan))
        # 1024^2 two-block chain on a quarter of the same buffers (same E and R)
        c2 = C.CHAIN_1024
        n2 = c2.B * c2.h * c2.w * c2.E
        x2 = x.view(-1)[:n2].view(c2.B, c2.h, c2.w, c2.E)
        z2 = z.view(-1)[:n2].view(c2.B, c2.h, c2.w, c2.E)
        z2b = z.view(-1)[n2:2 * n2].view(c2.B, c2.h, c2.w, c2.E)
        b1 = P.SSMCall(x2, z2, prm, P.POOL_COLS)
        b2 = P.SSMCall(b1.out, z2b, prm, P.POOL_ROWS, workspace=b1.workspace)

        def chain():
            b1.run(stream)
            b2.run(stream)
        chain()
        ch_ms, _ = time_steps(chain, n, stream)
        # the same chain with each block's scan and output stages in one launch
        one = P.tuning_scan_out(P.SCAN_OUT_ONE)
        b1o = P.SSMCall(x2, z2, prm, P.POOL_COLS, workspace=b1.workspace, out=b1.out, tuning=one)
        b2o = P.SSMCall(b1.out, z2b, prm, P.POOL_ROWS, workspace=b1.workspace, out=b2.out, tuning=one)

        def chain_one():
            b1o.run(stream)
            b2o.run(stream)
        chain_one()
        ch_one_ms, _ = time_steps(chain_one, n, stream)
        s1 = P.SSMCall(x2, z2, prm, P.POOL_COLS, workspace=b1.workspace, out=b2.out, flags=P.FLAG_STAGED)
        s1.run(stream)
        p_scan, _ = time_steps(lambda: s1.stage(P.STAGE_SCAN, stream), n, stream)
        u2 = P.SSMCall(x2, z2, prm, P.POOL_NONE_ROWMAJOR, out=b2.out)
        u2.run(stream)
        u2_ms, _ = time_steps(lambda: u2.run(stream), 3, stream)
        u2_scan, _ = time_steps(lambda: u2.stage(P.STAGE_SCAN, stream), 3, stream)
        extras["chain_1024"] = {"workload": c2.name, "two_block_ms": ch_ms, "images_per_s": c2.B / (ch_ms * 1e-3),
                                "hbm_frac": 2 * 12 * n2 / (ch_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                                "two_block_ms_scan_and_output_one_launch": ch_one_ms,
                                "pooled_scan_ms": p_scan, "unpooled_layer_ms": u2_ms, "unpooled_scan_ms": u2_scan,
                                "scan_speedup_pooled": u2_scan / p_scan,
                                "layer_speedup_pooled": u2_ms / (ch_ms / 2)}
        del b1, b2, b1o, b2o, s1, u2
        torch.cuda.empty_cache()
        extras["other_configs"] = small_configs(P, C, torch, stream)
        result["extras"] = extras

    if not args.no_cpu_baseline:
        log("timing the CPU oracle (>= %.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(wl["x"], wl["z"][0], wl["params"][0], 0, args.cpu_seconds)
        if not args.no_extras:
            log("timing the CPU oracle on the other workloads")
            result["extras"]["oracle_timings"] = oracle_timings(C, wl)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
