"""Seeded random layers against the fp64 oracle: every layer kind (dense COLS
or ROWS, masked, unpooled in either raster order) crossed with ragged sizes,
both element types, both paths of a dense pooled layer and the options that
combine with it (post-SSM LayerNorm, producer Conv1D, LBMamba's local
backward scan), so that combinations the fixed cases do not list are checked
too.  Each case compares out, the out of its D = 0 twin, and both scan
outputs, each on its own scale; cases of pooled layers also run the backward
pass (with the options the case has), with and without the pooled tokens
saved by the forward call.
Bar: 1e-4 fp32, 2e-2 bf16 (oracle on the bf16-rounded inputs).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, check, dev, dev_params, gpu_call, host, status_ok
from pins import rand_conv, rand_dir, rand_ln
from pooled_selective_state_amd.inputs import DIRECTIONS, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu

KINDS = ("cols", "rows", "masked_cols", "masked_rows", "unpooled_row", "unpooled_col")
AXIS = {"cols": P.POOL_COLS, "rows": P.POOL_ROWS, "masked_cols": P.POOL_COLS, "masked_rows": P.POOL_ROWS,
        "unpooled_row": P.POOL_NONE_ROWMAJOR, "unpooled_col": P.POOL_NONE_COLMAJOR}
FIELDS = ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")
# 400 seeds by default; FASTVIM_RANDOM_SEEDS="a:b" runs seeds a .. b-1 instead
# (for one-off wider sweeps)
_seed_env = os.environ.get("FASTVIM_RANDOM_SEEDS", "")
SEEDS = range(*map(int, _seed_env.split(":"))) if _seed_env else range(400)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def draw_case(seed):
    """A random layer: sizes, element type, path and options."""
    rng = np.random.default_rng(1000 + seed)
    kind = KINDS[seed % len(KINDS)]
    io = "bf16" if rng.random() < 0.4 else "f32"
    B = int(rng.integers(1, 4))
    big = rng.random() < 0.25  # a quarter of the cases on larger grids and wider channels
    h, w = int(rng.integers(1, 49 if big else 25)), int(rng.integers(1, 49 if big else 25))
    E = 8 * int(rng.integers(1, 130 if big else 66))
    R = int(rng.integers(1, 65))
    masked = kind.startswith("masked")
    K = int(rng.integers(1, h * w + 1)) if masked else 0
    dense_pooled = kind in ("cols", "rows")
    norm = bool(rng.random() < 0.3)
    conv = dense_pooled and not norm and bool(rng.random() < 0.35)
    local = bool(rng.random() < 0.3)
    path = ["default", "staged", "fused"][int(rng.integers(0, 3))]
    return dict(rng=rng, kind=kind, io=io, B=B, h=h, w=w, E=E, R=R, K=K, norm=norm, conv=conv, local=local,
                path=path)


def _tag(c):
    opts = [o for o in ("norm", "conv", "local") if c[o]]
    return "%s %s B=%d %dx%d E=%d R=%d K=%d %s [%s]" % (c["kind"], c["io"], c["B"], c["h"], c["w"], c["E"], c["R"],
                                                       c["K"], c["path"], ",".join(opts))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layer(seed):
    c = draw_case(seed)
    rng, tag = c["rng"], _tag(c)
    print("\n[random %d] %s" % (seed, tag), flush=True)
    axis = AXIS[c["kind"]]
    masked = c["K"] > 0
    shape = (c["B"], c["K"], c["E"]) if masked else (c["B"], c["h"], c["w"], c["E"])
    x = rng.standard_normal(shape).astype(np.float32)
    z = rng.standard_normal(shape).astype(np.float32)
    if c["io"] == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {d: rand_dir(rng, c["E"], 16, c["R"], 0.1) for d in DIRECTIONS}
    idx = random_mask(rng, c["B"], c["h"], c["w"], c["K"]) if masked else None
    hw = (c["h"], c["w"]) if masked else None
    ln = rand_ln(rng, c["E"]) if c["norm"] else None
    conv = rand_conv(rng, c["E"]) if c["conv"] else None
    window = P.LOCAL_WINDOW if c["local"] else 0
    flags = {"default": 0, "staged": P.FLAG_STAGED, "fused": P.FLAG_FUSED}[c["path"]]
    if c["local"]:
        flags |= P.FLAG_LOCAL_BWD
    tol = FP32_TOL if c["io"] == "f32" else BF16_TOL
    dt = torch.float32 if c["io"] == "f32" else torch.bfloat16

    call = gpu_call(x, z, prm, axis, idx=idx, hw=hw, dtype=dt, flags=flags, ln=ln, conv=conv)
    out = host(call.run())
    torch.cuda.synchronize()
    status_ok(call)
    sf, sb = host(call.export(P.EXPORT_S_FWD)), host(call.export(P.EXPORT_S_BWD))
    twin = host(gpu_call(x, z, zero_D(prm), axis, idx=idx, hw=hw, dtype=dt, flags=flags, ln=ln, conv=conv).run())
    torch.cuda.synchronize()
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, idx=idx, hw=hw, stages=True, ln=ln, conv=conv,
                       local_window=window)
    ref0 = oracle.layer(x, z, zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis, idx=idx, hw=hw, ln=ln, conv=conv,
                        local_window=window)
    check(out, ref["out"], tol, tag + " out")
    check(twin, ref0, tol, tag + " out(D=0)")
    check(sf, ref["fwd"]["s"], tol, tag + " s_fwd")
    check(sb, ref["bwd"]["s"], tol, tag + " s_bwd")

    # the backward pass covers pooled layers with every option
    if axis in (P.POOL_COLS, P.POOL_ROWS) and \
            (c["w"] if axis == P.POOL_ROWS else c["h"]) <= 128:
        dout = rng.standard_normal(shape).astype(np.float32)
        if c["io"] == "bf16":
            dout = round_to_bf16(dout)
        xd, zd, pd = dev(x, dt), dev(z, dt), dev_params(prm)
        idd = None if idx is None else dev(idx, torch.int32)
        lnd = None if ln is None else {"weight": dev(ln["weight"], torch.float32),
                                       "bias": dev(ln["bias"], torch.float32), "eps": ln["eps"]}
        cvd = None if conv is None else {"weight": dev(conv["weight"]), "bias": dev(conv["bias"])}
        su = None
        if seed % 2:
            T = c["h"] if axis == P.POOL_COLS else c["w"]
            su = torch.full((c["B"], T, c["E"]), float("nan"), device="cuda")
            P.SSMCall(xd, zd, pd, axis, mask_idx=idd, hw=hw, saved_u=su, ln=lnd, conv=cvd).run()
        bflags = P.FLAG_LOCAL_BWD if c["local"] else 0
        res = P.BwdCall(xd, zd, dev(dout, dt), pd, axis, mask_idx=idd, hw=hw, saved_u=su, ln=lnd, flags=bflags,
                        conv=cvd).run()
        torch.cuda.synchronize()
        rb = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], axis, idx=idx, hw=hw, ln=ln, local_window=window,
                              conv=conv)
        btag = tag + (" bwd saved-u" if su is not None else " bwd")
        check(host(res["dx"]), rb["dx"], tol, btag + " dx")
        check(host(res["dz"]), rb["dz"], tol, btag + " dz")
        for d in DIRECTIONS:
            for f in FIELDS:
                check(host(res[d][f]), rb[d][f], tol, "%s d%s.%s" % (btag, d, f))
        for opt in ("ln", "conv"):
            if opt in rb:
                for f in ("weight", "bias"):
                    check(host(res[opt][f]), rb[opt][f], tol, "%s d %s_%s" % (btag, opt, f))
