"""GPU parity of the pool scale (the factor on the pooled tokens of the MAE
transfer recipe, 0.25 there; FASTVIM_FLAG_POOL_SCALE) against the fp64
oracle: forward on every path and option of a pooled layer (out, its D = 0
twin, the pooled tokens and both scan outputs), the backward pass (dense,
masked, with the LayerNorm, with saved pooled tokens), and the 2048^2 layer at
full size on a sample of images.  Bar: 1e-4 fp32, 2e-2 bf16.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, check, dev, dev_params, gpu_call, host, status_ok
from pins import rand_conv, rand_dir, rand_ln
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import DIRECTIONS, draw_workload, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu

SCALE = 0.25
FIELDS = ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _inputs(rng, shape, io):
    x, z = (rng.standard_normal(shape).astype(np.float32) for _ in range(2))
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    return x, z


OPTIONS = ["plain", "norm", "conv", "local"]
PATHS = {"default": 0, "staged": P.FLAG_STAGED, "fused": P.FLAG_FUSED}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("option", OPTIONS)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_pool_scale_forward_dense(io, axis, option, path):
    B, h, w, E, R = 2, 24, 20, 136, 12
    rng = np.random.default_rng(zlib.crc32(repr(("pool-scale", io, axis, option, path)).encode()))
    x, z = _inputs(rng, (B, h, w, E), io)
    prm = {d: rand_dir(rng, E, 16, R, 0.1) for d in DIRECTIONS}
    ln = rand_ln(rng, E) if option == "norm" else None
    conv = rand_conv(rng, E) if option == "conv" else None
    window = P.LOCAL_WINDOW if option == "local" else 0
    flags = PATHS[path] | (P.FLAG_LOCAL_BWD if option == "local" else 0)
    tol = FP32_TOL if io == "f32" else BF16_TOL
    dt = torch.float32 if io == "f32" else torch.bfloat16
    tag = "scale %s axis %d %s %s" % (io, axis, option, path)
    print("\n[%s]" % tag, flush=True)
    call = gpu_call(x, z, prm, axis, dtype=dt, flags=flags, ln=ln, conv=conv, pool_scale=SCALE)
    out = host(call.run())
    torch.cuda.synchronize()
    status_ok(call)
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, stages=True, ln=ln, conv=conv, local_window=window,
                       pool_scale=SCALE)
    check(out, ref["out"], tol, tag + " out")
    check(host(call.export(P.EXPORT_U)), ref["u"], tol, tag + " u")
    check(host(call.export(P.EXPORT_S_FWD)), ref["fwd"]["s"], tol, tag + " s_fwd")
    check(host(call.export(P.EXPORT_S_BWD)), ref["bwd"]["s"], tol, tag + " s_bwd")
    p0 = zero_D(prm)
    twin = host(gpu_call(x, z, p0, axis, dtype=dt, flags=flags, ln=ln, conv=conv, pool_scale=SCALE).run())
    torch.cuda.synchronize()
    ref0 = oracle.layer(x, z, p0["fwd"], p0["bwd"], axis, ln=ln, conv=conv, local_window=window, pool_scale=SCALE)
    check(twin, ref0, tol, tag + " out(D=0)")


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_pool_scale_forward_masked(io, axis, norm):
    B, h, w, E, R, K = 3, 14, 14, 96, 8, 49
    rng = np.random.default_rng(zlib.crc32(repr(("pool-scale-masked", io, axis, norm)).encode()))
    x, z = _inputs(rng, (B, K, E), io)
    idx = random_mask(rng, B, h, w, K)
    prm = {d: rand_dir(rng, E, 16, R, 0.1) for d in DIRECTIONS}
    ln = rand_ln(rng, E) if norm else None
    tol = FP32_TOL if io == "f32" else BF16_TOL
    dt = torch.float32 if io == "f32" else torch.bfloat16
    tag = "scale masked %s axis %d norm %s" % (io, axis, norm)
    call = gpu_call(x, z, prm, axis, idx=idx, hw=(h, w), dtype=dt, ln=ln, pool_scale=SCALE)
    out = host(call.run())
    torch.cuda.synchronize()
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, idx=idx, hw=(h, w), stages=True, ln=ln, pool_scale=SCALE)
    check(out, ref["out"], tol, tag + " out")
    check(host(call.export(P.EXPORT_U)), ref["u"], tol, tag + " u")
    check(host(call.export(P.EXPORT_S_FWD)), ref["fwd"]["s"], tol, tag + " s_fwd")


def _bwd(x, z, dout, prm, axis, dt, idx=None, hw=None, ln=None, saved=False):
    idd = None if idx is None else dev(idx, torch.int32)
    xd, zd, pd = dev(x, dt), dev(z, dt), dev_params(prm)
    lnd = None if ln is None else {"weight": dev(ln["weight"]), "bias": dev(ln["bias"]), "eps": ln["eps"]}
    su = None
    if saved:
        h, w = (x.shape[1], x.shape[2]) if idx is None else hw
        su = torch.full((x.shape[0], h if axis == P.POOL_COLS else w, x.shape[-1]), float("nan"), device="cuda")
        P.SSMCall(xd, zd, pd, axis, mask_idx=idd, hw=hw, saved_u=su, ln=lnd, pool_scale=SCALE).run()
    res = P.BwdCall(xd, zd, dev(dout, dt), pd, axis, mask_idx=idd, hw=hw, saved_u=su, ln=lnd,
                    pool_scale=SCALE).run()
    torch.cuda.synchronize()
    return res


def _compare_bwd(res, ref, tol, tag, sel=None):
    s = slice(None) if sel is None else sel
    check(host(res["dx"])[s], ref["dx"], tol, tag + " dx")
    check(host(res["dz"])[s], ref["dz"], tol, tag + " dz")
    for d in DIRECTIONS:
        for f in FIELDS:
            check(host(res[d][f]), ref[d][f], tol, "%s d%s.%s" % (tag, d, f))
    if "ln" in ref:
        for f in ("weight", "bias"):
            check(host(res["ln"][f]), ref["ln"][f], tol, "%s d ln_%s" % (tag, f))


BWD_CASES = [("dense", False, False), ("dense", True, False), ("dense", False, True), ("masked", False, False),
             ("masked", True, True)]


@pytest.mark.parametrize("kind,norm,saved", BWD_CASES, ids=["%s-%s-%s" % (k, "norm" if n else "plain",
                                                                        "saved" if s else "pools")
                                                            for k, n, s in BWD_CASES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_pool_scale_backward(io, axis, kind, norm, saved):
    rng = np.random.default_rng(zlib.crc32(repr(("pool-scale-bwd", io, axis, kind, norm, saved)).encode()))
    if kind == "masked":
        B, h, w, E, R, K = 3, 7, 9, 64, 6, 30
        shape, idx, hw = (B, K, E), random_mask(rng, B, h, w, K), (h, w)
    else:
        B, h, w, E, R = 2, 21, 10, 136, 9
        shape, idx, hw = (B, h, w, E), None, None
    x, z = _inputs(rng, shape, io)
    dout = rng.standard_normal(shape).astype(np.float32)
    if io == "bf16":
        dout = round_to_bf16(dout)
    prm = {d: rand_dir(rng, E, 16, R, 0.1) for d in DIRECTIONS}
    ln = rand_ln(rng, E) if norm else None
    tol = FP32_TOL if io == "f32" else BF16_TOL
    dt = torch.float32 if io == "f32" else torch.bfloat16
    tag = "scale bwd %s axis %d %s norm %s saved %s" % (io, axis, kind, norm, saved)
    print("\n[%s]" % tag, flush=True)
    res = _bwd(x, z, dout, prm, axis, dt, idx=idx, hw=hw, ln=ln, saved=saved)
    ref = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], axis, idx=idx, hw=hw, ln=ln, pool_scale=SCALE)
    _compare_bwd(res, ref, tol, tag)


def test_pool_scale_full_size_2048():
    """The 2048^2 layer at full size (single launch) with the pool scale, and
    its backward pass with the upstream gradient on two images: the oracle
    on those images gives out there and every gradient."""
    cfg = C.HIRES_2048
    wl = draw_workload(cfg)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    sel = np.array([0, cfg.B - 1])
    print("\n[2048 pool scale] B=%d, outputs compared on images %s" % (cfg.B, list(sel)), flush=True)
    call = gpu_call(x, z, prm, P.POOL_COLS, pool_scale=SCALE)
    out = call.run()
    torch.cuda.synchronize()
    status_ok(call)
    got = host(out[torch.as_tensor(sel, device="cuda")])
    del out, call
    ref = oracle.layer(x[sel], z[sel], prm["fwd"], prm["bwd"], P.POOL_COLS, pool_scale=SCALE)
    check(got, ref, FP32_TOL, "2048 pool scale out")
    rng = np.random.default_rng(79)
    dout = np.zeros_like(x)
    dout[sel] = rng.standard_normal(dout[sel].shape).astype(np.float32)
    res = _bwd(x, z, dout, prm, P.POOL_COLS, torch.float32, saved=True)
    rest = torch.as_tensor(np.setdiff1d(np.arange(cfg.B), sel), device="cuda")
    for name in ("dx", "dz"):
        assert torch.count_nonzero(res[name][rest]).item() == 0, name + " nonzero without upstream gradient"
    ref = oracle.layer_bwd(x[sel], z[sel], dout[sel], prm["fwd"], prm["bwd"], P.POOL_COLS, pool_scale=SCALE)
    _compare_bwd(res, ref, FP32_TOL, "2048 pool scale bwd", sel=sel)
