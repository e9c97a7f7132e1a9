"""The autograd front end (pooled_selective_state_amd.pooled_ssm): gradients
that PyTorch's backward collects through the layer's forward and backward
calls against the fp64 oracle's chain rule, on single layers with each option
and on the two-block chain (COLS then ROWS) that alternates the pooling axis.
Bar: 1e-4 fp32, 2e-2 bf16 (oracle on the bf16-rounded inputs).
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, check, compare_stages, dev, gpu_call, host, stage_exports
from pins import rand_conv, rand_dir, rand_ln
from pooled_selective_state_amd.inputs import DIRECTIONS, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu
FIELDS = ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def leaf(a, dtype=torch.float32):
    return dev(a, dtype).requires_grad_(True)


def _case(rng, shape, E, R, io):
    x, z, dout = (rng.standard_normal(shape).astype(np.float32) for _ in range(3))
    if io == "bf16":
        x, z, dout = round_to_bf16(x), round_to_bf16(z), round_to_bf16(dout)
    prm = {d: rand_dir(rng, E, 16, R, 0.1) for d in DIRECTIONS}
    return x, z, dout, prm


CASES = ["plain", "norm_scale", "local", "conv", "masked", "bf16_norm_local"]


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("case", CASES)
def test_autograd_single_layer(case, axis):
    rng = np.random.default_rng(zlib.crc32(repr(("autograd", case, axis)).encode()))
    io = "bf16" if case.startswith("bf16") else "f32"
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    tol = BF16_TOL if io == "bf16" else FP32_TOL
    B_, h, w, E, R = 2, 12, 10, 72, 6
    masked = case == "masked"
    K = 50
    x, z, dout, prm = _case(rng, (B_, K, E) if masked else (B_, h, w, E), E, R, io)
    idx = random_mask(rng, B_, h, w, K) if masked else None
    ln = rand_ln(rng, E) if "norm" in case else None
    conv = rand_conv(rng, E) if case == "conv" else None
    scale = 0.25 if "scale" in case else None
    flags = P.FLAG_LOCAL_BWD if "local" in case else 0
    xd, zd = leaf(x, dt), leaf(z, dt)
    pd = {d: {f: leaf(prm[d][f]) for f in FIELDS} for d in DIRECTIONS}
    lnd = None if ln is None else {"weight": leaf(ln["weight"]), "bias": leaf(ln["bias"]), "eps": ln["eps"]}
    cvd = None if conv is None else {"weight": leaf(conv["weight"]), "bias": leaf(conv["bias"])}
    out = P.pooled_ssm(xd, zd, pd, axis, mask_idx=None if idx is None else dev(idx, torch.int32),
                       hw=(h, w) if masked else None, flags=flags, ln=lnd, conv=cvd, pool_scale=scale)
    (out.float() * dev(dout)).sum().backward()
    torch.cuda.synchronize()
    tag = "autograd %s axis %d" % (case, axis)
    ref_out = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, idx=idx, hw=(h, w) if masked else None, ln=ln,
                           conv=conv, local_window=P.LOCAL_WINDOW if flags else 0,
                           pool_scale=1.0 if scale is None else scale)
    check(host(out), ref_out, tol, tag + " out")
    ref = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], axis, idx=idx, hw=(h, w) if masked else None,
                           ln=ln, conv=conv, local_window=P.LOCAL_WINDOW if flags else 0,
                           pool_scale=1.0 if scale is None else scale)
    check(host(xd.grad), ref["dx"], tol, tag + " dx")
    check(host(zd.grad), ref["dz"], tol, tag + " dz")
    for d in DIRECTIONS:
        for f in FIELDS:
            check(host(pd[d][f].grad), ref[d][f], tol, "%s d%s.%s" % (tag, d, f))
    for opt, src in (("ln", lnd), ("conv", cvd)):
        if src is not None:
            for f in ("weight", "bias"):
                check(host(src[f].grad), ref[opt][f], tol, "%s d %s_%s" % (tag, opt, f))


def test_autograd_two_block_chain():
    """Block 1 pools over columns, block 2 over rows on block 1's output (the
    alternation of the layer); PyTorch's backward through both equals the
    oracle's chain rule applied block by block."""
    rng = np.random.default_rng(12)
    B_, h, w, E, R = 2, 16, 14, 64, 6
    x, z1, _, p1 = _case(rng, (B_, h, w, E), E, R, "f32")
    z2 = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    dout = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    p2 = {d: rand_dir(rng, E, 16, R, 0.1) for d in DIRECTIONS}
    xd, z1d, z2d = leaf(x), leaf(z1), leaf(z2)
    pd1 = {d: {f: leaf(p1[d][f]) for f in FIELDS} for d in DIRECTIONS}
    pd2 = {d: {f: leaf(p2[d][f]) for f in FIELDS} for d in DIRECTIONS}
    out1 = P.pooled_ssm(xd, z1d, pd1, P.POOL_COLS)
    out2 = P.pooled_ssm(out1, z2d, pd2, P.POOL_ROWS)
    (out2 * dev(dout)).sum().backward()
    torch.cuda.synchronize()
    o1 = oracle.layer(x, z1, p1["fwd"], p1["bwd"], P.POOL_COLS).astype(np.float32)
    # block 2's oracle input is the GPU block 1's output rounded to fp32 as the GPU passes it on
    o1_gpu = host(out1).astype(np.float32)
    check(o1_gpu, o1, FP32_TOL, "chain block 1 out")
    # each block's forward on its own input, where out alone could hide the
    # scan under the skip term: the same call through the C ABI gives the
    # autograd forward's out bit for bit, its stage exports (pooled tokens,
    # both x_proj directions, s_fwd, s_bwd) and its D = 0 twin match the oracle
    for tag, xin, zin, prm, axis, got in (("chain block 1", x, z1, p1, P.POOL_COLS, out1),
                                          ("chain block 2", o1_gpu, z2, p2, P.POOL_ROWS, out2)):
        call = gpu_call(xin, zin, prm, axis)
        same = call.run()
        torch.cuda.synchronize()
        assert torch.equal(same, got.detach()), tag + ": C ABI call differs from the autograd forward"
        ref = oracle.layer(xin, zin, prm["fwd"], prm["bwd"], axis, stages=True)
        compare_stages(stage_exports(call), ref, FP32_TOL, tag)
        twin = gpu_call(xin, zin, zero_D(prm), axis).run()
        torch.cuda.synchronize()
        check(host(twin), oracle.layer(xin, zin, zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis), FP32_TOL,
              tag + " out(D=0)")
    r2 = oracle.layer_bwd(o1_gpu, z2, dout, p2["fwd"], p2["bwd"], P.POOL_ROWS)
    r1 = oracle.layer_bwd(x, z1, r2["dx"].astype(np.float32), p1["fwd"], p1["bwd"], P.POOL_COLS)
    check(host(z2d.grad), r2["dz"], FP32_TOL, "chain dz2")
    check(host(xd.grad), r1["dx"], FP32_TOL, "chain dx")
    check(host(z1d.grad), r1["dz"], FP32_TOL, "chain dz1")
    for d in DIRECTIONS:
        for f in FIELDS:
            check(host(pd2[d][f].grad), r2[d][f], FP32_TOL, "chain block 2 d%s.%s" % (d, f))
            check(host(pd1[d][f].grad), r1[d][f], FP32_TOL, "chain block 1 d%s.%s" % (d, f))
