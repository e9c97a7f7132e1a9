"""GPU parity of the backward pass: fastvim_ssm_bwd (through the C ABI)
against the fp64 oracle's chain rule, which is pinned to central differences
of the forward oracle.

Every tensor is compared on its own scale, max|gpu - oracle| / max|oracle|:
dx, dz, and the five parameter gradients of each direction.  A D = 0 twin
repeats dx and dz with the skip removed, so the skip's share of them (which
dominates at the workloads' parameter scales) cannot hide the scan adjoint.
Bar: 1e-4 for fp32 I/O, 2e-2 for bf16 I/O (oracle on the bf16-rounded
inputs and upstream gradient).  Full-size workloads run on the GPU at their
real shape with the upstream gradient nonzero on a sample of images only:
every gradient then comes from those images alone, so the oracle on the
sample gives every parameter gradient, and the other images' dx and dz must
be exactly zero.  Cases marked "saved" run the GPU forward first, with
saved_u, and give the backward those pooled tokens instead of letting it
pool x again.  The later sections cover the options: the post-SSM LayerNorm
(every team shape of its first pass, masked layers and invalid indices),
LBMamba's local backward scan (T from one partial window to eight whole
ones), and the producer Conv1D (grids whose windows cross rows and columns),
each also at full size.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, check, dev, dev_params, host
from pins import rand_conv, rand_dir, rand_ln
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import DIRECTIONS, draw_workload, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu

FIELDS = ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _dev_ln(ln):
    if ln is None:
        return None
    return {"weight": dev(ln["weight"], torch.float32), "bias": dev(ln["bias"], torch.float32), "eps": ln["eps"]}


def gpu_bwd(x, z, dout, prm, axis, idx=None, hw=None, dtype=torch.float32, flags=0, saved=None, ln=None,
            pool_scale=None, conv=None, groups=0):
    """saved: None (the backward pools x itself) or the flags of a forward call
    that first writes the pooled tokens the backward then reads (saved_u).
    ln: the post-SSM LayerNorm (host arrays), for both calls.  groups: the
    backward call's image groups (0: the library's choice)."""
    idd = None if idx is None else dev(idx, torch.int32)
    xd, zd, pd = dev(x, dtype), dev(z, dtype), dev_params(prm)
    lnd = _dev_ln(ln)
    cvd = None if conv is None else {"weight": dev(conv["weight"]), "bias": dev(conv["bias"])}
    su = None
    if saved is not None:
        h, w = (x.shape[1], x.shape[2]) if idx is None else hw
        su = torch.full((x.shape[0], h if axis == P.POOL_COLS else w, x.shape[-1]), float("nan"), device="cuda")
        P.SSMCall(xd, zd, pd, axis, mask_idx=idd, hw=hw, flags=saved | (flags & P.FLAG_LOCAL_BWD), saved_u=su,
                  ln=lnd, pool_scale=pool_scale, conv=cvd).run()
    call = P.BwdCall(xd, zd, dev(dout, dtype), pd, axis, mask_idx=idd, hw=hw, flags=flags, saved_u=su, ln=lnd,
                     pool_scale=pool_scale, conv=cvd, groups=groups)
    res = call.run()
    torch.cuda.synchronize()
    out = {"dx": host(res["dx"]), "dz": host(res["dz"]),
           **{d: {f: host(res[d][f]) for f in FIELDS} for d in DIRECTIONS}}
    if ln is not None:
        out["ln"] = {f: host(res["ln"][f]) for f in ("weight", "bias")}
    if conv is not None:
        out["conv"] = {f: host(res["conv"][f]) for f in ("weight", "bias")}
    return out


def compare(got, ref, tol, tag, sel=None, params=True):
    s = slice(None) if sel is None else sel
    check(got["dx"][s], ref["dx"], tol, tag + " dx")
    check(got["dz"][s], ref["dz"], tol, tag + " dz")
    if params:
        for d in DIRECTIONS:
            for f in FIELDS:
                check(got[d][f], ref[d][f], tol, "%s d%s.%s" % (tag, d, f))
        for opt in ("ln", "conv"):
            if opt in ref:
                for f in ("weight", "bias"):
                    check(got[opt][f], ref[opt][f], tol, "%s d %s_%s" % (tag, opt, f))


def bwd_check(x, z, dout, prm, axis, tol, dtype, tag, idx=None, hw=None, twin=True, saved=None, ln=None,
              conv=None, flags=0, pool_scale=None):
    """GPU gradients and those of the D = 0 twin against the oracle."""
    local = P.LOCAL_WINDOW if flags & P.FLAG_LOCAL_BWD else 0
    ps = 1.0 if pool_scale is None else pool_scale
    kw = dict(idx=idx, hw=hw, dtype=dtype, saved=saved, ln=ln, conv=conv, flags=flags, pool_scale=pool_scale)
    got = gpu_bwd(x, z, dout, prm, axis, **kw)
    ref = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], axis, idx=idx, hw=hw, ln=ln, conv=conv,
                           local_window=local, pool_scale=ps)
    compare(got, ref, tol, tag)
    if twin:
        p0 = zero_D(prm)
        got0 = gpu_bwd(x, z, dout, p0, axis, **kw)
        ref0 = oracle.layer_bwd(x, z, dout, p0["fwd"], p0["bwd"], axis, idx=idx, hw=hw, ln=ln, conv=conv,
                                local_window=local, pool_scale=ps)
        compare(got0, ref0, tol, tag + " (D=0)", params=False)
    return got


def _io(io, *arrays):
    if io == "bf16":
        return [round_to_bf16(a) for a in arrays]
    return list(arrays)


def _tol(io):
    return (FP32_TOL, torch.float32) if io == "f32" else (BF16_TOL, torch.bfloat16)


# ------------------------------------------------------------------ small / ragged
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_tiny_fastvim_t(axis, io):
    wl = draw_workload(C.TINY)
    rng = np.random.default_rng(11 + axis)
    dout = rng.standard_normal(wl["x"].shape).astype(np.float32)
    x, z, dout = _io(io, wl["x"], wl["z"][0], dout)
    tol, dt = _tol(io)
    bwd_check(x, z, dout, wl["params"][0], axis, tol, dt, "tiny %s axis %d" % (io, axis))


RAGGED = [
    # B, h, w, E, R   (E not a multiple of 64, scan lengths not multiples of 16, every dt-rank bound)
    (3, 13, 7, 72, 5),
    (1, 1, 1, 8, 1),
    (2, 5, 9, 200, 20),
    (2, 3, 33, 136, 64),
    (1, 37, 2, 1032, 33),
    (2, 128, 3, 40, 12),
    (2, 17, 100, 64, 40),
]


# forward path whose pooled tokens the backward reads: None (it pools x
# itself), or the single launch where the layer allows it (else the stage kernels)
SAVED = [None, P.FLAG_FUSED]
SAVED_IDS = ["pools", "saved"]


@pytest.mark.parametrize("saved", SAVED, ids=SAVED_IDS)
@pytest.mark.parametrize("shape", RAGGED, ids=["x".join(map(str, s)) for s in RAGGED])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_ragged_shapes(shape, axis, io, saved):
    B, h, w, E, R = shape
    if (h if axis == P.POOL_COLS else w) > 128:
        pytest.skip("scan longer than the backward pass supports")
    rng = np.random.default_rng(zlib.crc32(repr(("bwd", shape, axis, io)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    dout = rng.standard_normal((B, h, w, E)).astype(np.float32)
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "ragged %s %s axis %d" % (shape, io, axis), saved=saved)


@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 17, 42])
def test_bwd_masked_small(axis, io, K, saved):
    B, h, w, E, R = 5, 6, 7, 64, 6
    rng = np.random.default_rng(200 + K + 7 * axis)
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    dout = rng.standard_normal((B, K, E)).astype(np.float32)
    x, z, dout = _io(io, x, z, dout)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "masked K=%d %s axis %d" % (K, io, axis), idx=idx, hw=(h, w),
              saved=saved)


def test_bwd_masked_invalid_indices():
    """Tokens with an out-of-range or repeated index get NaN in dx and dz and
    take no part in any sum: the rest equals the oracle on the valid tokens."""
    B, h, w, E, R, K = 3, 5, 6, 48, 4, 9
    rng = np.random.default_rng(19)
    idx = random_mask(rng, B, h, w, K)
    idx[0, 2] = h * w
    idx[1, 4] = idx[1, 7]
    idx[2, 0] = -5
    x, z, dout = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    got = gpu_bwd(x, z, dout, prm, P.POOL_COLS, idx=idx, hw=(h, w))
    invalid = {(0, 2), (1, 4), (1, 7), (2, 0)}
    sums = {d: {f: 0.0 for f in FIELDS} for d in DIRECTIONS}
    for b in range(B):
        keep = [k for k in range(K) if (b, k) not in invalid]
        bad = [k for k in range(K) if (b, k) in invalid]
        for name in ("dx", "dz"):
            assert np.all(np.isnan(got[name][b, bad])), "invalid token of image %d not NaN in %s" % (b, name)
        ref = oracle.layer_bwd(x[b:b + 1, keep], z[b:b + 1, keep], dout[b:b + 1, keep], prm["fwd"], prm["bwd"],
                               P.POOL_COLS, idx=idx[b:b + 1, keep], hw=(h, w))
        check(got["dx"][b:b + 1, keep], ref["dx"], FP32_TOL, "invalid-index image %d dx" % b)
        check(got["dz"][b:b + 1, keep], ref["dz"], FP32_TOL, "invalid-index image %d dz" % b)
        for d in DIRECTIONS:
            for f in FIELDS:
                sums[d][f] = sums[d][f] + ref[d][f]
    for d in DIRECTIONS:
        for f in FIELDS:
            check(got[d][f], sums[d][f], FP32_TOL, "invalid-index d%s.%s" % (d, f))


def test_bwd_empty_batch_zero_gradients():
    E, R = 16, 3
    rng = np.random.default_rng(3)
    prm = dev_params({d: rand_dir(rng, E, 16, R) for d in DIRECTIONS})
    x = torch.empty((0, 3, 4, E), device="cuda")
    grads = {d: {f: torch.full_like(prm[d][f], 7.0) for f in FIELDS} for d in DIRECTIONS}
    call = P.BwdCall(x, x.clone(), x.clone(), prm, P.POOL_COLS, grads=grads)
    res = call.run()
    torch.cuda.synchronize()
    for d in DIRECTIONS:
        for f in FIELDS:
            assert torch.count_nonzero(res[d][f]).item() == 0


def test_bwd_deterministic():
    """Fixed-order sums: two calls give bitwise identical gradients."""
    B, h, w, E, R = 4, 24, 20, 136, 12
    rng = np.random.default_rng(5)
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    a = gpu_bwd(x, z, dout, prm, P.POOL_ROWS)
    b = gpu_bwd(x, z, dout, prm, P.POOL_ROWS)
    for k in ("dx", "dz"):
        assert np.array_equal(a[k], b[k])
    for d in DIRECTIONS:
        for f in FIELDS:
            assert np.array_equal(a[d][f], b[d][f])


def test_bwd_rows_is_cols_on_transposed_grid():
    """ROWS gradients are the COLS gradients of the transposed grid."""
    B, h, w, E, R = 2, 9, 14, 64, 8
    rng = np.random.default_rng(6)
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    r = gpu_bwd(x, z, dout, prm, P.POOL_ROWS)
    t = gpu_bwd(*(np.ascontiguousarray(a.transpose(0, 2, 1, 3)) for a in (x, z, dout)), prm, P.POOL_COLS)
    check(r["dx"], t["dx"].transpose(0, 2, 1, 3), FP32_TOL, "transpose dx")
    check(r["dz"], t["dz"].transpose(0, 2, 1, 3), FP32_TOL, "transpose dz")
    for d in DIRECTIONS:
        for f in FIELDS:
            check(r[d][f], t[d][f], FP32_TOL, "transpose d%s.%s" % (d, f))


# ------------------------------------------------------------------ full size
def _sampled_full_size(cfg, axis=P.POOL_COLS, saved=None, norm=False, local=False, with_conv=False):
    wl = draw_workload(cfg)
    x, z, prm, idx = wl["x"], wl["z"][0], wl["params"][0], wl["idx"]
    ln = rand_ln(np.random.default_rng(78), cfg.E) if norm else None
    conv = rand_conv(np.random.default_rng(79), cfg.E) if with_conv else None
    sel = np.array([0, cfg.B - 1])
    rng = np.random.default_rng(77)
    dout = np.zeros_like(x)
    dout[sel] = rng.standard_normal(dout[sel].shape).astype(np.float32)
    if cfg.io_dtype == "bf16":
        dout = round_to_bf16(dout)
    tol, dt = _tol(cfg.io_dtype)
    hw = (cfg.h, cfg.w) if cfg.masked else None
    print("\n[%s bwd] B=%d grid=%dx%d E=%d axis %d, upstream gradient on images %s, pooled tokens %s%s%s"
          % (cfg.name, cfg.B, cfg.h, cfg.w, cfg.E, axis, list(sel), "saved" if saved is not None else "recomputed",
             ", post-SSM LayerNorm" if norm else "", ", local backward scan" if local else "")
          + (", producer Conv1D" if with_conv else ""), flush=True)
    got = gpu_bwd(x, z, dout, prm, axis, idx=idx, hw=hw, dtype=dt, saved=saved, ln=ln, conv=conv,
                  flags=P.FLAG_LOCAL_BWD if local else 0)
    rest = np.setdiff1d(np.arange(cfg.B), sel)
    for name in ("dx", "dz"):
        assert np.count_nonzero(got[name][rest]) == 0, name + " nonzero on images without upstream gradient"
    ref = oracle.layer_bwd(x[sel], z[sel], dout[sel], prm["fwd"], prm["bwd"], axis,
                           idx=None if idx is None else idx[sel], hw=hw, ln=ln, conv=conv,
                           local_window=P.LOCAL_WINDOW if local else 0)
    compare(got, ref, tol, cfg.name, sel=sel)


@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_full_size_2048(axis, saved):
    _sampled_full_size(C.HIRES_2048, axis, saved)


@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("cfg", [C.SHORT_224_S, C.MASKED_B], ids=lambda c: c.name)
def test_bwd_full_size_other(cfg, saved):
    _sampled_full_size(cfg, saved=saved)


def test_bwd_saved_u_matches_pooling_again():
    """The two ways of getting the pooled tokens give the same gradients within
    fp32 rounding (only u's summation order differs)."""
    B, h, w, E, R = 3, 40, 36, 96, 10
    rng = np.random.default_rng(41)
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    for axis in (P.POOL_COLS, P.POOL_ROWS):
        a = gpu_bwd(x, z, dout, prm, axis)
        for fl in (P.FLAG_STAGED, P.FLAG_FUSED):
            b = gpu_bwd(x, z, dout, prm, axis, saved=fl)
            compare(b, a, 1e-5, "saved vs pooled again, axis %d flags %d" % (axis, fl))


# ------------------------------------------------------------------ post-SSM LayerNorm
# widths that reach every team shape of the norm's first pass: fp32 E = 8 ..
# 200 (16-lane teams, 1 to 4 vectors a lane), 384 and 504 (32 lanes), 768,
# 1024 and 1032 (64 lanes, up to 8 vectors); bf16 E = 8, 200 (16 lanes), 384
# (32), 1024, 1032 and 2048 (64)
NORM_SHAPES = {
    "f32": [(2, 5, 7, 8, 3), (3, 13, 7, 72, 5), (2, 9, 11, 136, 12), (1, 6, 33, 200, 20), (2, 16, 16, 384, 12),
            (1, 7, 5, 504, 33), (1, 9, 4, 768, 48), (1, 4, 9, 1024, 64), (1, 3, 5, 1032, 7)],
    "bf16": [(2, 5, 7, 8, 3), (1, 6, 33, 200, 20), (2, 16, 16, 384, 12), (1, 4, 9, 1024, 64), (1, 3, 5, 1032, 7),
             (1, 3, 4, 2048, 16)],
}
NORM_CASES = [(io, s) for io in ("f32", "bf16") for s in NORM_SHAPES[io]]


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io,shape", NORM_CASES, ids=["%s-%s" % (io, "x".join(map(str, s))) for io, s in NORM_CASES])
def test_bwd_norm_shapes(io, shape, axis):
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-norm", shape, axis, io)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    ln = rand_ln(rng, E)
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "norm %s %s axis %d" % (shape, io, axis), ln=ln)


@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_norm_saved_and_ragged(axis, io, saved):
    B, h, w, E, R = 3, 21, 10, 136, 9
    rng = np.random.default_rng(301 + axis + (saved is not None))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    ln = rand_ln(rng, E)
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "norm ragged %s axis %d" % (io, axis), saved=saved, ln=ln)


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 17, 42])
def test_bwd_norm_masked(axis, io, K):
    B, h, w, E, R = 4, 6, 7, 96, 6
    rng = np.random.default_rng(400 + K + 7 * axis)
    x, z, dout = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    ln = rand_ln(rng, E)
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "norm masked K=%d %s axis %d" % (K, io, axis), idx=idx, hw=(h, w),
              ln=ln)


def test_bwd_norm_masked_invalid_indices():
    """With the LayerNorm too, tokens with an invalid index get NaN in dx and
    dz and the rest (every gradient included) equals the oracle on the valid
    tokens."""
    B, h, w, E, R, K = 3, 5, 6, 48, 4, 9
    rng = np.random.default_rng(23)
    idx = random_mask(rng, B, h, w, K)
    idx[0, 2] = h * w
    idx[1, 4] = idx[1, 7]
    idx[2, 0] = -5
    x, z, dout = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    ln = rand_ln(rng, E)
    got = gpu_bwd(x, z, dout, prm, P.POOL_ROWS, idx=idx, hw=(h, w), ln=ln)
    invalid = {(0, 2), (1, 4), (1, 7), (2, 0)}
    refs = []
    for b in range(B):
        keep = [k for k in range(K) if (b, k) not in invalid]
        bad = [k for k in range(K) if (b, k) in invalid]
        for name in ("dx", "dz"):
            assert np.all(np.isnan(got[name][b, bad])), "invalid token of image %d not NaN in %s" % (b, name)
        ref = oracle.layer_bwd(x[b:b + 1, keep], z[b:b + 1, keep], dout[b:b + 1, keep], prm["fwd"], prm["bwd"],
                               P.POOL_ROWS, idx=idx[b:b + 1, keep], hw=(h, w), ln=ln)
        check(got["dx"][b:b + 1, keep], ref["dx"], FP32_TOL, "norm invalid-index image %d dx" % b)
        check(got["dz"][b:b + 1, keep], ref["dz"], FP32_TOL, "norm invalid-index image %d dz" % b)
        refs.append(ref)
    for d in DIRECTIONS:
        for f in FIELDS:
            check(got[d][f], sum(r[d][f] for r in refs), FP32_TOL, "norm invalid-index d%s.%s" % (d, f))
    for f in ("weight", "bias"):
        check(got["ln"][f], sum(r["ln"][f] for r in refs), FP32_TOL, "norm invalid-index d ln_" + f)


def test_bwd_norm_deterministic_and_empty():
    """Fixed-order sums with the norm too; B = 0 zeroes the norm's gradients."""
    B, h, w, E, R = 3, 12, 20, 200, 12
    rng = np.random.default_rng(7)
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    ln = rand_ln(rng, E)
    a = gpu_bwd(x, z, dout, prm, P.POOL_COLS, ln=ln)
    b = gpu_bwd(x, z, dout, prm, P.POOL_COLS, ln=ln)
    for k in ("dx", "dz"):
        assert np.array_equal(a[k], b[k])
    for f in ("weight", "bias"):
        assert np.array_equal(a["ln"][f], b["ln"][f])
    pd = dev_params(prm)
    xe = torch.empty((0, h, w, E), device="cuda")
    grads = {d: {f: torch.full_like(pd[d][f], 7.0) for f in FIELDS} for d in DIRECTIONS}
    grads["ln"] = {f: torch.full((E,), 7.0, device="cuda") for f in ("weight", "bias")}
    res = P.BwdCall(xe, xe.clone(), xe.clone(), pd, P.POOL_COLS, grads=grads, ln=_dev_ln(ln)).run()
    torch.cuda.synchronize()
    for f in ("weight", "bias"):
        assert torch.count_nonzero(res["ln"][f]).item() == 0


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_norm_full_size_2048(axis):
    _sampled_full_size(C.HIRES_2048, axis, saved=0 if axis == P.POOL_COLS else None, norm=True)


def test_bwd_norm_full_size_vim_s():
    _sampled_full_size(C.SHORT_224_S, norm=True)


def test_bwd_norm_full_size_masked_b():
    _sampled_full_size(C.MASKED_B, norm=True)


# ------------------------------------------------------------------ LBMamba's local backward scan
# scan lengths below, at and above one window, with a partial last window, and the longest
LOCAL_T = [1, 7, 16, 21, 48, 128]


def _local_case(rng, T, axis, io, B=2, P_=5, E=72, R=6, masked=False):
    h, w = (T, P_) if axis == P.POOL_COLS else (P_, T)
    if masked:
        K = max(1, (h * w) // 2)
        shape, idx, hw = (B, K, E), random_mask(rng, B, h, w, K), (h, w)
    else:
        shape, idx, hw = (B, h, w, E), None, None
    x, z, dout = (rng.standard_normal(shape).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    return x, z, dout, prm, idx, hw


def _local_check(x, z, dout, prm, axis, io, tag, idx=None, hw=None, saved=None, ln=None, pool_scale=None):
    tol, dt = _tol(io)
    got = gpu_bwd(x, z, dout, prm, axis, idx=idx, hw=hw, dtype=dt, flags=P.FLAG_LOCAL_BWD, saved=saved, ln=ln,
                  pool_scale=pool_scale)
    ref = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], axis, idx=idx, hw=hw, ln=ln,
                           pool_scale=1.0 if pool_scale is None else pool_scale, local_window=P.LOCAL_WINDOW)
    compare(got, ref, tol, tag)
    for f in FIELDS[:4]:  # the backward set's unused parameters get zero gradients
        assert np.count_nonzero(got["bwd"][f]) == 0, tag + " nonzero d bwd." + f
    return got


@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("T", LOCAL_T)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_local_scan(io, axis, T, saved):
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-local", io, axis, T, saved)).encode()))
    x, z, dout, prm, idx, hw = _local_case(rng, T, axis, io)
    _local_check(x, z, dout, prm, axis, io, "local T=%d %s axis %d" % (T, io, axis), saved=saved)


@pytest.mark.parametrize("variant", ["masked", "norm", "pool_scale", "masked_norm_scale"])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_local_scan_options(axis, variant):
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-local-opt", axis, variant)).encode()))
    masked = variant.startswith("masked")
    x, z, dout, prm, idx, hw = _local_case(rng, 37, axis, "f32", E=136, masked=masked)
    ln = rand_ln(rng, x.shape[-1]) if "norm" in variant else None
    scale = 0.25 if "scale" in variant else None
    _local_check(x, z, dout, prm, axis, "f32", "local %s axis %d" % (variant, axis), idx=idx, hw=hw, ln=ln,
                 pool_scale=scale)


def test_bwd_local_scan_backward_set_may_be_null():
    """Only D of the backward set is read: the call with the other four
    absent gives the same gradients as with them present."""
    rng = np.random.default_rng(88)
    x, z, dout, prm, idx, hw = _local_case(rng, 30, P.POOL_COLS, "f32")
    full = gpu_bwd(x, z, dout, prm, P.POOL_COLS, flags=P.FLAG_LOCAL_BWD)
    slim = {"fwd": prm["fwd"], "bwd": {"D": prm["bwd"]["D"]}}
    xd, zd = dev(x), dev(z)
    pd = {"fwd": {k: dev(v) for k, v in slim["fwd"].items()}, "bwd": {"D": dev(slim["bwd"]["D"])}}
    res = P.BwdCall(xd, zd, dev(dout), pd, P.POOL_COLS, flags=P.FLAG_LOCAL_BWD).run()
    torch.cuda.synchronize()
    assert np.array_equal(host(res["dx"]), full["dx"]) and np.array_equal(host(res["dz"]), full["dz"])
    for d in DIRECTIONS:
        for f in FIELDS:
            assert np.array_equal(host(res[d][f]), full[d][f]), (d, f)


def test_bwd_local_scan_full_size_2048():
    _sampled_full_size(C.HIRES_2048, P.POOL_COLS, saved=0, local=True)


# ------------------------------------------------------------------ producer Conv1D
# grids whose sequence windows cross grid rows (COLS) or columns (ROWS) at
# every size, including one- and two-cell axes, and every channel slicing
CONV_SHAPES = [(2, 5, 7, 8, 3), (2, 13, 9, 72, 6), (1, 7, 33, 136, 12), (2, 16, 16, 384, 12), (1, 3, 2, 200, 5),
               (1, 1, 1, 8, 1), (1, 2, 40, 1032, 33), (2, 31, 1, 64, 4)]


@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("shape", CONV_SHAPES, ids=["x".join(map(str, s)) for s in CONV_SHAPES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_conv(io, axis, shape, saved):
    B, h, w, E, R = shape
    if (h if axis == P.POOL_COLS else w) > 128:
        pytest.skip("scan longer than the backward pass supports")
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-conv", shape, axis, io, saved)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "conv %s %s axis %d" % (shape, io, axis), saved=saved, conv=conv)


@pytest.mark.parametrize("variant", ["pool_scale", "local", "local_scale"])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_conv_options(axis, variant):
    B, h, w, E, R = 2, 21, 18, 136, 9
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-conv-opt", axis, variant)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    flags = P.FLAG_LOCAL_BWD if "local" in variant else 0
    scale = 0.25 if "scale" in variant else None
    bwd_check(x, z, dout, prm, axis, FP32_TOL, torch.float32, "conv %s axis %d" % (variant, axis), conv=conv,
              flags=flags, pool_scale=scale)


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_conv_full_size_2048(axis):
    _sampled_full_size(C.HIRES_2048, axis, saved=0 if axis == P.POOL_COLS else None, with_conv=True)


# ---------------------------------------- Conv1D written out: block and masked
@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_conv_norm_block(io, axis, saved):
    """The whole block's gradients (Conv1D and LayerNorm together): dx through
    the conv, dz, both parameter sets, the norm's and the conv's weight and
    bias, on a grid whose runs of the conv's adjoint cross rows and columns."""
    B, h, w, E, R = 2, 21, 18, 136, 9
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-block", axis, io, saved)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "block %s axis %d" % (io, axis), saved=saved, conv=rand_conv(rng, E),
              ln=rand_ln(rng, E))


# grids whose conv lines (grid rows for COLS, columns for ROWS) hold 1 to 3
# cells: the conv's adjoint walks chunks of several lines, finishing dx of the
# runs before the current one, and reads its halo past a chunk's end
BLOCK_SHORT_LINES = [(3, 3, 2, 64, 4), (2, 1, 5, 72, 5), (2, 7, 1, 72, 5), (1, 2, 40, 136, 9), (2, 5, 3, 8, 3)]


@pytest.mark.parametrize("shape", BLOCK_SHORT_LINES, ids=["x".join(map(str, s)) for s in BLOCK_SHORT_LINES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_conv_norm_block_short_lines(io, axis, shape):
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-block-short", shape, axis, io)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "block %s axis %d %s" % (io, axis, shape), conv=rand_conv(rng, E),
              ln=rand_ln(rng, E))


@pytest.mark.parametrize("variant", ["pool_scale", "local"])
def test_bwd_conv_norm_block_options(variant):
    B, h, w, E, R = 2, 12, 10, 64, 5
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-block-opt", variant)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    bwd_check(x, z, dout, prm, P.POOL_ROWS, FP32_TOL, torch.float32, "block " + variant, conv=rand_conv(rng, E),
              ln=rand_ln(rng, E), flags=P.FLAG_LOCAL_BWD if variant == "local" else 0,
              pool_scale=0.25 if variant == "pool_scale" else None)


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
@pytest.mark.parametrize("saved", [None, 0], ids=SAVED_IDS)
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_conv_masked(io, axis, saved, norm):
    """Masked layers with the Conv1D along the kept tokens (more kept tokens
    than one run of the conv's adjoint, so its halo is used)."""
    B, h, w, K, E, R = 3, 12, 11, 100, 72, 6
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-conv-masked", axis, io, saved, norm)).encode()))
    x, z, dout = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    tol, dt = _tol(io)
    bwd_check(x, z, dout, prm, axis, tol, dt, "masked conv %s axis %d" % (io, axis), idx=idx, hw=(h, w),
              saved=saved, conv=rand_conv(rng, E), ln=rand_ln(rng, E) if norm else None)


@pytest.mark.parametrize("K", [1, 2, 5])
@pytest.mark.parametrize("io", ["f32"])
def test_bwd_conv_masked_few_tokens(io, K):
    """Masked layers keeping fewer tokens than the conv's window: runs shorter
    than three positions, one per image.  (fp32 only: in bf16 the written-out
    x_conv is rounded to bf16, and with a handful of tokens per image the
    scan parameters' gradients do not average that rounding below the bf16
    bar; test_bwd_conv_masked covers bf16 with 100 tokens.)"""
    B, h, w, E, R = 5, 4, 3, 72, 6
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-conv-masked-few", io, K)).encode()))
    x, z, dout = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(3))
    x, z, dout = _io(io, x, z, dout)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    tol, dt = _tol(io)
    for axis in (P.POOL_COLS, P.POOL_ROWS):
        bwd_check(x, z, dout, prm, axis, tol, dt, "masked conv K=%d %s axis %d" % (K, io, axis), idx=idx,
                  hw=(h, w), conv=rand_conv(rng, E), ln=rand_ln(rng, E) if K != 2 else None)


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_conv_norm_block_full_size_2048(axis):
    _sampled_full_size(C.HIRES_2048, axis, saved=0 if axis == P.POOL_COLS else None, norm=True, with_conv=True)


@pytest.mark.parametrize("variant", ["saved", "block", "conv"])
def test_bwd_full_size_gradients_everywhere(variant):
    """2048^2 with an upstream gradient on every image (the image groups,
    every run of the conv's adjoint and every pass-2 workgroup carry data):
    dx and dz of sampled images against the oracle on those images alone
    (an image's dx and dz depend only on its own inputs)."""
    cfg = C.HIRES_2048
    wl = draw_workload(cfg)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    rng = np.random.default_rng(83)
    dout = rng.standard_normal(x.shape).astype(np.float32)
    ln = rand_ln(np.random.default_rng(84), cfg.E) if variant == "block" else None
    conv = rand_conv(np.random.default_rng(85), cfg.E) if variant in ("block", "conv") else None
    axis = P.POOL_ROWS if variant == "block" else P.POOL_COLS
    print("\n[%s bwd, gradients on every image] %s" % (cfg.name, variant), flush=True)
    got = gpu_bwd(x, z, dout, prm, axis, saved=0, ln=ln, conv=conv)
    for i in (0, cfg.B // 2, cfg.B - 1):
        s = np.array([i])
        ref = oracle.layer_bwd(x[s], z[s], dout[s], prm["fwd"], prm["bwd"], axis, ln=ln, conv=conv)
        check(got["dx"][s], ref["dx"], FP32_TOL, "image %d dx" % i)
        check(got["dz"][s], ref["dz"], FP32_TOL, "image %d dz" % i)


def test_bwd_conv_masked_full_size():
    _sampled_full_size(C.MASKED_B, saved=0, with_conv=True)


# ------------------------------------------------- scans longer than 128 steps
LONG_BWD = [
    # B, h, w, E, R, axis: up to the scan adjoint's longest (720 steps at dt
    # rank <= 16, 512 at <= 32, 384 at <= 48, 288 at <= 64)
    (2, 200, 3, 64, 8, P.POOL_COLS),
    (1, 2, 720, 64, 12, P.POOL_ROWS),
    (1, 512, 2, 40, 30, P.POOL_COLS),
    (1, 3, 288, 48, 64, P.POOL_ROWS),
]


@pytest.mark.parametrize("local", [False, True], ids=["global", "local"])
@pytest.mark.parametrize("case", LONG_BWD, ids=["x".join(map(str, c)) for c in LONG_BWD])
def test_bwd_long_scans(case, local):
    B, h, w, E, R, axis = case
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-long", case, local)).encode()))
    x, z, dout = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(3))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    bwd_check(x, z, dout, prm, axis, FP32_TOL, torch.float32, "long %s" % (case,), saved=0 if local else None,
              flags=P.FLAG_LOCAL_BWD if local else 0)


# ------------------------------------------------------------------ image groups
# A backward call in image groups: each group's first pass, scan adjoint
# (on the library's second stream) and second pass, and the groups' parameter
# sums added at the end.  dx and dz are per-image results and must equal the
# single-group call's bit for bit; the parameter gradients differ only by the
# order of their sums.
GROUP_CASES = [
    # B, h, w, E, R, groups
    (7, 12, 10, 64, 4, 3),    # groups of 3, 3 and 1 images
    (5, 9, 14, 136, 12, 5),   # one image a group
    (3, 16, 16, 64, 8, 32),   # more groups asked for than images
]
GROUP_VARIANTS = ["plain", "saved", "norm", "conv", "block", "local", "masked", "masked_conv", "bf16"]


def _group_inputs(case, variant):
    B, h, w, E, R, groups = case
    rng = np.random.default_rng(zlib.crc32(repr(("bwd-groups", case, variant)).encode()))
    masked = variant.startswith("masked")
    K = (h * w * 2) // 3
    shape = (B, K, E) if masked else (B, h, w, E)
    x, z, dout = (rng.standard_normal(shape).astype(np.float32) for _ in range(3))
    io = "bf16" if variant == "bf16" else "f32"
    x, z, dout = _io(io, x, z, dout)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    kw = dict(dtype=_tol(io)[1])
    if masked:
        kw.update(idx=random_mask(rng, B, h, w, K), hw=(h, w))
    if variant == "saved":
        kw["saved"] = P.FLAG_FUSED
    if variant in ("norm", "block"):
        kw["ln"] = rand_ln(rng, E)
    if variant in ("conv", "block", "masked_conv"):
        kw["conv"] = rand_conv(rng, E)
    if variant == "local":
        kw["flags"] = P.FLAG_LOCAL_BWD
    return (x, z, dout, prm), kw, groups, io


def _same(a, b, tag):
    assert np.array_equal(a, b, equal_nan=True), tag + " differs from the single-group call"


@pytest.mark.parametrize("variant", GROUP_VARIANTS)
@pytest.mark.parametrize("case", GROUP_CASES, ids=["x".join(map(str, c)) for c in GROUP_CASES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_bwd_groups_match_single_group(axis, case, variant):
    args, kw, groups, io = _group_inputs(case, variant)
    one = gpu_bwd(*args, axis, groups=1, **kw)
    many = gpu_bwd(*args, axis, groups=groups, **kw)
    tag = "groups=%d %s axis %d %s" % (groups, variant, axis, case)
    _same(many["dx"], one["dx"], tag + " dx")
    _same(many["dz"], one["dz"], tag + " dz")
    compare(many, one, FP32_TOL, tag)
    again = gpu_bwd(*args, axis, groups=groups, **kw)
    for d in DIRECTIONS:
        for f in FIELDS:
            _same(again[d][f], many[d][f], tag + " rerun d%s.%s" % (d, f))


@pytest.mark.parametrize("variant", ["plain", "block", "masked_conv"])
def test_bwd_groups_against_oracle(variant):
    """The grouped call against the oracle directly (with its D = 0 twin)."""
    args, kw, groups, io = _group_inputs(GROUP_CASES[0], variant)
    x, z, dout, prm = args
    tol, dt = _tol(io)
    for axis in (P.POOL_COLS, P.POOL_ROWS):
        local = P.LOCAL_WINDOW if kw.get("flags", 0) & P.FLAG_LOCAL_BWD else 0
        got = gpu_bwd(x, z, dout, prm, axis, groups=groups, **kw)
        ref = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], axis, idx=kw.get("idx"), hw=kw.get("hw"),
                               ln=kw.get("ln"), conv=kw.get("conv"), local_window=local)
        compare(got, ref, tol, "grouped %s axis %d" % (variant, axis))
        p0 = zero_D(prm)
        got0 = gpu_bwd(x, z, dout, p0, axis, groups=groups, **kw)
        ref0 = oracle.layer_bwd(x, z, dout, p0["fwd"], p0["bwd"], axis, idx=kw.get("idx"), hw=kw.get("hw"),
                                ln=kw.get("ln"), conv=kw.get("conv"), local_window=local)
        compare(got0, ref0, tol, "grouped %s axis %d (D=0)" % (variant, axis), params=False)


def test_bwd_groups_default_at_full_size_is_deterministic():
    """The 2048^2 layer runs in the library's default grouping: two calls give
    bitwise identical results, and they equal the single-group call's dx and
    dz bit for bit."""
    wl = draw_workload(C.HIRES_2048)
    rng = np.random.default_rng(81)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    dout = rng.standard_normal(x.shape).astype(np.float32)
    print("\n[2048^2 bwd] default grouping twice, then one group", flush=True)
    xd, zd, dd, pd = dev(x), dev(z), dev(dout), dev_params(prm)
    res = []
    for groups in (0, 0, 1):
        r = P.BwdCall(xd, zd, dd, pd, P.POOL_COLS, groups=groups).run()
        torch.cuda.synchronize()
        res.append({"dx": r["dx"].clone(), "dz": r["dz"].clone(),
                    **{d: {f: r[d][f].clone() for f in FIELDS} for d in DIRECTIONS}})
        del r
    a, b, one = res
    for k in ("dx", "dz"):
        assert torch.equal(a[k], b[k]), k
        assert torch.equal(a[k], one[k]), k
    for d in DIRECTIONS:
        for f in FIELDS:
            assert torch.equal(a[d][f], b[d][f]), (d, f)
            check(host(a[d][f]), host(one[d][f]), FP32_TOL, "default grouping d%s.%s" % (d, f))
