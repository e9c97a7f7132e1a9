"""GPU parity of the producer-fused layer (FASTVIM_FLAG_CONV): x is the input
of the depthwise causal Conv1D + SiLU, which the pool and the epilogue compute
on load, against the fp64 oracle (whose conv is pinned to numpy's
convolution).  Compared element by element, each tensor on its own scale:
out, out of the D = 0 twin, and the pooled tokens (the pool of x_conv).
Bar: 1e-4 fp32, 2e-2 bf16 (oracle on the bf16-rounded inputs).

The second part covers the layers whose conv is written out once: the
whole FastVim block (Conv1D with the post-SSM LayerNorm) on both paths and
axes, masked layers (the conv along the kept tokens, rows bit-exact), and
unpooled layers; there the scan outputs are compared too.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, MaxErr, check, gpu_call, host, status_ok
from pins import rand_conv, rand_dir, rand_ln
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import draw_workload, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def conv_check(x, z, prm, conv, axis, tol, dtype, tag, sel=None, flags=0):
    s = slice(None) if sel is None else sel
    call = gpu_call(x, z, prm, axis, dtype=dtype, conv=conv, flags=flags)
    out = call.run()
    torch.cuda.synchronize()
    u = host(call.export(P.EXPORT_U))
    twin = gpu_call(x, z, zero_D(prm), axis, dtype=dtype, conv=conv, flags=flags).run()
    torch.cuda.synchronize()
    ref = oracle.layer(x[s], z[s], prm["fwd"], prm["bwd"], axis, stages=True, conv=conv)
    ref0 = oracle.layer(x[s], z[s], zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis, conv=conv)
    check(host(out[s]), ref["out"], tol, tag + " out")
    check(host(twin[s]), ref0, tol, tag + " out(D=0)")
    check(u[s], ref["u"], tol, tag + " pooled x_conv")


SHAPES = [
    # B, h, w, E, R   (grids smaller than the conv window: halos cross rows and columns and reach the start)
    (2, 5, 7, 72, 5),
    (1, 1, 1, 8, 1),
    (2, 3, 2, 16, 3),
    (1, 2, 5, 40, 4),
    (1, 17, 9, 136, 20),
    (2, 14, 14, 384, 12),
]


@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_layer(shape, axis, io):
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr(("conv", shape, axis, io)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    conv_check(x, z, prm, conv, axis, FP32_TOL if io == "f32" else BF16_TOL,
               torch.float32 if io == "f32" else torch.bfloat16, "conv %s %s axis %d" % (shape, io, axis))


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_conv_fused_flag_paths(axis):
    """FASTVIM_FLAG_FUSED: the single launch computes the conv on load (equal
    to the stage kernels within rounding)."""
    B, h, w, E, R = 2, 6, 5, 32, 4
    rng = np.random.default_rng(61)
    x, z = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(2))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    a = host(gpu_call(x, z, prm, axis, conv=conv, flags=P.FLAG_FUSED).run())
    b = host(gpu_call(x, z, prm, axis, conv=conv, flags=P.FLAG_STAGED).run())
    check(a, b, FP32_TOL, "axis %d single launch vs stage kernels" % axis)


# COLS layers on the single launch with the conv on load: grids whose runs
# of the conv's window cross grid rows (the first run of a row takes its halo
# from the previous row) and reach the image's start, and scans longer than
# the resident length (the LONG instances)
FUSED_SHAPES = SHAPES + [(2, 200, 6, 64, 12), (1, 97, 11, 40, 33), (3, 9, 130, 136, 20)]


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=["x".join(map(str, s)) for s in FUSED_SHAPES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_single_launch(shape, axis, io, norm):
    """out, its D = 0 twin, the pooled tokens and both scan outputs of the
    single launch with the Conv1D computed on load (and the post-SSM
    LayerNorm), against the oracle: COLS walks the conv's runs along the grid
    rows, ROWS down the columns."""
    B, h, w, E, R = shape
    if axis == P.POOL_ROWS:
        h, w = w, h  # the same scan lengths on the other axis
    rng = np.random.default_rng(zlib.crc32(repr(("conv-fused", shape, axis, io, norm)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    ln = rand_ln(rng, E) if norm else None
    block_check(x, z, prm, conv, axis, FP32_TOL if io == "f32" else BF16_TOL,
                torch.float32 if io == "f32" else torch.bfloat16,
                "single launch conv%s %s %s axis %d" % (" + norm" if norm else "", shape, io, axis), ln=ln,
                flags=P.FLAG_FUSED)


def test_conv_single_launch_options():
    """The single launch with the conv on load and the pool scale; with the
    local backward scan the conv goes to the stage kernels (same result as
    the staged call, bit for bit)."""
    B, h, w, E, R = 2, 19, 13, 64, 6
    rng = np.random.default_rng(65)
    x, z = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(2))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    call = gpu_call(x, z, prm, P.POOL_COLS, conv=conv, flags=P.FLAG_FUSED, pool_scale=0.25)
    out = host(call.run())
    torch.cuda.synchronize()
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], P.POOL_COLS, conv=conv, pool_scale=0.25)
    check(out, ref, FP32_TOL, "single launch conv, pool scale 0.25")
    a = host(gpu_call(x, z, prm, P.POOL_COLS, conv=conv, flags=P.FLAG_FUSED | P.FLAG_LOCAL_BWD).run())
    b = host(gpu_call(x, z, prm, P.POOL_COLS, conv=conv, flags=P.FLAG_STAGED | P.FLAG_LOCAL_BWD).run())
    assert np.array_equal(a, b)


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_conv_full_size_2048(axis):
    cfg = C.HIRES_2048
    wl = draw_workload(cfg)
    rng = np.random.default_rng(62)
    conv = rand_conv(rng, cfg.E)
    sel = np.array([0, cfg.B // 2, cfg.B - 1])
    print("\n[%s conv] B=%d grid=%dx%d E=%d" % (cfg.name, cfg.B, cfg.h, cfg.w, cfg.E), flush=True)
    conv_check(wl["x"], wl["z"][0], wl["params"][0], conv, axis, FP32_TOL, torch.float32,
               "%s conv axis %d" % (cfg.name, axis), sel=sel)


# ------------------------------------------------- the conv written out first
def block_check(x, z, prm, conv, axis, tol, dtype, tag, idx=None, hw=None, ln=None, flags=0, sel=None, chunk=None):
    """out, the D = 0 twin, the pooled tokens (pooled layers), both scan
    outputs and (masked) the rows, against the oracle on images sel (all if
    None), chunk images per oracle call."""
    call = gpu_call(x, z, prm, axis, idx=idx, hw=hw, dtype=dtype, conv=conv, ln=ln, flags=flags)
    out = call.run()
    torch.cuda.synchronize()
    status_ok(call)
    pooled = axis in (P.POOL_COLS, P.POOL_ROWS)
    u = host(call.export(P.EXPORT_U)) if pooled else None
    sf, sb = host(call.export(P.EXPORT_S_FWD)), host(call.export(P.EXPORT_S_BWD))
    rows = host(call.export(P.EXPORT_ROWS)).astype(np.int64) if idx is not None else None
    twin = gpu_call(x, z, zero_D(prm), axis, idx=idx, hw=hw, dtype=dtype, conv=conv, ln=ln, flags=flags).run()
    torch.cuda.synchronize()
    images = np.arange(x.shape[0]) if sel is None else np.asarray(sel)
    step = len(images) if chunk is None else chunk
    acc = MaxErr()
    for i in range(0, len(images), step):
        s = images[i:i + step]
        ids = None if idx is None else idx[s]
        ref = oracle.layer(x[s], z[s], prm["fwd"], prm["bwd"], axis, idx=ids, hw=hw, stages=True, conv=conv, ln=ln)
        ref0 = oracle.layer(x[s], z[s], zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis, idx=ids, hw=hw, conv=conv,
                            ln=ln)
        acc.add(tag + " out", host(out[s]), ref["out"])
        acc.add(tag + " out(D=0)", host(twin[s]), ref0)
        if pooled:
            acc.add(tag + " pooled x_conv", u[s], ref["u"])
        acc.add(tag + " s_fwd", sf[s], ref["fwd"]["s"])
        acc.add(tag + " s_bwd", sb[s], ref["bwd"]["s"])
        if idx is not None:
            assert np.array_equal(rows[s], ref["rows"]), tag + " rows not bit-exact"
    acc.check(tol)


PATHS = {"staged": P.FLAG_STAGED, "fused": P.FLAG_FUSED}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_norm_block(shape, axis, io, path):
    """The FastVim block in one call: Conv1D, pool, scans, repeat, skip,
    post-SSM LayerNorm, gate; the single launch takes the norm after the conv
    is written out."""
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr(("conv-norm", shape, axis, io)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv, ln = rand_conv(rng, E), rand_ln(rng, E)
    block_check(x, z, prm, conv, axis, FP32_TOL if io == "f32" else BF16_TOL,
                torch.float32 if io == "f32" else torch.bfloat16, "block %s %s axis %d %s" % (shape, io, axis, path),
                ln=ln, flags=PATHS[path])


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
@pytest.mark.parametrize("K", [1, 5, 30, 42])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_masked(axis, io, K, norm):
    """Masked layers: the conv along the kept tokens in their given order
    (fewer tokens than the conv's window included)."""
    B, h, w, E, R = 3, 6, 7, 64, 6
    rng = np.random.default_rng(zlib.crc32(repr(("conv-masked", axis, io, K, norm)).encode()))
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    ln = rand_ln(rng, E) if norm else None
    block_check(x, z, prm, conv, axis, FP32_TOL if io == "f32" else BF16_TOL,
                torch.float32 if io == "f32" else torch.bfloat16, "masked conv K=%d %s axis %d" % (K, io, axis),
                idx=idx, hw=(h, w), ln=ln)


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
@pytest.mark.parametrize("axis", (P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR))
def test_conv_unpooled(axis, norm):
    B, h, w, E, R = 2, 9, 7, 96, 8
    rng = np.random.default_rng(zlib.crc32(repr(("conv-unpooled", axis, norm)).encode()))
    x, z = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(2))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    block_check(x, z, prm, conv, axis, FP32_TOL, torch.float32, "unpooled conv axis %d" % axis,
                ln=rand_ln(rng, E) if norm else None)


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_conv_norm_block_full_size_2048(axis):
    """The whole block at 2048^2 on the default path (COLS: the single launch
    with the conv on load; ROWS: the conv written out, then the layer),
    images covering the pipeline's intervals."""
    cfg = C.HIRES_2048
    wl = draw_workload(cfg)
    rng = np.random.default_rng(63)
    conv, ln = rand_conv(rng, cfg.E), rand_ln(rng, cfg.E)
    sel = np.array([0, 1, 2, 3, 5, 7, 8, 9, 16, 64, 119, 120, 121, 124, 125, 126, 127])
    print("\n[%s conv + norm] B=%d grid=%dx%d E=%d axis %d" % (cfg.name, cfg.B, cfg.h, cfg.w, cfg.E, axis), flush=True)
    block_check(wl["x"], wl["z"][0], wl["params"][0], conv, axis, FP32_TOL, torch.float32,
                "%s conv+norm axis %d" % (cfg.name, axis), ln=ln, sel=sel, chunk=9)


@pytest.mark.parametrize("norm", [False, True], ids=["plain", "norm"])
def test_conv_masked_full_size(norm):
    """The masked Vim-B workload with the Conv1D, every image, bf16."""
    cfg = C.MASKED_B
    wl = draw_workload(cfg)
    rng = np.random.default_rng(64)
    conv = rand_conv(rng, cfg.E)
    ln = rand_ln(rng, cfg.E) if norm else None
    block_check(wl["x"], wl["z"][0], wl["params"][0], conv, P.POOL_COLS, BF16_TOL, torch.bfloat16,
                "%s conv" % cfg.name, idx=wl["idx"], hw=(cfg.h, cfg.w), ln=ln)
