"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Every comparison is element by element with the max-norm relative error
max|gpu - oracle| / max|oracle| on each tensor's own scale: out, out of the
D = 0 twin (so the D*x skip cannot hide the scan), and the stage exports
(pooled tokens, x_proj outputs, both scan outputs).  Bar: 1e-4 for fp32 I/O,
2e-2 for bf16 I/O (oracle on the bf16-rounded inputs), bit-exact for mask
rows.  Full-size workloads run entirely on the GPU in the launch
configuration the benchmark times; the oracle checks a sample of images
(images are independent, so the oracle on a subset equals the full oracle
restricted to it).
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import (BF16_TOL, FP32_TOL, MaxErr, check, compare_stages, dev, dev_params, gpu_call, host,
                      rel_inf, stage_exports, status_ok)
from pins import rand_dir, rand_ln
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import draw_workload, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu

AXES = (P.POOL_COLS, P.POOL_ROWS, P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR)
# the two paths of a dense pooled layer, forced (by default the library picks by size)
PATHS = {"staged": P.FLAG_STAGED, "fused": P.FLAG_FUSED}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _layer_check(x, z, prm, axis, tol, dtype, tag, idx=None, hw=None, sel=None, flags=0, ln=None, chunk=None):
    """Run GPU layer + D=0 twin, compare out / twin / stages with the oracle
    on images ``sel`` (all if None).  chunk: run the oracle on that many
    images at a time (the error is still taken over all compared images)."""
    call = gpu_call(x, z, prm, axis, idx=idx, hw=hw, dtype=dtype, flags=flags, ln=ln)
    out = call.run()
    torch.cuda.synchronize()
    status_ok(call)
    st = stage_exports(call)
    rows = host(call.export(P.EXPORT_ROWS)).astype(np.int64) if idx is not None else None
    tcall = gpu_call(x, z, zero_D(prm), axis, idx=idx, hw=hw, dtype=dtype, flags=flags, ln=ln)
    twin = tcall.run()
    torch.cuda.synchronize()
    status_ok(tcall)
    images = np.arange(x.shape[0]) if sel is None else np.asarray(sel)
    step = len(images) if chunk is None else chunk
    acc = MaxErr()
    NXr = prm["fwd"]["x_proj_w"].shape[0]
    for i in range(0, len(images), max(step, 1)):
        s = images[i:i + step]
        ids = None if idx is None else idx[s]
        ref = oracle.layer(x[s], z[s], prm["fwd"], prm["bwd"], axis, idx=ids, hw=hw, stages=True, ln=ln)
        ref0 = oracle.layer(x[s], z[s], zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis, idx=ids, hw=hw, ln=ln)
        acc.add(tag + " out", host(out[s]), ref["out"])
        acc.add(tag + " out(D=0)", host(twin[s]), ref0)
        if "u" in st:
            acc.add(tag + " u", st["u"][s], ref["u"])
        acc.add(tag + " x_proj fwd", st["xdbl"][s][..., 0, :NXr], ref["fwd"]["v"])
        acc.add(tag + " x_proj bwd", st["xdbl"][s][..., 1, :NXr], ref["bwd"]["v"])
        acc.add(tag + " s_fwd", st["s_fwd"][s], ref["fwd"]["s"])
        acc.add(tag + " s_bwd", st["s_bwd"][s], ref["bwd"]["s"])
        if idx is not None:
            assert np.array_equal(rows[s], ref["rows"]), tag + " rows not bit-exact"
    acc.check(tol)
    if idx is not None:
        assert int(host(call.export(P.EXPORT_BAD_TOKENS)).sum()) == 0
    return call


# ------------------------------------------------------------------ small / ragged
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("axis", AXES)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_tiny_fastvim_t_layer(axis, io, path):
    wl = draw_workload(C.TINY)
    x, z = wl["x"], wl["z"][0]
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    _layer_check(x, z, wl["params"][0], axis, FP32_TOL if io == "f32" else BF16_TOL,
                 torch.float32 if io == "f32" else torch.bfloat16, "tiny %s axis %d %s" % (io, axis, path),
                 flags=PATHS[path])


# Short, wide pooled layers (E >= 1024 and enough pooled tokens for 192
# workgroups of 32 tokens) take the projection with 32-token workgroups and
# 8 waves over E: every image against the oracle (out, D = 0 twin, u, both
# x_proj directions, both scan outputs); the second case has a token count
# off multiples of 32 and E off multiples of 16 (the tail step of E).
SHORT_WIDE = [
    # B, h, w, E, R
    (48, 64, 2, 1024, 16),
    (50, 62, 3, 1032, 20),
]


@pytest.mark.parametrize("shape", SHORT_WIDE, ids=["x".join(map(str, s)) for s in SHORT_WIDE])
def test_projection_short_wide(shape):
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr(shape).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    _layer_check(x, z, prm, P.POOL_COLS, FP32_TOL, torch.float32, "short wide %s" % (shape,), chunk=16)


RAGGED = [
    # B, h, w, E, R   (E not a multiple of 64, row counts not multiples of 32, odd grids)
    (3, 13, 7, 72, 5),
    (1, 1, 1, 8, 1),
    (2, 5, 9, 200, 20),
    (2, 3, 33, 136, 64),
    (1, 37, 2, 1032, 33),
]


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("shape", RAGGED, ids=["x".join(map(str, s)) for s in RAGGED])
@pytest.mark.parametrize("axis", AXES)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ragged_shapes(shape, axis, io, path):
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr((shape, axis, io)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    _layer_check(x, z, prm, axis, FP32_TOL if io == "f32" else BF16_TOL,
                 torch.float32 if io == "f32" else torch.bfloat16, "ragged %s %s axis %d %s" % (shape, io, axis, path),
                 flags=PATHS[path])


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 17, 42])
def test_masked_small(axis, io, K):
    B, h, w, E, R = 5, 6, 7, 64, 6
    rng = np.random.default_rng(100 + K + 7 * axis)
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    _layer_check(x, z, prm, axis, FP32_TOL if io == "f32" else BF16_TOL,
                 torch.float32 if io == "f32" else torch.bfloat16, "masked K=%d %s axis %d" % (K, io, axis),
                 idx=idx, hw=(h, w))


@pytest.mark.parametrize("R", [1, 16, 17, 33, 64])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_NONE_COLMAJOR))
def test_projection_every_tile_count(R, axis):
    """The matrix-core projection covers 2(R + 32) output columns in tiles of
    16 (5 to 12 tiles for R = 1..64): every tile count's edge, a token count
    that is not a multiple of 16 (3 x 5 x 7 grid) and an E whose tail is not a
    multiple of the 16-wide k-step (E = 100)."""
    rng = np.random.default_rng(40 + R)
    B, h, w, E, N = 3, 5, 7, 100, 16
    x = rng.standard_normal((B, h, w, E), dtype=np.float32)
    z = rng.standard_normal((B, h, w, E), dtype=np.float32)
    prm = {d: rand_dir(rng, E, N, R, scale=0.1) for d in ("fwd", "bwd")}
    _layer_check(x, z, prm, axis, FP32_TOL, torch.float32, "proj R=%d" % R, flags=P.FLAG_STAGED)


@pytest.mark.parametrize("path", list(PATHS))
def test_step_size_extremes(path):
    """Step-size biases spread over [-25, 25] with tiny dt_proj weights drive
    softplus through all of its regimes: the identity above 20, e^q itself
    where 1 + e^q rounds to 1, and the log1p range between."""
    rng = np.random.default_rng(50)
    B, h, w, E, N, R = 2, 9, 6, 96, 16, 8
    x = rng.standard_normal((B, h, w, E), dtype=np.float32)
    z = rng.standard_normal((B, h, w, E), dtype=np.float32)
    prm = {}
    for d in ("fwd", "bwd"):
        p = rand_dir(rng, E, N, R, scale=0.05)
        p["dt_proj_w"] = (1e-3 * rng.standard_normal((E, R))).astype(np.float32)
        p["dt_proj_b"] = np.linspace(-25.0, 25.0, E).astype(np.float32)
        prm[d] = p
    _layer_check(x, z, prm, P.POOL_COLS, FP32_TOL, torch.float32, "softplus extremes", flags=PATHS[path])


@pytest.mark.parametrize("R", [1, 33, 64])
@pytest.mark.parametrize("axis", (P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR))
def test_projection_many_tokens(R, axis):
    """From 64 k tokens the projection switches to row-tiled waves over the
    whole of E: 256 x 257 tokens (not a multiple of the 128-row workgroup)
    with E = 100 (an E tail), compared with the oracle's x_proj of the
    tokens in scan order."""
    rng = np.random.default_rng(60 + R)
    B, h, w, E, N = 1, 256, 257, 100, 16
    x = rng.standard_normal((B, h, w, E), dtype=np.float32)
    z = rng.standard_normal((B, h, w, E), dtype=np.float32)
    prm = {d: rand_dir(rng, E, N, R, scale=0.1) for d in ("fwd", "bwd")}
    call = gpu_call(x, z, prm, axis, flags=P.FLAG_STAGED)
    call.stage(P.STAGE_PROJ)
    got = host(call.export(P.EXPORT_XDBL))
    torch.cuda.synchronize()
    seq = x if axis == P.POOL_NONE_ROWMAJOR else x.transpose(0, 2, 1, 3)
    seq = np.ascontiguousarray(seq).reshape(B, h * w, E)
    for d, name in enumerate(("fwd", "bwd")):
        check(got[:, :, d, :], oracle.xproj(seq, prm[name]["x_proj_w"]), FP32_TOL, "x_proj %s R=%d" % (name, R))


# ------------------------------------------------------------ scans longer than 128 steps
LONG = [
    # B, h, w, E, R, axis: more scan steps than the single launch's scan items
    # hold in LDS (128 at dt rank <= 16, 96 at <= 32, 64 at <= 64)
    (2, 200, 3, 64, 8, P.POOL_COLS),
    (2, 5, 300, 72, 20, P.POOL_ROWS),
    (1, 97, 4, 40, 40, P.POOL_COLS),
    (1, 2, 720, 64, 12, P.POOL_ROWS),
]


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", LONG, ids=["x".join(map(str, c)) for c in LONG])
def test_long_scans(case, path):
    """The single launch's scan items stage such a sequence's rows chunk by
    chunk; the stage kernels take any length."""
    B, h, w, E, R, axis = case
    rng = np.random.default_rng(zlib.crc32(repr(("long", case)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    _layer_check(x, z, prm, axis, FP32_TOL, torch.float32, "long %s %s" % (case, path), flags=PATHS[path])
    for flags in (P.FLAG_LOCAL_BWD, P.FLAG_LOCAL_BWD | PATHS[path]):
        call = gpu_call(x, z, prm, axis, flags=flags)
        out = host(call.run())
        torch.cuda.synchronize()
        status_ok(call)
        ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, local_window=P.LOCAL_WINDOW)
        check(out, ref, FP32_TOL, "long local %s %s" % (case, path))


# ------------------------------------------------------------ post-SSM LayerNorm
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("axis", AXES)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_post_norm_tiny(axis, io, path):
    """The post-SSM LayerNorm before the gate, every pooling axis, both paths
    of a dense pooled layer (the single launch takes the norm for E / V <= 128)."""
    wl = draw_workload(C.TINY)
    x, z = wl["x"], wl["z"][0]
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    ln = rand_ln(np.random.default_rng(70 + axis), C.TINY.E)
    _layer_check(x, z, wl["params"][0], axis, FP32_TOL if io == "f32" else BF16_TOL,
                 torch.float32 if io == "f32" else torch.bfloat16, "norm tiny %d %s %s" % (axis, io, path), ln=ln,
                 flags=PATHS[path])


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("E", [8, 72, 520, 1032, 2056, 4096])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_post_norm_widths(E, io, path):
    """Every lane-team size of the normalising epilogue (16, 32 or 64 lanes per
    token, up to 16 vectors per lane) and widths that leave part of the team
    idle, on a ragged grid."""
    if io == "bf16" and E % 8:
        pytest.skip("bf16 needs E % 8 == 0")
    rng = np.random.default_rng(80 + E)
    B, h, w, N, R = 2, 3, 5, 16, 5
    x = rng.standard_normal((B, h, w, E), dtype=np.float32)
    z = rng.standard_normal((B, h, w, E), dtype=np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {d: rand_dir(rng, E, N, R, scale=0.05) for d in ("fwd", "bwd")}
    ln = rand_ln(rng, E, eps=1e-5)
    _layer_check(x, z, prm, P.POOL_ROWS, FP32_TOL if io == "f32" else BF16_TOL,
                 torch.float32 if io == "f32" else torch.bfloat16, "norm E=%d %s %s" % (E, io, path), ln=ln,
                 flags=PATHS[path])


def test_post_norm_masked_with_invalid_index():
    """Masked layer with the norm; a duplicated index gives NaN for exactly
    the tokens that carry it, the others match the oracle on the valid set."""
    rng = np.random.default_rng(90)
    B, h, w, K, E, N, R = 2, 6, 7, 11, 96, 16, 6
    x = rng.standard_normal((B, K, E), dtype=np.float32)
    z = rng.standard_normal((B, K, E), dtype=np.float32)
    prm = {d: rand_dir(rng, E, N, R, scale=0.05) for d in ("fwd", "bwd")}
    ln = rand_ln(rng, E)
    idx = random_mask(rng, B, h, w, K)
    _layer_check(x, z, prm, P.POOL_COLS, FP32_TOL, torch.float32, "norm masked", idx=idx, hw=(h, w), ln=ln)
    bad = idx.copy()
    bad[1, 3] = bad[1, 5]  # a duplicate in image 1
    call = gpu_call(x, z, prm, P.POOL_COLS, idx=bad, hw=(h, w), ln=ln)
    out = host(call.run())
    torch.cuda.synchronize()
    nan_tok = np.isnan(out).all(axis=-1)
    assert nan_tok[1, 3] and nan_tok[1, 5] and nan_tok.sum() == 2
    assert np.isfinite(out[~nan_tok]).all()


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("path", list(PATHS))
def test_post_norm_full_size_2048(path, axis):
    """The 2048^2 layer with the norm, both paths and axes, sampled images."""
    wl = _workload(C.HIRES_2048)
    ln = rand_ln(np.random.default_rng(95), C.HIRES_2048.E)
    _layer_check(wl["x"], wl["z"][0], wl["params"][0], axis, FP32_TOL, torch.float32,
                 "norm 2048 %s axis %d" % (path, axis), sel=_sample(C.HIRES_2048.B), ln=ln, flags=PATHS[path])


def test_masked_integer_sums_exact():
    """x[b, k, :] = k + 1: the pooled sums are small integers, exact in fp32,
    so u * P must equal them bit for bit."""
    B, h, w, E, R, K = 4, 9, 8, 32, 4, 30
    rng = np.random.default_rng(7)
    idx = random_mask(rng, B, h, w, K)
    x = np.broadcast_to((np.arange(K, dtype=np.float32) + 1)[None, :, None], (B, K, E)).copy()
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R), "bwd": rand_dir(rng, E, 16, R)}
    for axis, T, Pn in ((P.POOL_COLS, h, w), (P.POOL_ROWS, w, h)):
        call = gpu_call(x, z, prm, axis, idx=idx, hw=(h, w))
        call.run()
        u = host(call.export(P.EXPORT_U))
        rows = host(call.export(P.EXPORT_ROWS)).astype(np.int64)
        ref_rows = oracle.mask_rows(idx, h, w, axis)
        assert np.array_equal(rows, ref_rows)
        sums = np.zeros((B, T, E))
        for b in range(B):
            np.add.at(sums[b], rows[b], x[b].astype(np.float64))
        # u = fp32(sum * fp32(1/P)); multiply back in fp64 and round to the integer
        assert np.array_equal(np.rint(u * Pn), sums)
        assert np.max(np.abs(u - sums / Pn)) <= 1e-6 * max(1.0, np.max(sums / Pn))


def test_masked_invalid_indices():
    """Out-of-range and repeated indices: those tokens get NaN and are counted;
    the other tokens equal the oracle on the valid tokens alone."""
    B, h, w, E, R, K = 3, 5, 6, 48, 4, 9
    rng = np.random.default_rng(9)
    idx = random_mask(rng, B, h, w, K)
    idx[0, 2] = h * w          # out of range
    idx[1, 4] = idx[1, 7]      # duplicate pair: both invalid
    idx[2, 0] = -5             # negative
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    call = gpu_call(x, z, prm, P.POOL_COLS, idx=idx, hw=(h, w))
    out = host(call.run())
    bad = host(call.export(P.EXPORT_BAD_TOKENS)).astype(np.int64)
    assert list(bad) == [1, 2, 1]
    invalid = {(0, 2), (1, 4), (1, 7), (2, 0)}
    for b in range(B):
        keep = [k for k in range(K) if (b, k) not in invalid]
        assert np.all(np.isnan(out[b, [k for k in range(K) if (b, k) in invalid]]))
        ref = oracle.layer(x[b:b + 1, keep], z[b:b + 1, keep], prm["fwd"], prm["bwd"], P.POOL_COLS,
                           idx=idx[b:b + 1, keep], hw=(h, w))
        check(out[b:b + 1, keep], ref, FP32_TOL, "invalid-index image %d" % b)


def test_empty_batch():
    E = 16
    x = torch.empty((0, 3, 4, E), device="cuda")
    prm = {d: {k: dev(v) for k, v in rand_dir(np.random.default_rng(0), E, 16, 2).items()} for d in ("fwd", "bwd")}
    out = P.ssm_fwd(x, x.clone(), prm, P.POOL_COLS)
    assert out.shape == x.shape


# -------------------------------------------------------------- invariants on GPU
def test_width_one_pooling_equals_unpooled():
    rng = np.random.default_rng(3)
    B, h, E, R = 3, 11, 96, 8
    x = rng.standard_normal((B, h, 1, E)).astype(np.float32)
    z = rng.standard_normal((B, h, 1, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    a = host(gpu_call(x, z, prm, P.POOL_COLS).run())
    b = host(gpu_call(x, z, prm, P.POOL_NONE_ROWMAJOR).run())
    assert rel_inf(a, b) <= 1e-6


def test_rows_is_cols_on_transposed_grid():
    rng = np.random.default_rng(4)
    B, h, w, E, R = 2, 9, 6, 64, 8
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    xt, zt = x.transpose(0, 2, 1, 3).copy(), z.transpose(0, 2, 1, 3).copy()
    for a, b in ((P.POOL_ROWS, P.POOL_COLS), (P.POOL_NONE_COLMAJOR, P.POOL_NONE_ROWMAJOR)):
        ra = host(gpu_call(x, z, prm, a).run())
        rb = host(gpu_call(xt, zt, prm, b).run()).transpose(0, 2, 1, 3)
        assert rel_inf(ra, rb) <= 1e-6


@pytest.mark.parametrize("path", list(PATHS))
def test_deterministic(path):
    """Bit-identical results on repeated calls (no reduction depends on timing)."""
    wl = draw_workload(C.SHORT_224_S, batch=16)
    call = gpu_call(wl["x"], wl["z"][0], wl["params"][0], P.POOL_COLS, flags=PATHS[path])
    a = call.run().clone()
    b = call.run().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_fused_matches_staged(axis):
    """The single-launch kernel and the stage kernels agree to rounding on
    every stage output."""
    wl = draw_workload(C.CHAIN_1024, batch=6)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    f = gpu_call(x, z, prm, axis, flags=P.FLAG_FUSED)
    s = gpu_call(x, z, prm, axis, flags=P.FLAG_STAGED)
    of, os_ = host(f.run()), host(s.run())
    torch.cuda.synchronize()
    status_ok(f)
    assert rel_inf(of, os_) <= 1e-5
    for what in (P.EXPORT_U, P.EXPORT_XDBL, P.EXPORT_S_FWD, P.EXPORT_S_BWD):
        assert rel_inf(host(f.export(what)), host(s.export(what))) <= 1e-5, what


@pytest.mark.parametrize("flags", (P.FLAG_STAGED, P.FLAG_FUSED), ids=["staged", "fused"])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_saved_u_forward(axis, flags):
    """With saved_u the forward writes the pooled tokens to the caller's buffer
    (equal to the oracle's u, and to the workspace's u of a call without it),
    and out is bit for bit the same as without saved_u."""
    wl = draw_workload(C.CHAIN_1024, batch=4)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    plain = gpu_call(x, z, prm, axis, flags=flags)
    o1 = plain.run().clone()
    T = x.shape[1] if axis == P.POOL_COLS else x.shape[2]
    su = torch.full((x.shape[0], T, x.shape[-1]), float("nan"), device="cuda")
    kept = P.SSMCall(plain.x, plain.z, dev_params(prm), axis, flags=flags, saved_u=su)
    o2 = kept.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(su, plain.export(P.EXPORT_U))
    assert torch.equal(kept.export(P.EXPORT_U), su)
    sel = np.array([0, x.shape[0] - 1])
    ref = oracle.layer(x[sel], z[sel], prm["fwd"], prm["bwd"], axis, stages=True)
    check(host(su[sel]), ref["u"], FP32_TOL, "saved u")


def test_saved_u_forward_masked():
    B, h, w, E, R, K = 3, 6, 7, 64, 6, 20
    rng = np.random.default_rng(23)
    x, z = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(2))
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    su = torch.full((B, h, E), float("nan"), device="cuda")
    call = P.SSMCall(dev(x), dev(z), dev_params(prm), P.POOL_COLS, mask_idx=dev(idx, torch.int32), hw=(h, w),
                     saved_u=su)
    out = host(call.run())
    torch.cuda.synchronize()
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], P.POOL_COLS, idx=idx, hw=(h, w), stages=True)
    check(host(su), ref["u"], FP32_TOL, "masked saved u")
    check(out, ref["out"], FP32_TOL, "masked out with saved u")


# --------------------------------------------------------------- full-size workloads
_cache = {}


def _workload(cfg):
    if cfg.name not in _cache:
        _cache.clear()
        _cache[cfg.name] = draw_workload(cfg)
    return _cache[cfg.name]


def _sample(B):
    """Images that cover every interval of the single launch's pipeline (its
    fill, the steady state and its drain, for lags up to 16 images) and a few
    seeded random ones."""
    fixed = [0, 1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, B // 2, B - 18, B - 17, B - 16, B - 9, B - 8, B - 7, B - 4,
             B - 3, B - 2, B - 1]
    rnd = np.random.default_rng(B).integers(0, B, 4).tolist()
    return np.unique(np.array([b for b in fixed + rnd if 0 <= b < B]))


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("cfg", [C.SHORT_224_S, C.HIRES_2048, C.MASKED_B], ids=lambda c: c.name)
def test_full_size_pooled(cfg, path):
    """Every image of the workload against the oracle (the 2048^2 layer 16
    images per oracle call)."""
    wl = _workload(cfg)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    tol = BF16_TOL if cfg.io_dtype == "bf16" else FP32_TOL
    dtype = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32
    idx = wl["idx"]
    hw = (cfg.h, cfg.w) if cfg.masked else None
    print("\n[%s] B=%d grid=%dx%d E=%d" % (cfg.name, cfg.B, cfg.h, cfg.w, cfg.E), flush=True)
    _layer_check(x, z, prm, P.POOL_COLS, tol, dtype, cfg.name + " " + path, idx=idx, hw=hw,
                 chunk=16 if cfg.h * cfg.w > 4096 else None, flags=PATHS[path])


def test_full_size_chain_1024():
    """Two blocks: COLS on x, then ROWS (transposed grid) on block 1's output.
    Each block is compared with the oracle on its own input, on every image:
    out, the D = 0 twin (the skip term is about 2e4 times the scan output
    here, so out alone cannot show the scan) and the stage exports (pooled
    tokens, both x_proj directions, s_fwd, s_bwd).  Block 2's input is block
    1's GPU output, as the chain passes it on; the chain end to end is
    compared with the oracle's chain on a sample."""
    cfg = C.CHAIN_1024
    wl = _workload(cfg)
    x, z1, z2 = wl["x"], wl["z"][0], wl["z"][1]
    p1, p2 = wl["params"]
    c1 = _layer_check(x, z1, p1, P.POOL_COLS, FP32_TOL, torch.float32, "chain block 1", chunk=32)
    out1 = c1.out.cpu().numpy()
    c2 = _layer_check(out1, z2, p2, P.POOL_ROWS, FP32_TOL, torch.float32, "chain block 2", chunk=32)
    sel = _sample(cfg.B)
    r1 = oracle.layer(x[sel], z1[sel], p1["fwd"], p1["bwd"], P.POOL_COLS)
    r2 = oracle.layer(r1.astype(np.float32), z2[sel], p2["fwd"], p2["bwd"], P.POOL_ROWS)
    check(host(c2.out[sel]), r2, FP32_TOL, "chain end to end out")


@pytest.mark.parametrize("cfg", [C.CHAIN_1024, C.HIRES_2048], ids=lambda c: c.name)
@pytest.mark.parametrize("axis", [P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR])
def test_full_size_unpooled(cfg, axis):
    wl = _workload(cfg)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    print("\n[%s unpooled axis %d] T=%d" % (cfg.name, axis, cfg.h * cfg.w), flush=True)
    call = gpu_call(x, z, prm, axis)
    out = call.run()
    torch.cuda.synchronize()
    sel = np.array([cfg.B - 1])
    ref = oracle.layer(x[sel], z[sel], prm["fwd"], prm["bwd"], axis, stages=True)
    check(host(out[sel]), ref["out"], FP32_TOL, "unpooled out")
    check(host(call.export(P.EXPORT_S_FWD)[sel]), ref["fwd"]["s"], FP32_TOL, "unpooled s_fwd")
    check(host(call.export(P.EXPORT_S_BWD)[sel]), ref["bwd"]["s"], FP32_TOL, "unpooled s_bwd")
    xd = host(call.export(P.EXPORT_XDBL)[sel])
    NX = ref["fwd"]["v"].shape[-1]
    check(xd[..., 0, :NX], ref["fwd"]["v"], FP32_TOL, "unpooled x_proj fwd")


def test_default_path_selection():
    """Without flags the library runs small dense layers as stage kernels and
    layers with large images (>= 8 MiB of x each) as the single launch; both
    paths are deterministic, so the default matches the chosen one bit for bit."""
    small = draw_workload(C.SHORT_224_S, batch=8)
    big = draw_workload(C.HIRES_2048, batch=2)
    for wl, chosen in ((small, P.FLAG_STAGED), (big, P.FLAG_FUSED)):
        x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
        d = gpu_call(x, z, prm, P.POOL_COLS).run().clone()
        c = gpu_call(x, z, prm, P.POOL_COLS, flags=chosen).run().clone()
        torch.cuda.synchronize()
        assert torch.equal(d, c), chosen
