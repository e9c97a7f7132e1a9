"""GPU parity of LBMamba's local backward scan (FASTVIM_FLAG_LOCAL_BWD)
against the fp64 oracle, whose local scan is pinned to the global scan (one
window), a closed form (windows of one step) and window-by-window reverse
scans.  The backward parameter set passed to the library holds only D, so
the test also shows that nothing else of it is read.  Dense pooled layers run
both as stage kernels and as the single launch (whose scan items then run
the local scan); the 2048^2 layer takes the single launch by default.  Compared element by
element, each on its own scale: out, out of the D = 0 twin, and both scan
outputs.  Bar: 1e-4 fp32, 2e-2 bf16.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, check, dev, host
from pins import rand_dir
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import draw_workload, random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu
L = P.LOCAL_WINDOW


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _run(x, z, prm, axis, dtype, idx=None, hw=None, flags=0):
    pd = {"fwd": {k: dev(v) for k, v in prm["fwd"].items()}, "bwd": {"D": dev(prm["bwd"]["D"])}}
    call = P.SSMCall(dev(x, dtype), dev(z, dtype), pd, axis, mask_idx=None if idx is None else dev(idx, torch.int32),
                     hw=hw, flags=P.FLAG_LOCAL_BWD | flags)
    out = host(call.run())
    torch.cuda.synchronize()
    return out, host(call.export(P.EXPORT_S_FWD)), host(call.export(P.EXPORT_S_BWD))


def local_check(x, z, prm, axis, tol, dtype, tag, idx=None, hw=None, sel=None, flags=0):
    s = slice(None) if sel is None else sel
    out, sf, sb = _run(x, z, prm, axis, dtype, idx, hw, flags)
    twin, _, _ = _run(x, z, zero_D(prm), axis, dtype, idx, hw, flags)
    ix = None if idx is None else idx[s]
    ref = oracle.layer(x[s], z[s], prm["fwd"], prm["bwd"], axis, idx=ix, hw=hw, stages=True, local_window=L)
    ref0 = oracle.layer(x[s], z[s], zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis, idx=ix, hw=hw, local_window=L)
    check(out[s], ref["out"], tol, tag + " out")
    check(twin[s], ref0, tol, tag + " out(D=0)")
    check(sf[s], ref["fwd"]["s"], tol, tag + " s_fwd")
    check(sb[s], ref["bwd"]["s"], tol, tag + " s_bwd (local)")


SHAPES = [
    # B, h, w, E, R: scans shorter than a window, exactly one, one plus a step, ragged, and several windows
    (2, 5, 7, 72, 5),
    (1, 16, 3, 40, 12),
    (2, 17, 4, 64, 20),
    (1, 37, 2, 136, 33),
    (2, 128, 3, 48, 12),
]
AXES = (P.POOL_COLS, P.POOL_ROWS, P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR)


PATHS = {"staged": P.FLAG_STAGED, "fused": P.FLAG_FUSED}  # FUSED falls back to stage kernels where unsupported


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
@pytest.mark.parametrize("axis", AXES)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_local_layer(shape, axis, io, path):
    if path == "fused" and axis not in (P.POOL_COLS, P.POOL_ROWS):
        pytest.skip("the single launch covers pooled layers only")
    B, h, w, E, R = shape
    rng = np.random.default_rng(zlib.crc32(repr(("local", shape, axis, io)).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    local_check(x, z, prm, axis, FP32_TOL if io == "f32" else BF16_TOL,
                torch.float32 if io == "f32" else torch.bfloat16, "local %s %s axis %d %s" % (shape, io, axis, path),
                flags=PATHS[path])


@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_local_masked(axis):
    B, h, w, E, R, K = 3, 20, 18, 64, 6, 50
    rng = np.random.default_rng(70 + axis)
    x, z = (rng.standard_normal((B, K, E)).astype(np.float32) for _ in range(2))
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    local_check(x, z, prm, axis, FP32_TOL, torch.float32, "local masked axis %d" % axis, idx=idx, hw=(h, w))


@pytest.mark.parametrize("axis,flags", [(P.POOL_COLS, 0), (P.POOL_COLS, P.FLAG_STAGED), (P.POOL_ROWS, 0),
                                        (P.POOL_NONE_ROWMAJOR, 0)],
                         ids=["cols-default", "cols-staged", "rows-default", "unpooled"])
def test_local_full_size_2048(axis, flags):
    cfg = C.HIRES_2048
    wl = draw_workload(cfg)
    sel = np.array([0, cfg.B - 1]) if axis in (P.POOL_COLS, P.POOL_ROWS) else np.array([cfg.B // 2])
    print("\n[%s local, axis %d, flags %d] B=%d grid=%dx%d E=%d" % (cfg.name, axis, flags, cfg.B, cfg.h, cfg.w,
                                                                  cfg.E), flush=True)
    local_check(wl["x"], wl["z"][0], wl["params"][0], axis, FP32_TOL, torch.float32,
                "%s local axis %d" % (cfg.name, axis), sel=sel, flags=flags)
