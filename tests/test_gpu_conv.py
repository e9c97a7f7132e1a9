"""GPU parity of the producer-fused layer (FASTVIM_FLAG_CONV): x is the input
of the depthwise causal Conv1D + SiLU, which the pool and the epilogue compute
on load, against the fp64 oracle (whose conv is pinned to numpy's
convolution).  Compared element by element, each tensor on its own scale:
out, out of the D = 0 twin, and the pooled tokens (the pool of x_conv).
Bar: 1e-4 fp32, 2e-2 bf16 (oracle on the bf16-rounded inputs).
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, check, gpu_call, host
from pins import rand_conv, rand_dir
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import draw_workload, round_to_bf16, zero_D

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


def test_conv_ignores_fused_flag():
    """The single launch does not take the conv: FASTVIM_FLAG_FUSED falls back
    to the stage kernels and gives the same result."""
    B, h, w, E, R = 2, 6, 5, 32, 4
    rng = np.random.default_rng(61)
    x, z = (rng.standard_normal((B, h, w, E)).astype(np.float32) for _ in range(2))
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    conv = rand_conv(rng, E)
    a = host(gpu_call(x, z, prm, P.POOL_COLS, conv=conv, flags=P.FLAG_FUSED).run())
    b = host(gpu_call(x, z, prm, P.POOL_COLS, conv=conv, flags=P.FLAG_STAGED).run())
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
