"""GPU parity of the scan and output stages run as one launch.

Short pooled layers on the stage kernels (scans of at most 64 steps, no
post-SSM LayerNorm, no Conv1D computed on load) run their scan and output
stages as one kernel by default for masked layers and images of at most 1024
tokens.  The tuning word forces either form: SCAN_OUT_TWO the separate scan
and output kernels, SCAN_OUT_ONE the single one.  Each case runs both forms
and checks, for each, out, its D = 0 twin and the stage exports (pooled
tokens, both x_proj directions, both scan outputs) against the fp64 oracle
at 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O), mask rows bit-exact; and the two
forms against each other bit for bit (the same arithmetic in the same order).
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, MaxErr, gpu_call, host, stage_exports, status_ok
from pins import rand_dir
from pooled_selective_state_amd.inputs import random_mask, round_to_bf16, zero_D

pytestmark = pytest.mark.gpu

FORMS = {"two": P.tuning_scan_out(P.SCAN_OUT_TWO), "one": P.tuning_scan_out(P.SCAN_OUT_ONE)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run_forms(x, z, prm, axis, dtype, tol, tag, idx=None, hw=None, flags=0, pool_scale=None, local=None):
    """Both forms on the GPU, each against the oracle, then against each other."""
    outs = {}
    for form, tuning in FORMS.items():
        kw = dict(idx=idx, hw=hw, dtype=dtype, flags=flags | P.FLAG_STAGED, pool_scale=pool_scale, tuning=tuning)
        call = gpu_call(x, z, prm, axis, **kw)
        out = call.run()
        tcall = gpu_call(x, z, zero_D(prm), axis, **kw)
        twin = tcall.run()
        torch.cuda.synchronize()
        status_ok(call)
        st = stage_exports(call)
        okw = dict(idx=idx, hw=hw, pool_scale=1.0 if pool_scale is None else pool_scale,
                   local_window=local or 0)
        ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, stages=True, **okw)
        ref0 = oracle.layer(x, z, zero_D(prm)["fwd"], zero_D(prm)["bwd"], axis, **okw)
        acc = MaxErr()
        t = "%s [%s]" % (tag, form)
        NXr = prm["fwd"]["x_proj_w"].shape[0]
        acc.add(t + " out", host(out), ref["out"])
        acc.add(t + " out(D=0)", host(twin), ref0)
        acc.add(t + " u", st["u"], ref["u"])
        acc.add(t + " x_proj fwd", st["xdbl"][..., 0, :NXr], ref["fwd"]["v"])
        if local is None:
            acc.add(t + " x_proj bwd", st["xdbl"][..., 1, :NXr], ref["bwd"]["v"])
        acc.add(t + " s_fwd", st["s_fwd"], ref["fwd"]["s"])
        acc.add(t + " s_bwd", st["s_bwd"], ref["bwd"]["s"])
        if idx is not None:
            rows = host(call.export(P.EXPORT_ROWS)).astype(np.int64)
            assert np.array_equal(rows, ref["rows"]), t + " rows not bit-exact"
        acc.check(tol)
        outs[form] = (out, twin)
    for k in range(2):
        a, b = _bits(outs["two"][k]), _bits(outs["one"][k])
        assert torch.equal(a, b), tag + " the two forms differ (%s)" % ("out", "out(D=0)")[k]


def _inputs(shape, io, seed_key, R):
    B, h, w, E = shape
    rng = np.random.default_rng(zlib.crc32(repr(seed_key).encode()))
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    return rng, x, z, prm


DENSE = [
    # B, h, w, E, R: E off multiples of 64, one cell, a 14 x 14 grid, scans of
    # 1, 5, 17 (past one chunk: matrix-core step sizes) and 64 (the longest) steps
    (3, 13, 7, 72, 5),
    (1, 1, 1, 8, 1),
    (2, 14, 14, 384, 12),
    (2, 17, 9, 1032, 33),
    (2, 64, 3, 200, 64),
    (2, 5, 64, 136, 48),
]


@pytest.mark.parametrize("shape", DENSE, ids=["x".join(map(str, s)) for s in DENSE])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_out_dense(shape, axis, io):
    B, h, w, E, R = shape
    _, x, z, prm = _inputs((B, h, w, E), io, (shape, axis, io), R)
    _run_forms(x, z, prm, axis, torch.float32 if io == "f32" else torch.bfloat16,
               FP32_TOL if io == "f32" else BF16_TOL, "dense %s axis %d %s" % (shape, axis, io))


@pytest.mark.parametrize("option", ["local", "pool_scale"])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
def test_scan_out_options(option, axis):
    shape = (3, 14, 11, 264, 24)
    B, h, w, E, R = shape
    _, x, z, prm = _inputs((B, h, w, E), "f32", (shape, axis, option), R)
    if option == "local":
        _run_forms(x, z, prm, axis, torch.float32, FP32_TOL, "local axis %d" % axis, flags=P.FLAG_LOCAL_BWD,
                   local=P.LOCAL_WINDOW)
    else:
        _run_forms(x, z, prm, axis, torch.float32, FP32_TOL, "pool scale axis %d" % axis, pool_scale=0.25)


MASKED = [
    # B, h, w, K, E, R: the masked Vim-B width, a ragged grid, every token kept,
    # the most kept tokens the one-launch mask validation and pooling takes
    # (1024), and more (1100: the mask-rows and per-row pooling kernels)
    (3, 14, 14, 49, 1536, 48),
    (2, 9, 13, 30, 136, 7),
    (2, 6, 5, 30, 72, 16),
    (1, 40, 33, 1024, 64, 8),
    (1, 40, 40, 1100, 64, 8),
]


@pytest.mark.parametrize("shape", MASKED, ids=["x".join(map(str, s)) for s in MASKED])
@pytest.mark.parametrize("axis", (P.POOL_COLS, P.POOL_ROWS))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_out_masked(shape, axis, io):
    B, h, w, K, E, R = shape
    rng, _, _, prm = _inputs((1, 1, 1, E), io, (shape, axis, io), R)
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    if io == "bf16":
        x, z = round_to_bf16(x), round_to_bf16(z)
    idx = random_mask(rng, B, h, w, K)
    _run_forms(x, z, prm, axis, torch.float32 if io == "f32" else torch.bfloat16,
               FP32_TOL if io == "f32" else BF16_TOL, "masked %s axis %d %s" % (shape, axis, io), idx=idx, hw=(h, w))


def test_scan_out_masked_invalid_index():
    """An out-of-range and a duplicated index: NaN at exactly those tokens in
    both forms, the forms equal bit for bit, and the other tokens equal the
    oracle on the valid tokens alone."""
    B, h, w, K, E, R = 2, 7, 6, 12, 72, 9
    rng, _, _, prm = _inputs((1, 1, 1, E), "f32", "invalid", R)
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    idx = random_mask(rng, B, h, w, K)
    idx[0, 2] = h * w + 2
    idx[1, 3] = idx[1, 5]
    invalid = {(0, 2), (1, 3), (1, 5)}
    outs = []
    for tuning in FORMS.values():
        call = gpu_call(x, z, prm, P.POOL_COLS, idx=idx, hw=(h, w), flags=P.FLAG_STAGED, tuning=tuning)
        outs.append(call.run())
    torch.cuda.synchronize()
    assert torch.equal(_bits(outs[0]), _bits(outs[1]))
    out = host(outs[1])
    for b in range(B):
        keep = [k for k in range(K) if (b, k) not in invalid]
        assert np.all(np.isnan(out[b, [k for k in range(K) if (b, k) in invalid]]))
        assert not np.isnan(out[b, keep]).any()
        ref = oracle.layer(x[b:b + 1, keep], z[b:b + 1, keep], prm["fwd"], prm["bwd"], P.POOL_COLS,
                           idx=idx[b:b + 1, keep], hw=(h, w))
        acc = MaxErr()
        acc.add("invalid-index image %d" % b, out[b:b + 1, keep], ref)
        acc.check(FP32_TOL)


def test_scan_out_default_matches_forced():
    """The default (automatic) form of a 14 x 14 layer is the one launch: same
    bits as SCAN_OUT_ONE."""
    shape = (2, 14, 14, 128)
    _, x, z, prm = _inputs(shape, "f32", "default", 12)
    res = []
    for tuning in (0, FORMS["one"]):
        call = gpu_call(x, z, prm, P.POOL_COLS, flags=P.FLAG_STAGED, tuning=tuning)
        res.append(call.run())
    torch.cuda.synchronize()
    assert torch.equal(_bits(res[0]), _bits(res[1]))
