"""fastvim_ssm_fwd_noalloc, the entry point that allocates nothing (its
scratch is the library's fixed per-GPU buffer), against fastvim_ssm_fwd with
a workspace of its own, through the C ABI.

Two calls in a row, the second on a smaller input, so the second finds the
first one's intermediates and counters in the shared buffer: each output
must still equal fastvim_ssm_fwd's (bar 1e-4 fp32, 2e-2 bf16; the kernels
are the same, so they agree bit for bit).  Covered: the single launch (its
counters live in the buffer), the stage kernels, masked layers (row ids),
bf16, and a layer too large for the buffer (FASTVIM_ERR_SCRATCH, nothing
run).  Collected last, since it leaves the buffer in use.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import pooled_selective_state_amd as P
from gpu_util import BF16_TOL, FP32_TOL, dev, dev_params, rel_inf
from pins import rand_dir
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import draw_workload, random_mask, round_to_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _pair(x, z, prm, axis, dtype=torch.float32, idx=None, hw=None, flags=0):
    """(no-alloc output, output of fastvim_ssm_fwd with its own workspace)."""
    xd, zd = dev(x, dtype), dev(z, dtype)
    idd = None if idx is None else dev(idx, torch.int32)
    pd = dev_params(prm)
    out = torch.empty_like(xd)
    na = P.SSMCall(xd, zd, pd, axis, mask_idx=idd, hw=hw, out=out, workspace=P.NO_WORKSPACE, flags=flags)
    got = na.run_noalloc()
    want = P.SSMCall(xd, zd, pd, axis, mask_idx=idd, hw=hw, flags=flags).run()
    torch.cuda.synchronize()
    return got, want


def _agree(got, want, tol, what):
    g = got.float().cpu().numpy().astype(np.float64)
    w = want.float().cpu().numpy().astype(np.float64)
    err = rel_inf(g, w)
    print("  %-40s rel_inf=%.3e (tol %.0e)" % (what, err, tol), flush=True)
    assert err <= tol, what
    assert torch.equal(got, want), what + ": not bit-identical to fastvim_ssm_fwd"


def test_noalloc_two_calls_single_launch_then_smaller():
    """2048^2 images (the single launch, counters in the buffer), then a
    smaller 1024^2 batch on the same buffer."""
    big = draw_workload(C.HIRES_2048, batch=6)
    got, want = _pair(big["x"], big["z"][0], big["params"][0], P.POOL_COLS)
    _agree(got, want, FP32_TOL, "2048^2 B=6 COLS (single launch)")
    small = draw_workload(C.CHAIN_1024, batch=3)
    got, want = _pair(small["x"], small["z"][0], small["params"][0], P.POOL_ROWS, flags=P.FLAG_FUSED)
    _agree(got, want, FP32_TOL, "1024^2 B=3 ROWS (single launch), second call")


def test_noalloc_two_calls_stage_kernels_then_smaller():
    rng = np.random.default_rng(300)
    for B, h, w, E, R in ((8, 24, 20, 256, 16), (2, 5, 7, 64, 4)):
        x = rng.standard_normal((B, h, w, E)).astype(np.float32)
        z = rng.standard_normal((B, h, w, E)).astype(np.float32)
        prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
        for axis in (P.POOL_COLS, P.POOL_NONE_COLMAJOR):
            got, want = _pair(x, z, prm, axis, flags=P.FLAG_STAGED)
            _agree(got, want, FP32_TOL, "staged %dx%dx%dx%d axis %d" % (B, h, w, E, axis))


def test_noalloc_masked_bf16_then_smaller():
    wl = draw_workload(C.MASKED_B)
    got, want = _pair(wl["x"], wl["z"][0], wl["params"][0], P.POOL_COLS, dtype=torch.bfloat16, idx=wl["idx"],
                      hw=(14, 14))
    _agree(got, want, BF16_TOL, "masked Vim-B B=256 bf16")
    rng = np.random.default_rng(301)
    B, h, w, K, E, R = 3, 6, 7, 11, 64, 6
    x = round_to_bf16(rng.standard_normal((B, K, E)).astype(np.float32))
    z = round_to_bf16(rng.standard_normal((B, K, E)).astype(np.float32))
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    got, want = _pair(x, z, prm, P.POOL_ROWS, dtype=torch.bfloat16, idx=idx, hw=(h, w))
    _agree(got, want, BF16_TOL, "masked small bf16 ROWS, second call")


def test_noalloc_rejects_layers_beyond_the_buffer():
    rng = np.random.default_rng(302)
    B, h, w, E, R = 4, 128, 128, 256, 4  # unpooled: (B, h*w) tokens of projections and scan outputs
    need = P.workspace_bytes(P.make_dims(B, h, w, E, 16, R), P.POOL_NONE_ROWMAJOR)
    assert need > P.binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, h, w, E), device="cuda")
    prm = {d: {k: dev(v) for k, v in rand_dir(rng, E, 16, R).items()} for d in ("fwd", "bwd")}
    out = torch.full_like(x, 7.0)
    call = P.SSMCall(x, x.clone(), prm, P.POOL_NONE_ROWMAJOR, out=out, workspace=P.NO_WORKSPACE)
    with pytest.raises(P.FastVimError, match="SCRATCH"):
        call.run_noalloc()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call wrote its output"
    # the buffer still serves the next call
    wl = draw_workload(C.TINY)
    got, want = _pair(wl["x"], wl["z"][0], wl["params"][0], P.POOL_COLS)
    _agree(got, want, FP32_TOL, "tiny after a rejected call")
