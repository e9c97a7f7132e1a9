"""The C ABI's call forms beyond fastvim_ssm_fwd, on the GPU:

- fastvim_ssm_fwd_stages: the layer and its pooled tokens, both scan outputs
  and the mask rows in one call, against the oracle (and bit for bit against
  the exports of an ordinary call);
- a NULL workspace (stream-ordered scratch) for the forward, stages and
  backward calls, bit for bit against the same call with a caller workspace
  and against the oracle;
- fastvim_get_device_error: FASTVIM_FLAG_CHECK_IDX reports a repeated or
  out-of-range mask index (forward and backward), nothing without the flag
  or with valid indices; a single launch whose waits are made to give up
  after one poll (FASTVIM_TUNING_POLL1, set from the host: every kernel still
  finishes) reports FASTVIM_ERR_DEVICE_WAIT, and every output element is NaN
  (it followed a failed wait) or equal to a normal call's;
- calls enqueued on a side stream.
Bars as the parity tests: 1e-4 fp32, bit-exact rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import pooled_selective_state_amd as P
from gpu_util import FP32_TOL, check, dev, dev_params, gpu_call, host
from pins import rand_dir
from pooled_selective_state_amd import configs as C
from pooled_selective_state_amd.inputs import draw_workload, random_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    P.lib()
    yield
    torch.cuda.synchronize()


def _dense_case(seed, B=3, h=9, w=7, E=96, R=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B, h, w, E)).astype(np.float32)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    return x, z, prm


def _masked_case(seed, B=4, h=6, w=7, K=20, E=64, R=6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, K, E)).astype(np.float32)
    z = rng.standard_normal((B, K, E)).astype(np.float32)
    idx = random_mask(rng, B, h, w, K)
    prm = {"fwd": rand_dir(rng, E, 16, R, 0.1), "bwd": rand_dir(rng, E, 16, R, 0.1)}
    return x, z, idx, prm


@pytest.mark.parametrize("flags", [P.FLAG_STAGED, P.FLAG_FUSED], ids=["staged", "fused"])
@pytest.mark.parametrize("axis", [P.POOL_COLS, P.POOL_ROWS, P.POOL_NONE_ROWMAJOR])
def test_fwd_stages_dense(axis, flags):
    x, z, prm = _dense_case(200 + axis)
    call = gpu_call(x, z, prm, axis, flags=flags)
    res = call.run_stages()
    torch.cuda.synchronize()
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, stages=True)
    tag = "stages axis %d" % axis
    check(host(res["out"]), ref["out"], FP32_TOL, tag + " out")
    check(host(res["s_fwd"]), ref["fwd"]["s"], FP32_TOL, tag + " s_fwd")
    check(host(res["s_bwd"]), ref["bwd"]["s"], FP32_TOL, tag + " s_bwd")
    if axis in (P.POOL_COLS, P.POOL_ROWS):
        check(host(res["u"]), ref["u"], FP32_TOL, tag + " u")
        assert torch.equal(res["u"], call.export(P.EXPORT_U))
    else:
        assert "u" not in res
    # the same call's workspace holds what was copied out
    assert torch.equal(res["s_fwd"], call.export(P.EXPORT_S_FWD))
    assert torch.equal(res["s_bwd"], call.export(P.EXPORT_S_BWD))


@pytest.mark.parametrize("axis", [P.POOL_COLS, P.POOL_ROWS])
def test_fwd_stages_masked_rows_exact(axis):
    x, z, idx, prm = _masked_case(210 + axis)
    h, w = 6, 7
    call = gpu_call(x, z, prm, axis, idx=idx, hw=(h, w))
    res = call.run_stages()
    torch.cuda.synchronize()
    ref = oracle.layer(x, z, prm["fwd"], prm["bwd"], axis, idx=idx, hw=(h, w), stages=True)
    assert np.array_equal(host(res["rows"]).astype(np.int64), ref["rows"]), "rows not bit-exact"
    check(host(res["out"]), ref["out"], FP32_TOL, "masked stages out")
    check(host(res["u"]), ref["u"], FP32_TOL, "masked stages u")
    check(host(res["s_fwd"]), ref["fwd"]["s"], FP32_TOL, "masked stages s_fwd")
    check(host(res["s_bwd"]), ref["bwd"]["s"], FP32_TOL, "masked stages s_bwd")


@pytest.mark.parametrize("case", ["dense_fused", "dense_staged", "masked", "unpooled", "hires_default"])
def test_null_workspace_forward(case):
    """A NULL workspace gives the same bits as a caller workspace."""
    if case == "hires_default":
        wl = draw_workload(C.HIRES_2048, batch=4)  # the single launch by default
        x, z, prm, idx, hw, axis, flags = wl["x"], wl["z"][0], wl["params"][0], None, None, P.POOL_COLS, 0
    elif case == "masked":
        x, z, idx, prm = _masked_case(220)
        hw, axis, flags = (6, 7), P.POOL_ROWS, 0
    else:
        x, z, prm = _dense_case(221)
        idx = hw = None
        axis = P.POOL_NONE_COLMAJOR if case == "unpooled" else P.POOL_COLS
        flags = {"dense_fused": P.FLAG_FUSED, "dense_staged": P.FLAG_STAGED}.get(case, 0)
    a = gpu_call(x, z, prm, axis, idx=idx, hw=hw, flags=flags)
    want = a.run().clone()
    b = P.SSMCall(a.x, a.z, dev_params(prm), axis, mask_idx=a.mask_idx, hw=hw, flags=flags,
                  workspace=P.NO_WORKSPACE)
    assert b.params.workspace is None
    got = b.run()
    torch.cuda.synchronize()
    assert torch.equal(got, want), case
    with pytest.raises(P.FastVimError, match="WORKSPACE"):
        b.export(P.EXPORT_S_FWD)
    sel = np.array([0, x.shape[0] - 1])
    ref = oracle.layer(x[sel], z[sel], prm["fwd"], prm["bwd"], axis, idx=None if idx is None else idx[sel], hw=hw)
    check(host(got[sel]), ref, FP32_TOL, "NULL workspace " + case)
    # the stages call with a NULL workspace copies before the scratch is freed
    st = P.SSMCall(a.x, a.z, dev_params(prm), axis, mask_idx=a.mask_idx, hw=hw, flags=flags,
                   workspace=P.NO_WORKSPACE).run_stages()
    torch.cuda.synchronize()
    assert torch.equal(st["out"], want)
    assert torch.equal(st["s_fwd"], a.export(P.EXPORT_S_FWD))
    assert torch.equal(st["s_bwd"], a.export(P.EXPORT_S_BWD))


@pytest.mark.parametrize("masked", [False, True], ids=["dense", "masked"])
def test_null_workspace_backward(masked):
    if masked:
        x, z, idx, prm = _masked_case(230)
        hw = (6, 7)
    else:
        x, z, prm = _dense_case(231)
        idx = hw = None
    dout = np.random.default_rng(232).standard_normal(x.shape).astype(np.float32)
    xd, zd, dd = dev(x), dev(z), dev(dout)
    idd = None if idx is None else dev(idx, torch.int32)
    pd = dev_params(prm)
    want = P.BwdCall(xd, zd, dd, pd, P.POOL_COLS, mask_idx=idd, hw=hw).run()
    got = P.BwdCall(xd, zd, dd, pd, P.POOL_COLS, mask_idx=idd, hw=hw, workspace=P.NO_WORKSPACE).run()
    torch.cuda.synchronize()
    assert torch.equal(got["dx"], want["dx"]) and torch.equal(got["dz"], want["dz"])
    for d in ("fwd", "bwd"):
        for f in P.binding.DIR_FIELDS:
            assert torch.equal(got[d][f], want[d][f]), (d, f)
    ref = oracle.layer_bwd(x, z, dout, prm["fwd"], prm["bwd"], P.POOL_COLS, idx=idx, hw=hw)
    check(host(got["dx"]), ref["dx"], FP32_TOL, "NULL workspace backward dx")
    check(host(got["fwd"]["x_proj_w"]), ref["fwd"]["x_proj_w"], FP32_TOL, "NULL workspace backward dWx")


def test_check_idx_reports_bad_index():
    x, z, idx, prm = _masked_case(240)
    hw = (6, 7)
    bad = idx.copy()
    bad[2, 3] = bad[2, 9]  # a repeated index in image 2
    for indices, flags, expect in ((idx, P.FLAG_CHECK_IDX, None), (bad, 0, None),
                                   (bad, P.FLAG_CHECK_IDX, "BAD_INDEX")):
        call = gpu_call(x, z, prm, P.POOL_COLS, idx=indices, hw=hw, flags=flags)
        out = host(call.run())
        if expect is None:
            call.check_device()
        else:
            with pytest.raises(P.FastVimError, match=expect):
                call.check_device()
        nan_tok = np.isnan(out).all(axis=-1)
        assert nan_tok.sum() == (2 if indices is bad else 0)
    # the status word is the last call's: a clean call after a bad one reports nothing
    call = gpu_call(x, z, prm, P.POOL_COLS, idx=bad, hw=hw, flags=P.FLAG_CHECK_IDX)
    call.run()
    with pytest.raises(P.FastVimError, match="BAD_INDEX"):
        call.check_device()
    clean = P.SSMCall(call.x, call.z, dev_params(prm), P.POOL_COLS, mask_idx=dev(idx, torch.int32), hw=hw,
                      workspace=call.workspace, flags=P.FLAG_CHECK_IDX)
    clean.run(check_device=True)
    # the backward pass reports through its own workspace
    dout = dev(np.ones(x.shape, np.float32))
    bcall = P.BwdCall(call.x, call.z, dout, dev_params(prm), P.POOL_COLS, mask_idx=dev(bad, torch.int32), hw=hw,
                      flags=P.FLAG_CHECK_IDX)
    with pytest.raises(P.FastVimError, match="BAD_INDEX"):
        bcall.run(check_device=True)
    P.BwdCall(call.x, call.z, dout, dev_params(prm), P.POOL_COLS, mask_idx=dev(idx, torch.int32), hw=hw,
              flags=P.FLAG_CHECK_IDX).run(check_device=True)


@pytest.mark.parametrize("axis", [P.POOL_COLS, P.POOL_ROWS])
def test_single_launch_give_up_poisons_outputs(axis):
    """Every wait allowed one poll, with both lags at one image, so output
    items start while their image's scans still run: their waits give up.
    Each output element is then NaN (its block followed a give-up, or its
    scan rows came from a scan item whose wait gave up) or equal to the
    normal call's, and the device error is reported."""
    wl = draw_workload(C.CHAIN_1024, batch=12)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    normal = gpu_call(x, z, prm, axis, flags=P.FLAG_FUSED)
    want = normal.run().clone()
    normal.check_device()
    forced = P.SSMCall(normal.x, normal.z, dev_params(prm), axis, flags=P.FLAG_FUSED,
                       tuning=P.tuning_lags(1, 1) | P.TUNING_POLL1)
    got = forced.run()
    torch.cuda.synchronize()
    nan = torch.isnan(got)
    assert bool(nan.any()), "no wait gave up: the case does not exercise the give-up path"
    assert torch.equal(got[~nan], want[~nan])
    assert int(forced.export(P.EXPORT_STATUS).item()) & 1
    with pytest.raises(P.FastVimError, match="DEVICE_WAIT"):
        forced.check_device()
    # the next normal call on the same workspace starts from a cleared status
    again = P.SSMCall(normal.x, normal.z, dev_params(prm), axis, flags=P.FLAG_FUSED, workspace=forced.workspace)
    assert torch.equal(again.run(check_device=True), want)


def test_lag_tuning_keeps_results():
    """Lags chosen through the tuning word change the schedule, not the bits."""
    wl = draw_workload(C.CHAIN_1024, batch=10)
    x, z, prm = wl["x"], wl["z"][0], wl["params"][0]
    base = gpu_call(x, z, prm, P.POOL_COLS, flags=P.FLAG_FUSED)
    want = base.run().clone()
    for ls, le in ((1, 1), (2, 5), (3, 12), (4, 2)):
        got = P.SSMCall(base.x, base.z, dev_params(prm), P.POOL_COLS, flags=P.FLAG_FUSED,
                        tuning=P.tuning_lags(ls, le)).run(check_device=True)
        assert torch.equal(got, want), (ls, le)


def test_side_stream():
    """Calls enqueued on a side stream (the binding allocates out and the
    workspace on the current stream and records them on the side stream)."""
    x, z, prm = _dense_case(250, B=4, h=16, w=16, E=128)
    want = host(gpu_call(x, z, prm, P.POOL_COLS).run())
    side = torch.cuda.Stream()
    xd, zd, pd = dev(x), dev(z), dev_params(prm)
    torch.cuda.current_stream().synchronize()
    outs = []
    for _ in range(3):
        outs.append(P.ssm_fwd(xd, zd, pd, P.POOL_COLS, stream=side))
    side.synchronize()
    for o in outs:
        assert np.array_equal(host(o), want)
    dout = dev(np.ones(x.shape, np.float32))
    res = P.ssm_bwd(xd, zd, dout, pd, P.POOL_COLS, stream=side)
    side.synchronize()
    ref = P.ssm_bwd(xd, zd, dout, pd, P.POOL_COLS)
    torch.cuda.synchronize()
    assert torch.equal(res["dx"], ref["dx"])
