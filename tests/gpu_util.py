"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP layer through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import pooled_selective_state_amd as P
from pooled_selective_state_amd.inputs import DIRECTIONS

FP32_TOL = 1e-4   # max |gpu - oracle| / max |oracle|, fp32 I/O
BF16_TOL = 2e-2   # same metric, bf16 I/O (oracle on the bf16-rounded inputs)


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype)


def dev_params(params):
    return {d: {k: dev(v) for k, v in params[d].items()} for d in DIRECTIONS}


def host(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_inf(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    scale = np.max(np.abs(ref))
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref)) / max(scale, 1e-30))


class MaxErr:
    """rel_inf accumulated over pieces of a tensor (images compared in groups):
    max |gpu - oracle| and max |oracle| per named tensor, so the error checked
    at the end is that of the whole tensor."""

    def __init__(self):
        self.num, self.den = {}, {}

    def add(self, what, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (what, got.shape, ref.shape)
        assert np.all(np.isfinite(got)), "non-finite GPU output in " + what
        if ref.size:
            self.num[what] = max(self.num.get(what, 0.0), float(np.max(np.abs(got - ref))))
            self.den[what] = max(self.den.get(what, 0.0), float(np.max(np.abs(ref))))

    def check(self, tol):
        for what in self.num:
            err = self.num[what] / max(self.den[what], 1e-30)
            print("  %-28s rel_inf=%.3e (tol %.0e)" % (what, err, tol), flush=True)
            assert err <= tol, "%s: rel_inf %.3e > %.1e" % (what, err, tol)


def check(got, ref, tol, what):
    err = rel_inf(got, ref)
    print("  %-28s rel_inf=%.3e (tol %.0e)" % (what, err, tol), flush=True)
    assert err <= tol, "%s: rel_inf %.3e > %.1e" % (what, err, tol)
    return err


def io_dtype(cfg_or_name):
    return torch.bfloat16 if cfg_or_name == "bf16" else torch.float32


def gpu_call(x, z, params, axis, idx=None, hw=None, dtype=torch.float32, flags=0, ln=None, conv=None,
             pool_scale=None, tuning=0):
    """Prepared call on device copies of numpy inputs; returns the SSMCall.
    ln: None or {"weight", "bias", "eps"} (numpy) for the post-SSM LayerNorm;
    conv: None or {"weight", "bias"} (numpy) for the producer Conv1D;
    pool_scale: None or the factor on the pooled tokens; tuning: the params.tuning word."""
    xd, zd = dev(x, dtype), dev(z, dtype)
    idd = None if idx is None else dev(idx, torch.int32)
    lnd = None if ln is None else {"weight": dev(ln["weight"]), "bias": dev(ln["bias"]), "eps": ln["eps"]}
    cvd = None if conv is None else {"weight": dev(conv["weight"]), "bias": dev(conv["bias"])}
    return P.SSMCall(xd, zd, dev_params(params), axis, mask_idx=idd, hw=hw, flags=flags, ln=lnd, conv=cvd,
                     pool_scale=pool_scale, tuning=tuning)


def status_ok(call):
    """The single-launch kernel's status word is 0 (no wait gave up)."""
    st = int(call.export(P.EXPORT_STATUS).cpu().item())
    assert st == 0, "fused-kernel status %#x" % st


def stage_exports(call):
    out = {
        "xdbl": host(call.export(P.EXPORT_XDBL)),
        "s_fwd": host(call.export(P.EXPORT_S_FWD)),
        "s_bwd": host(call.export(P.EXPORT_S_BWD)),
    }
    if call.pool_axis in (P.POOL_COLS, P.POOL_ROWS):
        out["u"] = host(call.export(P.EXPORT_U))
    return out


def compare_stages(got, ref, tol, tag):
    """GPU stage exports vs the oracle's stage outputs (each on its own scale)."""
    if "u" in got:
        check(got["u"], ref["u"], tol, tag + " u")
    NX = ref["fwd"]["v"].shape[-1]
    check(got["xdbl"][..., 0, :NX], ref["fwd"]["v"], tol, tag + " x_proj fwd")
    check(got["xdbl"][..., 1, :NX], ref["bwd"]["v"], tol, tag + " x_proj bwd")
    check(got["s_fwd"], ref["fwd"]["s"], tol, tag + " s_fwd")
    check(got["s_bwd"], ref["bwd"]["s"], tol, tag + " s_bwd")
