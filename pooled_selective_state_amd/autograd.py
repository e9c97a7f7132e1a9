"""PyTorch autograd front end of the layer: forward through fastvim_ssm_fwd,
backward through fastvim_ssm_bwd (both HIP, through the C ABI).  Argument
marshalling only; every step of the layer runs in the library's kernels.

The forward call keeps the pooled tokens (saved_u) for the backward call, as
training keeps a layer's activations, so the backward pass does not pool x
again.  Gradients flow to x, z, both directions' parameters and, when given,
the post-SSM LayerNorm's and the producer Conv1D's weight and bias.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import torch

from . import binding as B

DIRS = ("fwd", "bwd")


class _PooledSSM(torch.autograd.Function):
    @staticmethod
    def forward(ctx, meta, x, z, *tensors):
        (pool_axis, mask_idx, hw, flags, ln_eps, pool_scale, has_ln, has_conv) = meta
        params = {d: dict(zip(B.DIR_FIELDS, tensors[5 * i:5 * i + 5])) for i, d in enumerate(DIRS)}
        k = 10
        ln = conv = None
        if has_ln:
            ln = {"weight": tensors[k], "bias": tensors[k + 1], "eps": ln_eps}
            k += 2
        if has_conv:
            conv = {"weight": tensors[k], "bias": tensors[k + 1]}
        pooled = pool_axis in (B.POOL_COLS, B.POOL_ROWS)
        su = None
        if pooled:
            d = B._layer_dims(x, z, params, mask_idx, hw)
            T = d.h if pool_axis == B.POOL_COLS else d.w
            su = torch.empty((d.B, T, d.E), dtype=torch.float32, device=x.device)
        out = B.SSMCall(x, z, params, pool_axis, mask_idx=mask_idx, hw=hw, flags=flags, ln=ln, conv=conv,
                        saved_u=su, pool_scale=pool_scale).run()
        ctx.meta = meta
        ctx.save_for_backward(x, z, *tensors, *(() if su is None else (su,)))
        ctx.has_su = su is not None
        return out

    @staticmethod
    def backward(ctx, dout):
        (pool_axis, mask_idx, hw, flags, ln_eps, pool_scale, has_ln, has_conv) = ctx.meta
        saved = ctx.saved_tensors
        x, z = saved[0], saved[1]
        tensors = saved[2:-1] if ctx.has_su else saved[2:]
        su = saved[-1] if ctx.has_su else None
        params = {d: dict(zip(B.DIR_FIELDS, tensors[5 * i:5 * i + 5])) for i, d in enumerate(DIRS)}
        k = 10
        ln = conv = None
        if has_ln:
            ln = {"weight": tensors[k], "bias": tensors[k + 1], "eps": ln_eps}
            k += 2
        if has_conv:
            conv = {"weight": tensors[k], "bias": tensors[k + 1]}
        res = B.BwdCall(x, z, dout.contiguous(), params, pool_axis, mask_idx=mask_idx, hw=hw,
                        flags=flags & ~(B.FLAG_STAGED | B.FLAG_FUSED), saved_u=su, ln=ln, pool_scale=pool_scale,
                        conv=conv).run()
        grads = [res[d][f] for d in DIRS for f in B.DIR_FIELDS]
        if has_ln:
            grads += [res["ln"]["weight"], res["ln"]["bias"]]
        if has_conv:
            grads += [res["conv"]["weight"], res["conv"]["bias"]]
        return (None, res["dx"], res["dz"], *grads)


def pooled_ssm(x: torch.Tensor, z: torch.Tensor, params: Dict[str, Dict[str, torch.Tensor]], pool_axis: int,
               mask_idx: Optional[torch.Tensor] = None, hw: Optional[Tuple[int, int]] = None, flags: int = 0,
               ln: Optional[Dict[str, object]] = None, conv: Optional[Dict[str, torch.Tensor]] = None,
               pool_scale: Optional[float] = None) -> torch.Tensor:
    """The layer with autograd: arguments as SSMCall (fp32 parameters; x, z
    fp32 or bf16, contiguous).  With FLAG_LOCAL_BWD the backward set needs
    only D; its other four entries, if given, get zero gradients."""
    if pool_axis not in (B.POOL_COLS, B.POOL_ROWS):
        raise ValueError("the backward pass covers pooled layers (POOL_COLS or POOL_ROWS)")
    tensors = []
    for d in DIRS:
        for f in B.DIR_FIELDS:
            t = params[d].get(f)
            if t is None:  # FLAG_LOCAL_BWD: the forward set stands in (never read by the library)
                t = params["fwd"][f].detach()
            tensors.append(t)
    if ln is not None:
        tensors += [ln["weight"], ln["bias"]]
    if conv is not None:
        tensors += [conv["weight"], conv["bias"]]
    meta = (pool_axis, mask_idx, hw, flags, float(ln["eps"]) if ln is not None else 0.0, pool_scale,
            ln is not None, conv is not None)
    return _PooledSSM.apply(meta, x, z, *tensors)
