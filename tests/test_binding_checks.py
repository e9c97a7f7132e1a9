"""The Python binding rejects bad tensors before anything reaches the
library: a tensor off the GPU (its host pointer would be read as device
memory), a non-contiguous view (the kernels assume dense rows), and a wrong
dtype or shape of any argument, parameter, gradient or option tensor (the
kernels would read or write out of bounds).  CPU tensors stand in for device
tensors, so every check runs without a GPU: shape checks come first, the
device check last.
"""
import numpy as np
import pytest
import torch

import pooled_selective_state_amd as P

B, H, W, E, N, R = 2, 4, 5, 16, 16, 4


def _params(E=E, R=R, N=N):
    def one():
        return {"x_proj_w": torch.zeros(R + 2 * N, E), "dt_proj_w": torch.zeros(E, R), "dt_proj_b": torch.zeros(E),
                "A_log": torch.zeros(E, N), "D": torch.zeros(E)}
    return {"fwd": one(), "bwd": one()}


def _xz(dtype=torch.float32):
    return torch.zeros(B, H, W, E, dtype=dtype), torch.zeros(B, H, W, E, dtype=dtype)


def _fwd(**kw):
    x, z = _xz()
    args = dict(x=x, z=z, params=_params(), pool_axis=P.POOL_COLS)
    args.update(kw)
    return P.SSMCall(**args)


def _bwd(**kw):
    x, z = _xz()
    args = dict(x=x, z=z, dout=torch.zeros_like(x), params=_params(), pool_axis=P.POOL_COLS)
    args.update(kw)
    return P.BwdCall(**args)


def test_cpu_tensors_rejected():
    with pytest.raises(ValueError, match="GPU"):
        _fwd()
    with pytest.raises(ValueError, match="GPU"):
        _bwd()


@pytest.mark.parametrize("d", ["fwd", "bwd"])
@pytest.mark.parametrize("f,shape", [("x_proj_w", (R + 2 * N, E + 4)), ("dt_proj_w", (E, R + 1)),
                                     ("dt_proj_b", (E + 4,)), ("A_log", (E, N + 1)), ("D", (E - 4,))])
def test_parameter_shapes(d, f, shape):
    prm = _params()
    prm[d][f] = torch.zeros(shape)
    with pytest.raises(ValueError, match="shape|rows"):
        _fwd(params=prm)


def test_parameter_dtype_and_layout():
    prm = _params()
    prm["bwd"]["D"] = torch.zeros(E, dtype=torch.float64)
    with pytest.raises(ValueError, match="float32"):
        _fwd(params=prm)
    prm = _params()
    prm["fwd"]["A_log"] = torch.zeros(N, E).t()  # the right shape, transposed strides
    with pytest.raises(ValueError, match="contiguous"):
        _fwd(params=prm)


def test_io_tensors():
    x, z = _xz()
    with pytest.raises(ValueError, match="z"):
        _fwd(z=z[:, :3])
    with pytest.raises(ValueError, match="z"):
        _fwd(z=z.to(torch.bfloat16))
    xt = torch.zeros(B, W, H, E).transpose(1, 2)  # the next block's grid as a view
    with pytest.raises(ValueError, match="contiguous"):
        _fwd(x=xt, z=xt.contiguous())
    with pytest.raises(ValueError, match="out"):
        _fwd(out=torch.zeros(B, H, W, E, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        _fwd(out=torch.zeros(B, H, W + 1, E))
    with pytest.raises(TypeError):
        _fwd(x=np.zeros((B, H, W, E), np.float32))


def test_option_tensors():
    with pytest.raises(ValueError, match="ln"):
        _fwd(ln={"weight": torch.zeros(E + 4), "bias": torch.zeros(E), "eps": 1e-5})
    with pytest.raises(ValueError, match="conv"):
        _fwd(conv={"weight": torch.zeros(E, 3), "bias": torch.zeros(E)})
    with pytest.raises(ValueError, match="saved_u"):
        _fwd(saved_u=torch.zeros(B, W, E))  # COLS scans H rows
    with pytest.raises(ValueError, match="workspace"):
        _fwd(workspace="elsewhere")


def test_masked_index_tensor():
    x = torch.zeros(B, 7, E)
    with pytest.raises(ValueError, match="mask_idx"):
        P.SSMCall(x, x.clone(), _params(), P.POOL_COLS, mask_idx=torch.zeros(B, 7, dtype=torch.int64), hw=(H, W))
    with pytest.raises(ValueError, match="mask_idx"):
        P.SSMCall(x, x.clone(), _params(), P.POOL_COLS, mask_idx=torch.zeros(B, 6, dtype=torch.int32), hw=(H, W))


def test_backward_tensors():
    x, _ = _xz()
    with pytest.raises(ValueError, match="dout"):
        _bwd(dout=torch.zeros(B, H, W, E + 4))
    with pytest.raises(ValueError, match="dx"):
        _bwd(dx=torch.zeros(B, H, W, E, dtype=torch.bfloat16))
    grads = {d: {f: torch.zeros_like(t) for f, t in _params()[d].items()} for d in ("fwd", "bwd")}
    grads["bwd"]["dt_proj_w"] = torch.zeros(E, R + 2)
    with pytest.raises(ValueError, match="grads.bwd.dt_proj_w"):
        _bwd(grads=grads)
    grads = {d: {f: torch.zeros_like(t) for f, t in _params()[d].items()} for d in ("fwd", "bwd")}
    grads["ln"] = {"weight": torch.zeros(E), "bias": torch.zeros(E + 1)}
    with pytest.raises(ValueError, match="grads.ln.bias"):
        _bwd(grads=grads, ln={"weight": torch.zeros(E), "bias": torch.zeros(E), "eps": 1e-5})
