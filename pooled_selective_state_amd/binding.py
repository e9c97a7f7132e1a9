"""ctypes binding of ``libfastvim.so`` (declared in ``include/fastvim.h``).

Argument marshalling only: torch provides device memory and the current HIP
stream, every step of the layer runs in the library's HIP kernels.  There is
no fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfastvim.so")

# fastvim_pool_axis
POOL_COLS, POOL_ROWS, POOL_NONE_ROWMAJOR, POOL_NONE_COLMAJOR = 0, 1, 2, 3
# fastvim_dtype
F32, BF16 = 0, 1
# fastvim_stage
STAGE_ROWS, STAGE_POOL, STAGE_PROJ, STAGE_SCAN, STAGE_EPILOGUE = 0, 1, 2, 3, 4
# fastvim_export
EXPORT_U, EXPORT_XDBL, EXPORT_S_FWD, EXPORT_S_BWD, EXPORT_ROWS, EXPORT_BAD_TOKENS, EXPORT_STATUS = 0, 1, 2, 3, 4, 5, 6
# params.flags: FLAG_STAGED runs every layer as its stage kernels, FLAG_FUSED
# every dense pooled layer as the single pipelined launch; by default the
# library picks by size
FLAG_STAGED, FLAG_FUSED = 1, 2
# FLAG_POST_NORM: post-SSM LayerNorm between the skip and the gate
FLAG_POST_NORM = 4
FLAG_CONV = 8
CONV_TAPS = 4
FLAG_LOCAL_BWD = 16
LOCAL_WINDOW = 16
# FLAG_POOL_SCALE: the pooled tokens times params.pool_scale (0.25 in the MAE transfer recipe)
FLAG_POOL_SCALE = 32

STATUS = {
    0: "FASTVIM_OK", -1: "FASTVIM_ERR_NULL", -2: "FASTVIM_ERR_DIMS", -3: "FASTVIM_ERR_UNSUPPORTED",
    -4: "FASTVIM_ERR_ALIGN", -5: "FASTVIM_ERR_OVERLAP", -6: "FASTVIM_ERR_WORKSPACE", -7: "FASTVIM_ERR_HIP",
    -8: "FASTVIM_ERR_ARG",
}

DIR_FIELDS = ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")


class FastVimError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().fastvim_status_string(status).decode()
        super().__init__("%s: %s (%d, %s)" % (where, msg, status, STATUS.get(status, "?")))


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64), ("E", ctypes.c_int64),
                ("N", ctypes.c_int64), ("R", ctypes.c_int64), ("K", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class DirParams(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in DIR_FIELDS]


class Params(ctypes.Structure):
    _fields_ = [("fwd", DirParams), ("bwd", DirParams), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("ln_weight", ctypes.c_void_p), ("ln_bias", ctypes.c_void_p), ("ln_eps", ctypes.c_float),
                ("pool_scale", ctypes.c_float), ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
                ("saved_u", ctypes.c_void_p)]


class DirGrads(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in DIR_FIELDS]


class Grads(ctypes.Structure):
    _fields_ = [("fwd", DirGrads), ("bwd", DirGrads), ("ln_weight", ctypes.c_void_p), ("ln_bias", ctypes.c_void_p),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p)]


EXPORTED_SYMBOLS = (
    "fastvim_ssm_workspace_bytes", "fastvim_ssm_fwd", "fastvim_ssm_stage", "fastvim_ssm_export",
    "fastvim_ssm_export_bytes", "fastvim_ssm_bwd_workspace_bytes", "fastvim_ssm_bwd", "fastvim_calib_copy",
    "fastvim_status_string", "fastvim_abi_version",
)

_lock = threading.Lock()
_lib = None


def lib():
    """Load ``libfastvim.so`` (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libfastvim.so is not built; run `python -m pooled_selective_state_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            PD, PP = ctypes.POINTER(Dims), ctypes.POINTER(Params)
            L.fastvim_ssm_workspace_bytes.argtypes = [PD, ci]
            L.fastvim_ssm_workspace_bytes.restype = sz
            L.fastvim_ssm_fwd.argtypes = [vp, vp, PP, PD, ci, vp, vp, vp]
            L.fastvim_ssm_fwd.restype = ci
            L.fastvim_ssm_stage.argtypes = [ci, vp, vp, PP, PD, ci, vp, vp, vp]
            L.fastvim_ssm_stage.restype = ci
            L.fastvim_ssm_export.argtypes = [PP, PD, ci, ci, vp, sz, vp]
            L.fastvim_ssm_export.restype = ci
            L.fastvim_ssm_export_bytes.argtypes = [PD, ci, ci]
            L.fastvim_ssm_export_bytes.restype = sz
            L.fastvim_ssm_bwd_workspace_bytes.argtypes = [PD, ci]
            L.fastvim_ssm_bwd_workspace_bytes.restype = sz
            L.fastvim_ssm_bwd.argtypes = [vp, vp, vp, PP, PD, ci, vp, vp, vp, ctypes.POINTER(Grads), vp]
            L.fastvim_ssm_bwd.restype = ci
            L.fastvim_calib_copy.argtypes = [vp, vp, sz, vp]
            L.fastvim_calib_copy.restype = ci
            L.fastvim_status_string.argtypes = [ci]
            L.fastvim_status_string.restype = ctypes.c_char_p
            L.fastvim_abi_version.argtypes = []
            L.fastvim_abi_version.restype = ci
            _lib = L
    return _lib


def make_dims(B, h, w, E, N=16, R=12, K=0, io_dtype=F32) -> Dims:
    return Dims(B, h, w, E, N, R, K, io_dtype, 0)


def workspace_bytes(dims: Dims, pool_axis: int) -> int:
    return int(lib().fastvim_ssm_workspace_bytes(ctypes.byref(dims), pool_axis))


def bwd_workspace_bytes(dims: Dims, pool_axis: int) -> int:
    return int(lib().fastvim_ssm_bwd_workspace_bytes(ctypes.byref(dims), pool_axis))


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("x, z must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _layer_dims(x, z, params, mask_idx, hw) -> Dims:
    io = _io_dtype(x)
    if z.dtype != x.dtype or z.shape != x.shape:
        raise ValueError("z must match x in shape and dtype")
    E = x.shape[-1]
    pf = params["fwd"]
    NX = pf["x_proj_w"].shape[0]
    N = pf["A_log"].shape[1]
    R = NX - 2 * N
    if mask_idx is None:
        if x.dim() != 4:
            raise ValueError("dense x must be (B, h, w, E)")
        B, h, w, _ = x.shape
        K = 0
    else:
        if x.dim() != 3 or hw is None:
            raise ValueError("masked x must be (B, K, E) with hw=(h, w)")
        B, K, _ = x.shape
        h, w = hw
        if mask_idx.dtype != torch.int32 or tuple(mask_idx.shape) != (B, K):
            raise ValueError("mask_idx must be int32 (B, K)")
    return make_dims(B, h, w, E, N, R, K, io)


def _dir_params(params, keep):
    """DirParams of both directions; a parameter that is absent or None is
    passed as NULL (FASTVIM_FLAG_LOCAL_BWD reads only D of the backward set)."""
    dirs = []
    for name in ("fwd", "bwd"):
        p = params[name]
        ptrs = []
        for f in DIR_FIELDS:
            t = p.get(f)
            if t is None:
                ptrs.append(None)
                continue
            if t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("parameter %s.%s must be contiguous float32" % (name, f))
            keep.append(t)
            ptrs.append(t.data_ptr())
        dirs.append(DirParams(*ptrs))
    return dirs


def _check_saved_u(t: Optional[torch.Tensor]) -> None:
    if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
        raise ValueError("saved_u must be a contiguous float32 tensor (B, T, E)")


class SSMCall:
    """One prepared layer call: sizes, parameter pointers, workspace and out.

    Dense: x, z (B, h, w, E).  Masked: x, z (B, K, E), mask_idx (B, K) int32
    and hw = (h, w).  params = {"fwd": {...}, "bwd": {...}} holding fp32
    device tensors x_proj_w (R+2N, E), dt_proj_w (E, R), dt_proj_b (E),
    A_log (E, N), D (E).  ln = {"weight": (E,), "bias": (E,), "eps": float}
    (fp32 device tensors) adds the post-SSM LayerNorm before the gate.
    conv = {"weight": (E, 4), "bias": (E,)} (fp32 device tensors) makes x the
    input of the producer Conv1D + SiLU, computed inside the layer.
    saved_u (B, T, E) fp32 (pooled layers) receives the pooled tokens, for a
    later backward call given the same tensor.  pool_scale (pooled layers):
    multiply the pooled tokens by this factor (FLAG_POOL_SCALE)."""

    def __init__(self, x: torch.Tensor, z: torch.Tensor, params: Dict[str, Dict[str, torch.Tensor]],
                 pool_axis: int, mask_idx: Optional[torch.Tensor] = None, hw: Optional[Tuple[int, int]] = None,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 flags: int = 0, ln: Optional[Dict[str, object]] = None,
                 conv: Optional[Dict[str, torch.Tensor]] = None, saved_u: Optional[torch.Tensor] = None,
                 pool_scale: Optional[float] = None):
        self.dims = _layer_dims(x, z, params, mask_idx, hw)
        self.pool_axis = pool_axis
        self.x, self.z, self.mask_idx = x, z, mask_idx
        self.out = torch.empty_like(x) if out is None else out
        self._keep = []
        dirs = _dir_params(params, self._keep)
        nbytes = workspace_bytes(self.dims, pool_axis)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
        self.workspace = workspace
        ln_w = ln_b = None
        ln_eps = 0.0
        if ln is not None:
            ln_w, ln_b, ln_eps = ln["weight"], ln["bias"], float(ln["eps"])
            for t in (ln_w, ln_b):
                if t.dtype != torch.float32 or not t.is_contiguous():
                    raise ValueError("LayerNorm weight and bias must be contiguous float32")
            self._keep.extend([ln_w, ln_b])
            flags |= FLAG_POST_NORM
        conv_w = conv_b = None
        if conv is not None:
            conv_w, conv_b = conv["weight"], conv["bias"]
            for t in (conv_w, conv_b):
                if t.dtype != torch.float32 or not t.is_contiguous():
                    raise ValueError("Conv1D weight and bias must be contiguous float32")
            self._keep.extend([conv_w, conv_b])
            flags |= FLAG_CONV
        _check_saved_u(saved_u)
        self.saved_u = saved_u
        if pool_scale is not None:
            flags |= FLAG_POOL_SCALE
        self.params = Params(dirs[0], dirs[1], workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             flags, 0, _ptr(ln_w), _ptr(ln_b), ln_eps,
                             1.0 if pool_scale is None else float(pool_scale), _ptr(conv_w), _ptr(conv_b),
                             _ptr(saved_u))

    def _args(self):
        return (_ptr(self.x), _ptr(self.z), ctypes.byref(self.params), ctypes.byref(self.dims), self.pool_axis,
                _ptr(self.mask_idx), _ptr(self.out))

    def run(self, stream=None) -> torch.Tensor:
        st = lib().fastvim_ssm_fwd(*self._args(), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_fwd")
        return self.out

    def stage(self, stage: int, stream=None) -> None:
        st = lib().fastvim_ssm_stage(stage, *self._args(), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_stage(%d)" % stage)

    def export(self, what: int, stream=None) -> torch.Tensor:
        """Copy of an intermediate of the last run (U, XDBL, S_FWD, S_BWD: fp32; ROWS, BAD_TOKENS: int32)."""
        n = int(lib().fastvim_ssm_export_bytes(ctypes.byref(self.dims), self.pool_axis, what))
        d = self.dims
        T = {POOL_COLS: d.h, POOL_ROWS: d.w}.get(self.pool_axis, d.h * d.w)
        shapes = {
            EXPORT_U: (d.B, T, d.E), EXPORT_XDBL: (d.B, T, 2, d.R + 2 * d.N), EXPORT_S_FWD: (d.B, T, d.E),
            EXPORT_S_BWD: (d.B, T, d.E), EXPORT_ROWS: (d.B, d.K), EXPORT_BAD_TOKENS: (d.B,), EXPORT_STATUS: (1,),
        }
        dtype = torch.int32 if what in (EXPORT_ROWS, EXPORT_BAD_TOKENS, EXPORT_STATUS) else torch.float32
        dst = torch.empty(shapes[what], dtype=dtype, device=self.x.device)
        st = lib().fastvim_ssm_export(ctypes.byref(self.params), ctypes.byref(self.dims), self.pool_axis, what,
                                      _ptr(dst), max(n, dst.numel() * dst.element_size()), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_export(%d)" % what)
        return dst


def ssm_fwd(x, z, params, pool_axis=POOL_COLS, mask_idx=None, hw=None, out=None, workspace=None, stream=None,
            flags=0, ln=None, conv=None, saved_u=None, pool_scale=None):
    """The pooled bidirectional selective-scan layer; returns out."""
    return SSMCall(x, z, params, pool_axis, mask_idx=mask_idx, hw=hw, out=out, workspace=workspace,
                   flags=flags, ln=ln, conv=conv, saved_u=saved_u, pool_scale=pool_scale).run(stream)


class BwdCall:
    """One prepared backward call (gradients of sum(dout * out)).

    Arguments as SSMCall, plus dout shaped like x.  dx, dz (like x) and the
    gradients grads = {"fwd": {...}, "bwd": {...}} (fp32, shaped like the
    parameters; with ln also "ln": {"weight", "bias"}) are allocated unless
    given.  ln: the post-SSM LayerNorm of the forward call.  saved_u: the
    pooled tokens a forward call with the same x wrote (then x is read once,
    not twice).  pool_scale: as for the forward call.  run() returns
    {"dx": dx, "dz": dz, "fwd": {...}, "bwd": {...}} and, with ln,
    "ln": {"weight": ..., "bias": ...}."""

    def __init__(self, x: torch.Tensor, z: torch.Tensor, dout: torch.Tensor,
                 params: Dict[str, Dict[str, torch.Tensor]], pool_axis: int,
                 mask_idx: Optional[torch.Tensor] = None, hw: Optional[Tuple[int, int]] = None,
                 dx: Optional[torch.Tensor] = None, dz: Optional[torch.Tensor] = None,
                 grads: Optional[Dict[str, Dict[str, torch.Tensor]]] = None,
                 workspace: Optional[torch.Tensor] = None, flags: int = 0,
                 saved_u: Optional[torch.Tensor] = None, ln: Optional[Dict[str, object]] = None,
                 pool_scale: Optional[float] = None, conv: Optional[Dict[str, torch.Tensor]] = None):
        self.dims = _layer_dims(x, z, params, mask_idx, hw)
        if dout.dtype != x.dtype or dout.shape != x.shape:
            raise ValueError("dout must match x in shape and dtype")
        self.pool_axis = pool_axis
        self.x, self.z, self.dout, self.mask_idx = x, z, dout, mask_idx
        self.dx = torch.empty_like(x) if dx is None else dx
        self.dz = torch.empty_like(x) if dz is None else dz
        self._keep = []
        dirs = _dir_params(params, self._keep)
        # gradients are shaped like the forward set (the backward set may lack
        # all but D with FLAG_LOCAL_BWD)
        if grads is None:
            grads = {d: {f: torch.empty_like(params["fwd"][f]) for f in DIR_FIELDS} for d in ("fwd", "bwd")}
        ln_w = ln_b = None
        ln_eps = 0.0
        if ln is not None:
            ln_w, ln_b, ln_eps = ln["weight"], ln["bias"], float(ln["eps"])
            for t in (ln_w, ln_b):
                if t.dtype != torch.float32 or not t.is_contiguous():
                    raise ValueError("LayerNorm weight and bias must be contiguous float32")
            self._keep.extend([ln_w, ln_b])
            flags |= FLAG_POST_NORM
            if "ln" not in grads:
                grads = dict(grads, ln={"weight": torch.empty_like(ln_w), "bias": torch.empty_like(ln_b)})
            for f in ("weight", "bias"):
                t = grads["ln"][f]
                if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != ln_w.shape:
                    raise ValueError("LayerNorm gradient %s must be contiguous float32 shaped like the weight" % f)
        self.grads = grads
        gd = []
        for d in ("fwd", "bwd"):
            for f in DIR_FIELDS:
                t = grads[d][f]
                if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != params["fwd"][f].shape:
                    raise ValueError("gradient %s.%s must be contiguous float32 shaped like the parameter" % (d, f))
            gd.append(DirGrads(*[grads[d][f].data_ptr() for f in DIR_FIELDS]))
        conv_w = conv_b = None
        if conv is not None:
            conv_w, conv_b = conv["weight"], conv["bias"]
            for t in (conv_w, conv_b):
                if t.dtype != torch.float32 or not t.is_contiguous():
                    raise ValueError("Conv1D weight and bias must be contiguous float32")
            self._keep.extend([conv_w, conv_b])
            flags |= FLAG_CONV
            if "conv" not in grads:
                grads = dict(grads, conv={"weight": torch.empty_like(conv_w), "bias": torch.empty_like(conv_b)})
            for f, ref in (("weight", conv_w), ("bias", conv_b)):
                t = grads["conv"][f]
                if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != ref.shape:
                    raise ValueError("Conv1D gradient %s must be contiguous float32 shaped like the parameter" % f)
            self.grads = grads
        lg = grads["ln"] if ln is not None else None
        cg = grads["conv"] if conv is not None else None
        self.cgrads = Grads(gd[0], gd[1], _ptr(lg["weight"]) if lg else None, _ptr(lg["bias"]) if lg else None,
                            _ptr(cg["weight"]) if cg else None, _ptr(cg["bias"]) if cg else None)
        nbytes = bwd_workspace_bytes(self.dims, pool_axis)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
        self.workspace = workspace
        _check_saved_u(saved_u)
        self.saved_u = saved_u
        if pool_scale is not None:
            flags |= FLAG_POOL_SCALE
        self.params = Params(dirs[0], dirs[1], workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             flags, 0, _ptr(ln_w), _ptr(ln_b), ln_eps,
                             1.0 if pool_scale is None else float(pool_scale), _ptr(conv_w), _ptr(conv_b),
                             _ptr(saved_u))

    def run(self, stream=None) -> Dict[str, object]:
        st = lib().fastvim_ssm_bwd(_ptr(self.x), _ptr(self.z), _ptr(self.dout), ctypes.byref(self.params),
                                   ctypes.byref(self.dims), self.pool_axis, _ptr(self.mask_idx), _ptr(self.dx),
                                   _ptr(self.dz), ctypes.byref(self.cgrads), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_bwd")
        res = {"dx": self.dx, "dz": self.dz, "fwd": self.grads["fwd"], "bwd": self.grads["bwd"]}
        if "ln" in self.grads and self.params.flags & FLAG_POST_NORM:
            res["ln"] = self.grads["ln"]
        if "conv" in self.grads and self.params.flags & FLAG_CONV:
            res["conv"] = self.grads["conv"]
        return res


def ssm_bwd(x, z, dout, params, pool_axis=POOL_COLS, mask_idx=None, hw=None, workspace=None, stream=None,
            flags=0, saved_u=None, ln=None, pool_scale=None, conv=None):
    """Gradients of the layer; returns {"dx", "dz", "fwd": {...}, "bwd": {...}} (and "ln" / "conv" with those)."""
    return BwdCall(x, z, dout, params, pool_axis, mask_idx=mask_idx, hw=hw, workspace=workspace,
                   flags=flags, saved_u=saved_u, ln=ln, pool_scale=pool_scale, conv=conv).run(stream)


def calib_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Streaming copy of src into dst (same byte size) by the library's
    calibration kernel; a measurement aid, not part of the layer."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("calib_copy needs contiguous tensors of equal byte size")
    st = lib().fastvim_calib_copy(_ptr(dst), _ptr(src), n, _stream(stream))
    if st:
        raise FastVimError(st, "fastvim_calib_copy")
