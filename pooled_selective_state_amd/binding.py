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
# FLAG_CHECK_IDX: record invalid mask indices for fastvim_get_device_error
FLAG_CHECK_IDX = 64
# params.tuning: single-launch lags (bits 0-7 LS, 8-15 LE; 0 = automatic) and
# TUNING_POLL1 (every wait gives up after one poll: tests of the give-up path)
TUNING_POLL1 = 1 << 16
# bits 20-25: image groups of the backward call (0 = automatic, 1 = none, at most 32)
MAX_BWD_GROUPS = 32


def tuning_bwd_groups(n: int) -> int:
    return (int(n) & 0x3F) << 20


def tuning_lags(ls: int = 0, le: int = 0) -> int:
    return (int(ls) & 0xFF) | ((int(le) & 0xFF) << 8)


# bits 26-27: the scan and output stages of short pooled stage-kernel layers
# as one launch (0 = automatic, 1 = two launches, 2 = one launch)
SCAN_OUT_AUTO, SCAN_OUT_TWO, SCAN_OUT_ONE = 0, 1, 2


def tuning_scan_out(n: int) -> int:
    return (int(n) & 0x3) << 26


# workspace=NO_WORKSPACE: pass a NULL workspace, so the library takes its
# scratch from the stream-ordered allocator on the call's stream
NO_WORKSPACE = "stream-ordered"

STATUS = {
    0: "FASTVIM_OK", -1: "FASTVIM_ERR_NULL", -2: "FASTVIM_ERR_DIMS", -3: "FASTVIM_ERR_UNSUPPORTED",
    -4: "FASTVIM_ERR_ALIGN", -5: "FASTVIM_ERR_OVERLAP", -6: "FASTVIM_ERR_WORKSPACE", -7: "FASTVIM_ERR_HIP",
    -8: "FASTVIM_ERR_ARG", -9: "FASTVIM_ERR_BAD_INDEX", -10: "FASTVIM_ERR_DEVICE_WAIT", -11: "FASTVIM_ERR_SCRATCH",
}

# fastvim_ssm_fwd_noalloc's fixed scratch buffer (one per GPU, inside the library)
NOALLOC_SCRATCH_BYTES = 96 << 20

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
                ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32), ("tuning", ctypes.c_uint32),
                ("ln_weight", ctypes.c_void_p), ("ln_bias", ctypes.c_void_p), ("ln_eps", ctypes.c_float),
                ("pool_scale", ctypes.c_float), ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
                ("saved_u", ctypes.c_void_p)]


class DirGrads(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in DIR_FIELDS]


class Grads(ctypes.Structure):
    _fields_ = [("fwd", DirGrads), ("bwd", DirGrads), ("ln_weight", ctypes.c_void_p), ("ln_bias", ctypes.c_void_p),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p)]


EXPORTED_SYMBOLS = (
    "fastvim_ssm_workspace_bytes", "fastvim_ssm_fwd", "fastvim_ssm_fwd_stages", "fastvim_ssm_fwd_noalloc",
    "fastvim_get_device_error",
    "fastvim_ssm_stage", "fastvim_ssm_export", "fastvim_ssm_export_bytes", "fastvim_ssm_bwd_workspace_bytes",
    "fastvim_ssm_bwd", "fastvim_calib_copy", "fastvim_status_string", "fastvim_abi_version",
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
            L.fastvim_ssm_fwd_stages.argtypes = [vp, vp, PP, PD, ci, vp, vp, vp, vp, vp, vp, vp]
            L.fastvim_ssm_fwd_stages.restype = ci
            L.fastvim_ssm_fwd_noalloc.argtypes = [vp, vp, PP, PD, ci, vp, vp, vp]
            L.fastvim_ssm_fwd_noalloc.restype = ci
            L.fastvim_get_device_error.argtypes = [PP, vp]
            L.fastvim_get_device_error.restype = ci
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


def _side_stream(stream):
    """The torch stream a call runs on when it is not the current one, else
    None (then tensors the binding allocated need no record_stream)."""
    if stream is None:
        return None
    if not hasattr(stream, "cuda_stream"):
        stream = torch.cuda.ExternalStream(int(stream))
    return None if stream.cuda_stream == torch.cuda.current_stream().cuda_stream else stream


def _check_tensor(name: str, t, dtype, shape) -> None:
    """dtype, shape and contiguity of one argument (the device is checked
    for all arguments together, by _check_devices)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_devices(x: torch.Tensor, named) -> None:
    """Every tensor on the GPU, on x's device: the library dereferences the
    pointers as device memory of the stream's device."""
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor (the layer runs in HIP kernels), got device %s" % x.device)
    for name, t in named:
        if t is not None and t.device != x.device:
            raise ValueError("%s must be on %s like x, got %s" % (name, x.device, t.device))


def _layer_dims(x, z, params, mask_idx, hw) -> Dims:
    """Sizes of a call, after checking x, z, mask_idx and every parameter's
    dtype, shape and contiguity (x_proj_w (R+2N, E), dt_proj_w (E, R),
    dt_proj_b (E,), A_log (E, N), D (E,))."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    io = _io_dtype(x)
    _check_tensor("x", x, None, None)
    _check_tensor("z", z, x.dtype, x.shape)
    E = x.shape[-1]
    pf = params["fwd"]
    for f in ("x_proj_w", "A_log"):
        _check_tensor("fwd." + f, pf.get(f), torch.float32, None)
        if pf[f].dim() != 2:
            raise ValueError("fwd.%s must be 2-D" % f)
    NX = pf["x_proj_w"].shape[0]
    N = pf["A_log"].shape[1]
    R = NX - 2 * N
    if R < 1:
        raise ValueError("x_proj_w must have R + 2N rows with R >= 1 (N = %d from A_log), got %d" % (N, NX))
    shapes = {"x_proj_w": (NX, E), "dt_proj_w": (E, R), "dt_proj_b": (E,), "A_log": (E, N), "D": (E,)}
    for d in ("fwd", "bwd"):
        for f in DIR_FIELDS:
            t = params[d].get(f)
            if t is None and d == "bwd" and f != "D":
                continue  # FLAG_LOCAL_BWD reads only D of the backward set; the library checks the rest
            _check_tensor("%s.%s" % (d, f), t, torch.float32, shapes[f])
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
        _check_tensor("mask_idx", mask_idx, torch.int32, (B, K))
    return make_dims(B, h, w, E, N, R, K, io)


def _param_tensors(params):
    return [("%s.%s" % (d, f), params[d].get(f)) for d in ("fwd", "bwd") for f in DIR_FIELDS]


def _scan_len(dims: Dims, pool_axis: int) -> int:
    return {POOL_COLS: dims.h, POOL_ROWS: dims.w}.get(pool_axis, dims.h * dims.w)


def _dir_params(params, keep):
    """DirParams of both directions (checked by _layer_dims); a parameter that
    is absent or None is passed as NULL (FASTVIM_FLAG_LOCAL_BWD reads only D
    of the backward set)."""
    dirs = []
    for name in ("fwd", "bwd"):
        p = params[name]
        ptrs = []
        for f in DIR_FIELDS:
            t = p.get(f)
            if t is not None:
                keep.append(t)
            ptrs.append(_ptr(t))
        dirs.append(DirParams(*ptrs))
    return dirs


def _check_saved_u(t: Optional[torch.Tensor], dims: Dims, pool_axis: int) -> None:
    if t is not None:
        _check_tensor("saved_u", t, torch.float32, (dims.B, _scan_len(dims, pool_axis), dims.E))


def _check_ln(ln, E):
    if ln is not None:
        for f in ("weight", "bias"):
            _check_tensor("ln." + f, ln[f], torch.float32, (E,))


def _check_conv(conv, E):
    if conv is not None:
        _check_tensor("conv.weight", conv["weight"], torch.float32, (E, CONV_TAPS))
        _check_tensor("conv.bias", conv["bias"], torch.float32, (E,))


def _check_workspace_kind(workspace) -> None:
    if isinstance(workspace, str) and workspace != NO_WORKSPACE:
        raise ValueError("workspace must be a tensor, None or NO_WORKSPACE")
    if workspace is not None and not isinstance(workspace, (str, torch.Tensor)):
        raise TypeError("workspace must be a tensor, None or NO_WORKSPACE")


def _workspace_arg(workspace, nbytes: int, device):
    """(tensor or None, pointer, bytes) of the workspace argument: a tensor
    (contiguous, on device), NO_WORKSPACE (NULL: stream-ordered scratch), or
    None (a new torch tensor of nbytes)."""
    if isinstance(workspace, str):
        if workspace != NO_WORKSPACE:
            raise ValueError("workspace must be a tensor, None or NO_WORKSPACE")
        return None, None, 0
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    _check_tensor("workspace", workspace, None, None)
    if workspace.device != device:
        raise ValueError("workspace must be on %s like x, got %s" % (device, workspace.device))
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def check_device_error(params: "Params", stream=None) -> None:
    """fastvim_get_device_error for the last call that used this workspace:
    raises FastVimError on a device-side error (waits for the stream)."""
    st = lib().fastvim_get_device_error(ctypes.byref(params), _stream(stream))
    if st:
        raise FastVimError(st, "fastvim_get_device_error")


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
    multiply the pooled tokens by this factor (FLAG_POOL_SCALE).  workspace:
    a device tensor, None (allocated here), or NO_WORKSPACE (the library
    allocates and frees it on the call's stream; no exports then).  tuning:
    the params.tuning word.  Every tensor must be contiguous and on x's GPU
    (ValueError otherwise, before anything runs)."""

    def __init__(self, x: torch.Tensor, z: torch.Tensor, params: Dict[str, Dict[str, torch.Tensor]],
                 pool_axis: int, mask_idx: Optional[torch.Tensor] = None, hw: Optional[Tuple[int, int]] = None,
                 out: Optional[torch.Tensor] = None, workspace=None,
                 flags: int = 0, ln: Optional[Dict[str, object]] = None,
                 conv: Optional[Dict[str, torch.Tensor]] = None, saved_u: Optional[torch.Tensor] = None,
                 pool_scale: Optional[float] = None, tuning: int = 0):
        self.dims = _layer_dims(x, z, params, mask_idx, hw)
        E = self.dims.E
        if out is not None:
            _check_tensor("out", out, x.dtype, x.shape)
        _check_ln(ln, E)
        _check_conv(conv, E)
        _check_saved_u(saved_u, self.dims, pool_axis)
        _check_workspace_kind(workspace)
        _check_devices(x, [("z", z), ("mask_idx", mask_idx), ("out", out), ("saved_u", saved_u)]
                       + _param_tensors(params)
                       + ([("ln.weight", ln["weight"]), ("ln.bias", ln["bias"])] if ln is not None else [])
                       + ([("conv.weight", conv["weight"]), ("conv.bias", conv["bias"])] if conv is not None
                          else []))
        self.pool_axis = pool_axis
        self.x, self.z, self.mask_idx = x, z, mask_idx
        self.out = torch.empty_like(x) if out is None else out
        self._owned = [] if out is not None else [self.out]  # tensors this call allocated
        self._keep = []
        dirs = _dir_params(params, self._keep)
        ws_given = workspace is not None
        self.workspace, ws_ptr, ws_bytes = _workspace_arg(workspace, workspace_bytes(self.dims, pool_axis),
                                                          x.device)
        if not ws_given:
            self._owned.append(self.workspace)
        ln_w = ln_b = None
        ln_eps = 0.0
        if ln is not None:
            ln_w, ln_b, ln_eps = ln["weight"], ln["bias"], float(ln["eps"])
            self._keep.extend([ln_w, ln_b])
            flags |= FLAG_POST_NORM
        conv_w = conv_b = None
        if conv is not None:
            conv_w, conv_b = conv["weight"], conv["bias"]
            self._keep.extend([conv_w, conv_b])
            flags |= FLAG_CONV
        self.saved_u = saved_u
        if pool_scale is not None:
            flags |= FLAG_POOL_SCALE
        self.params = Params(dirs[0], dirs[1], ws_ptr, ws_bytes, flags, tuning, _ptr(ln_w), _ptr(ln_b), ln_eps,
                             1.0 if pool_scale is None else float(pool_scale), _ptr(conv_w), _ptr(conv_b),
                             _ptr(saved_u))

    def _args(self):
        return (_ptr(self.x), _ptr(self.z), ctypes.byref(self.params), ctypes.byref(self.dims), self.pool_axis,
                _ptr(self.mask_idx), _ptr(self.out))

    def _after(self, stream, check_device: bool) -> None:
        side = _side_stream(stream)
        if side is not None:  # the caching allocator must not reuse them before the side stream is done
            for t in self._owned:
                t.record_stream(side)
        if check_device:
            self.check_device(stream)

    def run(self, stream=None, check_device: bool = False) -> torch.Tensor:
        """Enqueue the layer; with check_device, also wait for it and raise on
        a device-side error (fastvim_get_device_error)."""
        st = lib().fastvim_ssm_fwd(*self._args(), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_fwd")
        self._after(stream, check_device)
        return self.out

    def run_noalloc(self, stream=None) -> torch.Tensor:
        """The layer through fastvim_ssm_fwd_noalloc: scratch from the
        library's fixed per-GPU buffer, nothing allocated (construct the call
        with workspace=NO_WORKSPACE and an out tensor to allocate nothing
        here either).  Calls that overlap on one GPU race."""
        st = lib().fastvim_ssm_fwd_noalloc(*self._args(), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_fwd_noalloc")
        self._after(stream, False)
        return self.out

    def run_stages(self, stream=None, u: bool = True, s: bool = True, rows: bool = True) -> Dict[str, torch.Tensor]:
        """The layer through fastvim_ssm_fwd_stages: returns out and, in new
        tensors, the pooled tokens u (pooled layers), both scan outputs s_fwd,
        s_bwd and the mask rows (masked layers), as asked."""
        d = self.dims
        T = _scan_len(d, self.pool_axis)
        dev = self.x.device
        pooled = self.pool_axis in (POOL_COLS, POOL_ROWS)
        res = {"out": self.out}
        if u and pooled:
            res["u"] = torch.empty((d.B, T, d.E), dtype=torch.float32, device=dev)
        if s:
            res["s_fwd"] = torch.empty((d.B, T, d.E), dtype=torch.float32, device=dev)
            res["s_bwd"] = torch.empty((d.B, T, d.E), dtype=torch.float32, device=dev)
        if rows and d.K > 0:
            res["rows"] = torch.empty((d.B, d.K), dtype=torch.int32, device=dev)
        st = lib().fastvim_ssm_fwd_stages(*self._args(), _stream(stream), _ptr(res.get("u")), _ptr(res.get("s_fwd")),
                                          _ptr(res.get("s_bwd")), _ptr(res.get("rows")))
        if st:
            raise FastVimError(st, "fastvim_ssm_fwd_stages")
        side = _side_stream(stream)
        if side is not None:
            for k, t in res.items():
                if k != "out":
                    t.record_stream(side)
        self._after(stream, False)
        return res

    def check_device(self, stream=None) -> None:
        """Raise FastVimError if the last run found an error on the device
        (waits for the stream)."""
        check_device_error(self.params, stream)

    def stage(self, stage: int, stream=None) -> None:
        st = lib().fastvim_ssm_stage(stage, *self._args(), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_stage(%d)" % stage)

    def export(self, what: int, stream=None) -> torch.Tensor:
        """Copy of an intermediate of the last run (U, XDBL, S_FWD, S_BWD: fp32; ROWS, BAD_TOKENS: int32)."""
        n = int(lib().fastvim_ssm_export_bytes(ctypes.byref(self.dims), self.pool_axis, what))
        d = self.dims
        T = _scan_len(d, self.pool_axis)
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
        side = _side_stream(stream)
        if side is not None:
            dst.record_stream(side)
        return dst


def ssm_fwd(x, z, params, pool_axis=POOL_COLS, mask_idx=None, hw=None, out=None, workspace=None, stream=None,
            flags=0, ln=None, conv=None, saved_u=None, pool_scale=None, check_device=False):
    """The pooled bidirectional selective-scan layer; returns out."""
    return SSMCall(x, z, params, pool_axis, mask_idx=mask_idx, hw=hw, out=out, workspace=workspace,
                   flags=flags, ln=ln, conv=conv, saved_u=saved_u, pool_scale=pool_scale).run(stream, check_device)


def ssm_fwd_stages(x, z, params, pool_axis=POOL_COLS, mask_idx=None, hw=None, out=None, workspace=None,
                   stream=None, flags=0, ln=None, conv=None, saved_u=None, pool_scale=None):
    """The layer and its intermediates in one call (fastvim_ssm_fwd_stages):
    {"out", "u" (pooled), "s_fwd", "s_bwd", "rows" (masked)}."""
    return SSMCall(x, z, params, pool_axis, mask_idx=mask_idx, hw=hw, out=out, workspace=workspace,
                   flags=flags, ln=ln, conv=conv, saved_u=saved_u, pool_scale=pool_scale).run_stages(stream)


class BwdCall:
    """One prepared backward call (gradients of sum(dout * out)).

    Arguments as SSMCall, plus dout shaped like x.  dx, dz (like x) and the
    gradients grads = {"fwd": {...}, "bwd": {...}} (fp32, shaped like the
    parameters; with ln also "ln": {"weight", "bias"}) are allocated unless
    given.  ln: the post-SSM LayerNorm of the forward call.  saved_u: the
    pooled tokens a forward call with the same x wrote (then x is read once,
    not twice).  pool_scale: as for the forward call.  groups: the call's
    image groups (0: the library's choice, 1: none; see fastvim_ssm_bwd in
    fastvim.h).  run() returns
    {"dx": dx, "dz": dz, "fwd": {...}, "bwd": {...}}, with ln also
    "ln": {"weight": ..., "bias": ...} and with conv "conv": {"weight": ...,
    "bias": ...}."""

    def __init__(self, x: torch.Tensor, z: torch.Tensor, dout: torch.Tensor,
                 params: Dict[str, Dict[str, torch.Tensor]], pool_axis: int,
                 mask_idx: Optional[torch.Tensor] = None, hw: Optional[Tuple[int, int]] = None,
                 dx: Optional[torch.Tensor] = None, dz: Optional[torch.Tensor] = None,
                 grads: Optional[Dict[str, Dict[str, torch.Tensor]]] = None,
                 workspace=None, flags: int = 0,
                 saved_u: Optional[torch.Tensor] = None, ln: Optional[Dict[str, object]] = None,
                 pool_scale: Optional[float] = None, conv: Optional[Dict[str, torch.Tensor]] = None,
                 groups: int = 0):
        self.dims = _layer_dims(x, z, params, mask_idx, hw)
        E = self.dims.E
        if not (isinstance(groups, int) and 0 <= groups <= MAX_BWD_GROUPS):
            raise ValueError("groups must be an int in [0, %d] (0: automatic)" % MAX_BWD_GROUPS)
        _check_tensor("dout", dout, x.dtype, x.shape)
        for name, t in (("dx", dx), ("dz", dz)):
            if t is not None:
                _check_tensor(name, t, x.dtype, x.shape)
        _check_ln(ln, E)
        _check_conv(conv, E)
        _check_saved_u(saved_u, self.dims, pool_axis)
        _check_workspace_kind(workspace)
        self.pool_axis = pool_axis
        self.x, self.z, self.dout, self.mask_idx = x, z, dout, mask_idx
        self._owned = []
        self.dx = torch.empty_like(x) if dx is None else dx
        self.dz = torch.empty_like(x) if dz is None else dz
        self._owned += [t for t, given in ((self.dx, dx), (self.dz, dz)) if given is None]
        self._keep = []
        dirs = _dir_params(params, self._keep)
        # gradients are shaped like the forward set (the backward set may lack
        # all but D with FLAG_LOCAL_BWD)
        if grads is None:
            grads = {d: {f: torch.empty_like(params["fwd"][f]) for f in DIR_FIELDS} for d in ("fwd", "bwd")}
            self._owned += [grads[d][f] for d in ("fwd", "bwd") for f in DIR_FIELDS]
        ln_w = ln_b = None
        ln_eps = 0.0
        if ln is not None:
            ln_w, ln_b, ln_eps = ln["weight"], ln["bias"], float(ln["eps"])
            self._keep.extend([ln_w, ln_b])
            flags |= FLAG_POST_NORM
            if "ln" not in grads:
                grads = dict(grads, ln={"weight": torch.empty_like(ln_w), "bias": torch.empty_like(ln_b)})
                self._owned += [grads["ln"]["weight"], grads["ln"]["bias"]]
            for f in ("weight", "bias"):
                _check_tensor("grads.ln." + f, grads["ln"][f], torch.float32, (E,))
        gd = []
        for d in ("fwd", "bwd"):
            for f in DIR_FIELDS:
                _check_tensor("grads.%s.%s" % (d, f), grads[d][f], torch.float32, params["fwd"][f].shape)
            gd.append(DirGrads(*[grads[d][f].data_ptr() for f in DIR_FIELDS]))
        conv_w = conv_b = None
        if conv is not None:
            conv_w, conv_b = conv["weight"], conv["bias"]
            self._keep.extend([conv_w, conv_b])
            flags |= FLAG_CONV
            if "conv" not in grads:
                grads = dict(grads, conv={"weight": torch.empty_like(conv_w), "bias": torch.empty_like(conv_b)})
                self._owned += [grads["conv"]["weight"], grads["conv"]["bias"]]
            _check_tensor("grads.conv.weight", grads["conv"]["weight"], torch.float32, (E, CONV_TAPS))
            _check_tensor("grads.conv.bias", grads["conv"]["bias"], torch.float32, (E,))
        self.grads = grads
        lg = grads["ln"] if ln is not None else None
        cg = grads["conv"] if conv is not None else None
        named = [("z", z), ("dout", dout), ("mask_idx", mask_idx), ("dx", self.dx), ("dz", self.dz),
                 ("saved_u", saved_u)] + _param_tensors(params)
        named += [("grads.%s.%s" % (d, f), grads[d][f]) for d in ("fwd", "bwd") for f in DIR_FIELDS]
        if ln is not None:
            named += [("ln.weight", ln_w), ("ln.bias", ln_b), ("grads.ln.weight", lg["weight"]),
                      ("grads.ln.bias", lg["bias"])]
        if conv is not None:
            named += [("conv.weight", conv_w), ("conv.bias", conv_b), ("grads.conv.weight", cg["weight"]),
                      ("grads.conv.bias", cg["bias"])]
        _check_devices(x, named)
        self.cgrads = Grads(gd[0], gd[1], _ptr(lg["weight"]) if lg else None, _ptr(lg["bias"]) if lg else None,
                            _ptr(cg["weight"]) if cg else None, _ptr(cg["bias"]) if cg else None)
        ws_given = workspace is not None
        self.workspace, ws_ptr, ws_bytes = _workspace_arg(workspace, bwd_workspace_bytes(self.dims, pool_axis),
                                                          x.device)
        if not ws_given:
            self._owned.append(self.workspace)
        self.saved_u = saved_u
        if pool_scale is not None:
            flags |= FLAG_POOL_SCALE
        self.params = Params(dirs[0], dirs[1], ws_ptr, ws_bytes, flags, tuning_bwd_groups(groups), _ptr(ln_w),
                             _ptr(ln_b), ln_eps,
                             1.0 if pool_scale is None else float(pool_scale), _ptr(conv_w), _ptr(conv_b),
                             _ptr(saved_u))

    def run(self, stream=None, check_device: bool = False) -> Dict[str, object]:
        st = lib().fastvim_ssm_bwd(_ptr(self.x), _ptr(self.z), _ptr(self.dout), ctypes.byref(self.params),
                                   ctypes.byref(self.dims), self.pool_axis, _ptr(self.mask_idx), _ptr(self.dx),
                                   _ptr(self.dz), ctypes.byref(self.cgrads), _stream(stream))
        if st:
            raise FastVimError(st, "fastvim_ssm_bwd")
        side = _side_stream(stream)
        if side is not None:
            for t in self._owned:
                if t is not None:
                    t.record_stream(side)
        if check_device:
            check_device_error(self.params, stream)
        res = {"dx": self.dx, "dz": self.dz, "fwd": self.grads["fwd"], "bwd": self.grads["bwd"]}
        if "ln" in self.grads and self.params.flags & FLAG_POST_NORM:
            res["ln"] = self.grads["ln"]
        if "conv" in self.grads and self.params.flags & FLAG_CONV:
            res["conv"] = self.grads["conv"]
        return res


def ssm_bwd(x, z, dout, params, pool_axis=POOL_COLS, mask_idx=None, hw=None, workspace=None, stream=None,
            flags=0, saved_u=None, ln=None, pool_scale=None, conv=None, check_device=False, groups=0):
    """Gradients of the layer; returns {"dx", "dz", "fwd": {...}, "bwd": {...}} (and "ln" / "conv" with those)."""
    return BwdCall(x, z, dout, params, pool_axis, mask_idx=mask_idx, hw=hw, workspace=workspace,
                   flags=flags, saved_u=saved_u, ln=ln, pool_scale=pool_scale, conv=conv,
                   groups=groups).run(stream, check_device)


def calib_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Streaming copy of src into dst (same byte size) by the library's
    calibration kernel; a measurement aid, not part of the layer."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("calib_copy needs contiguous tensors of equal byte size")
    st = lib().fastvim_calib_copy(_ptr(dst), _ptr(src), n, _stream(stream))
    if st:
        raise FastVimError(st, "fastvim_calib_copy")
