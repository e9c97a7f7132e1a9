"""fp64 CPU oracle of FastVim's pooled bidirectional selective-scan layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
The arithmetic lives in ``fastvim_oracle.c`` (plain C, fp64, sequential loops);
this module only marshals numpy arrays into it.

Every function takes fp32 numpy arrays (bf16 data is passed as its exact fp32
widening) and returns fp64 numpy arrays.  See the C file's header for the
passages each stage follows and the readings it takes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fastvim_oracle.c")
_LIB = os.path.join(_HERE, "libfastvim_oracle.so")

COLS, ROWS, NONE_ROWMAJOR, NONE_COLMAJOR = 0, 1, 2, 3

class _Dir(ctypes.Structure):
    _fields_ = [
        ("x_proj_w", ctypes.c_void_p),
        ("dt_proj_w", ctypes.c_void_p),
        ("dt_proj_b", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p),
        ("D", ctypes.c_void_p),
    ]


class _DirOut(ctypes.Structure):
    _fields_ = [("v", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("s", ctypes.c_void_p)]


class _DirGrad(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")]


class _BwdStages(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("gs", "du", "dv_f", "dv_b")]

PARAM_NAMES = ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle C source with gcc into a shared library."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", src, "-o", tmp, "-lm"]
        )
        os.replace(tmp, out)
    return out


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """The oracle's entry points bound to one build of the C library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.fvo_max_threads.restype = ci
        lib.fvo_set_threads.argtypes = [ci]
        lib.fvo_set_threads.restype = None
        lib.fvo_pool_dense.argtypes = [vp, i64, i64, i64, i64, ci, vp]
        lib.fvo_pool_dense.restype = ci
        lib.fvo_mask_rows.argtypes = [vp, i64, i64, i64, i64, ci, vp]
        lib.fvo_mask_rows.restype = ci
        lib.fvo_pool_masked.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp]
        lib.fvo_pool_masked.restype = ci
        lib.fvo_xproj.argtypes = [vp, i64, i64, vp, i64, vp]
        lib.fvo_xproj.restype = None
        lib.fvo_delta.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp]
        lib.fvo_delta.restype = None
        lib.fvo_scan.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, ci, vp, vp]
        lib.fvo_scan.restype = None
        lib.fvo_layer.argtypes = [
            vp, vp, ctypes.POINTER(_Dir), ctypes.POINTER(_Dir),
            i64, i64, i64, i64, i64, i64, i64, ci, vp,
            vp, vp, vp, ctypes.POINTER(_DirOut), ctypes.POINTER(_DirOut),
            vp, vp, ctypes.c_double, vp, vp, i64, i64, ctypes.c_double,
        ]
        lib.fvo_layer.restype = ci
        lib.fvo_conv_silu.argtypes = [vp, i64, i64, i64, i64, ci, vp, vp, i64, vp]
        lib.fvo_conv_silu.restype = ci
        lib.fvo_layer_bwd.argtypes = [
            vp, vp, vp, ctypes.POINTER(_Dir), ctypes.POINTER(_Dir),
            i64, i64, i64, i64, i64, i64, i64, ci, vp,
            vp, vp, ctypes.POINTER(_DirGrad), ctypes.POINTER(_DirGrad), ctypes.POINTER(_BwdStages),
            vp, vp, ctypes.c_double, vp, vp, ctypes.c_double, i64, vp, vp, i64, vp, vp,
        ]
        lib.fvo_layer_bwd.restype = ci
        self._lib = lib
        self.path = path

    def max_threads(self) -> int:
        """OpenMP threads the oracle's image-parallel loops use."""
        return int(self._lib.fvo_max_threads())

    def set_threads(self, n: int) -> None:
        """Threads for later calls (timing only: results do not depend on it)."""
        self._lib.fvo_set_threads(int(n))

    def pool_dense(self, x, axis):
        """u (B,T,E) from a dense grid x (B,h,w,E)."""
        x = _f32(x)
        B, h, w, E = x.shape
        T = {COLS: h, ROWS: w}.get(axis, h * w)
        u = np.empty((B, T, E), np.float64)
        rc = self._lib.fvo_pool_dense(_ptr(x), B, h, w, E, axis, _ptr(u))
        if rc:
            raise ValueError("fvo_pool_dense failed: %d" % rc)
        return u

    def mask_rows(self, idx, h, w, axis):
        """Scan row (COLS) or column (ROWS) of every kept token; raises on bad idx."""
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        B, K = idx.shape
        rows = np.empty((B, K), np.int32)
        rc = self._lib.fvo_mask_rows(_ptr(idx), B, K, h, w, axis, _ptr(rows))
        if rc:
            raise ValueError("fvo_mask_rows: invalid mask index (%d)" % rc)
        return rows

    def pool_masked(self, x, rows, T, P):
        x = _f32(x)
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        B, K, E = x.shape
        u = np.empty((B, T, E), np.float64)
        self._lib.fvo_pool_masked(_ptr(x), _ptr(rows), B, K, T, P, E, _ptr(u))
        return u

    def xproj(self, u, x_proj_w):
        """v (..., NX) = u (..., E) contracted with x_proj_w (NX, E)."""
        u = _f64(u)
        W = _f32(x_proj_w)
        NX, E = W.shape
        M = u.size // E
        v = np.empty(u.shape[:-1] + (NX,), np.float64)
        self._lib.fvo_xproj(_ptr(u), M, E, _ptr(W), NX, _ptr(v))
        return v

    def delta(self, v, R, dt_proj_w, dt_proj_b):
        v = _f64(v)
        Wdt = _f32(dt_proj_w)
        bdt = _f32(dt_proj_b)
        E = Wdt.shape[0]
        NX = v.shape[-1]
        M = v.size // NX
        out = np.empty(v.shape[:-1] + (E,), np.float64)
        self._lib.fvo_delta(_ptr(v), M, NX, R, _ptr(Wdt), _ptr(bdt), E, _ptr(out))
        return out

    def scan(self, u, dlt, v, A_log, R, reverse=False, reset=None):
        """s (B,T,E) of one scan direction from u, delta (B,T,E) and v (B,T,NX)."""
        u, dlt, v = _f64(u), _f64(dlt), _f64(v)
        A_log = _f32(A_log)
        B, T, E = u.shape
        N = A_log.shape[1]
        NX = v.shape[-1]
        rs = None
        if reset is not None:
            rs = np.ascontiguousarray(reset, dtype=np.uint8)
            assert rs.shape == (T,)
        s = np.empty((B, T, E), np.float64)
        self._lib.fvo_scan(_ptr(u), _ptr(dlt), _ptr(v), B, T, E, N, R, NX, _ptr(A_log),
                           1 if reverse else 0, _ptr(rs), _ptr(s))
        return s

    def conv_silu(self, x, axis, conv):
        """x_conv (B,h,w,E) fp64: the depthwise causal Conv1D (conv["weight"]
        (E, KC), oldest tap first; conv["bias"] (E,)) along the oriented grid's
        sequence, then SiLU."""
        x = _f32(x)
        Wc, bc = _f32(conv["weight"]), _f32(conv["bias"])
        B, h, w, E = x.shape
        xc = np.empty(x.shape, np.float64)
        rc = self._lib.fvo_conv_silu(_ptr(x), B, h, w, E, axis, _ptr(Wc), _ptr(bc), Wc.shape[1], _ptr(xc))
        if rc:
            raise ValueError("fvo_conv_silu failed: %d" % rc)
        return xc

    def layer(self, x, z, fwd, bwd, axis, idx=None, hw=None, stages=False, ln=None, conv=None, local_window=0,
              pool_scale=1.0):
        """Full layer.  Dense: x, z (B,h,w,E).  Masked: x, z (B,K,E), idx (B,K),
        hw=(h, w).  fwd / bwd: dicts with x_proj_w, dt_proj_w, dt_proj_b, A_log, D.
        ln: None, or {"weight": (E,), "bias": (E,), "eps": float} for the
        post-SSM LayerNorm before the gate.  conv: None, or {"weight": (E, KC),
        "bias": (E,)}: x is then the Conv1D's input and the layer runs on
        conv_silu(x) (masked: the conv along the kept tokens k = 0..K-1).  local_window = L > 0: LBMamba's
        local backward scan (forward parameters, state reset at the top of
        every window of L steps) replaces the global backward scan; of bwd only
        D is used.  pool_scale multiplies the pooled tokens u (not the skip).
        Returns out (fp64), or with stages=True a dict of out, u, rows and the
        per-direction v, delta, s."""
        x, z = _f32(x), _f32(z)
        conv_w = conv_b = None
        conv_k = 0
        if conv is not None:
            conv_w, conv_b = _f32(conv["weight"]), _f32(conv["bias"])
            conv_k = conv_w.shape[1]
        ln_w = ln_b = None
        ln_eps = 0.0
        if ln is not None:
            ln_w, ln_b, ln_eps = _f32(ln["weight"]), _f32(ln["bias"]), float(ln["eps"])
        keep = []
        pf, pb = _dir_struct(fwd, keep), _dir_struct(bwd, keep)
        NX, E = keep[0].shape
        N = keep[3].shape[1]
        R = NX - 2 * N
        if idx is None:
            B, h, w, _ = x.shape
            K = 0
            idx_a = None
        else:
            B, K, _ = x.shape
            h, w = hw
            idx_a = np.ascontiguousarray(idx, dtype=np.int32)
            assert idx_a.shape == (B, K)
        T = {COLS: h, ROWS: w}.get(axis, h * w)
        out = np.empty(x.shape, np.float64)
        st = {}
        u = rows = None
        fo = bo = None
        if stages:
            u = np.empty((B, T, E), np.float64)
            rows = np.empty((B, K), np.int32) if idx is not None else None
            for name in ("fwd", "bwd"):
                st[name] = {
                    "v": np.empty((B, T, NX), np.float64),
                    "delta": np.empty((B, T, E), np.float64),
                    "s": np.empty((B, T, E), np.float64),
                }
            fo = _DirOut(*[st["fwd"][k].ctypes.data for k in ("v", "delta", "s")])
            bo = _DirOut(*[st["bwd"][k].ctypes.data for k in ("v", "delta", "s")])
        rc = self._lib.fvo_layer(
            _ptr(x), _ptr(z), ctypes.byref(pf), ctypes.byref(pb),
            B, h, w, E, N, R, K, axis, _ptr(idx_a),
            _ptr(out), _ptr(u), _ptr(rows),
            ctypes.byref(fo) if fo is not None else None,
            ctypes.byref(bo) if bo is not None else None,
            _ptr(ln_w), _ptr(ln_b), ln_eps, _ptr(conv_w), _ptr(conv_b), conv_k, int(local_window),
            float(pool_scale),
        )
        if rc:
            raise ValueError("fvo_layer failed: %d" % rc)
        if not stages:
            return out
        return {"out": out, "u": u, "rows": rows, "fwd": st["fwd"], "bwd": st["bwd"]}

    def layer_bwd(self, x, z, dout, fwd, bwd, axis, idx=None, hw=None, stages=False, ln=None, pool_scale=1.0,
                  local_window=0, conv=None):
        """Gradients of sum(dout * layer(x, z, ...)).  Arguments as layer();
        dout is shaped like x.  Returns a dict with dx, dz (fp64, shaped like
        x) and "fwd" / "bwd" dicts of parameter gradients keyed like the
        parameters; with ln (as in layer()) also "ln": {"weight", "bias"}, the
        LayerNorm's gradients; with stages=True also gs (dL/ds, which is dL/dy
        of the LayerNorm's input when ln is given), du (B,T,E) and dv_fwd,
        dv_bwd (B,T,NX).  local_window, pool_scale: as in layer(); with the local
        backward scan the shared parameters' gradients are in "fwd" and the
        backward set's x_proj_w, dt_proj_w, dt_proj_b and A_log gradients
        are zero.  conv (dense layers): as in layer(); dx is then the gradient
        of the Conv1D's input and "conv": {"weight", "bias"} holds the conv's
        gradients."""
        x, z, dout = _f32(x), _f32(z), _f32(dout)
        conv_w = conv_b = dcw = dcb = None
        conv_k = 0
        if conv is not None:
            conv_w, conv_b = _f32(conv["weight"]), _f32(conv["bias"])
            conv_k = conv_w.shape[1]
        ln_w = ln_b = dln_w = dln_b = None
        ln_eps = 0.0
        if ln is not None:
            ln_w, ln_b, ln_eps = _f32(ln["weight"]), _f32(ln["bias"]), float(ln["eps"])
        assert dout.shape == x.shape
        keep = []
        pf, pb = _dir_struct(fwd, keep), _dir_struct(bwd, keep)
        NX, E = keep[0].shape
        N = keep[3].shape[1]
        R = NX - 2 * N
        if idx is None:
            B, h, w, _ = x.shape
            K = 0
            idx_a = None
        else:
            B, K, _ = x.shape
            h, w = hw
            idx_a = np.ascontiguousarray(idx, dtype=np.int32)
            assert idx_a.shape == (B, K)
        T = {COLS: h, ROWS: w}.get(axis, h * w)
        dx = np.empty(x.shape, np.float64)
        dz = np.empty(x.shape, np.float64)
        grads = {}
        structs = []
        for name, p in (("fwd", fwd), ("bwd", bwd)):
            grads[name] = {k: np.empty(np.shape(p[k]), np.float64) for k in PARAM_NAMES}
            structs.append(_DirGrad(*[grads[name][k].ctypes.data for k in PARAM_NAMES]))
        st = None
        res = {"dx": dx, "dz": dz, "fwd": grads["fwd"], "bwd": grads["bwd"]}
        if ln is not None:
            dln_w, dln_b = np.empty(E, np.float64), np.empty(E, np.float64)
            res["ln"] = {"weight": dln_w, "bias": dln_b}
        if conv is not None:
            dcw, dcb = np.empty((E, conv_k), np.float64), np.empty(E, np.float64)
            res["conv"] = {"weight": dcw, "bias": dcb}
        if stages:
            res["gs"] = np.empty((B, T, E), np.float64)
            res["du"] = np.empty((B, T, E), np.float64)
            res["dv_fwd"] = np.empty((B, T, NX), np.float64)
            res["dv_bwd"] = np.empty((B, T, NX), np.float64)
            st = _BwdStages(*[res[k].ctypes.data for k in ("gs", "du", "dv_fwd", "dv_bwd")])
        rc = self._lib.fvo_layer_bwd(
            _ptr(x), _ptr(z), _ptr(dout), ctypes.byref(pf), ctypes.byref(pb),
            B, h, w, E, N, R, K, axis, _ptr(idx_a), _ptr(dx), _ptr(dz),
            ctypes.byref(structs[0]), ctypes.byref(structs[1]),
            ctypes.byref(st) if st is not None else None,
            _ptr(ln_w), _ptr(ln_b), ln_eps, _ptr(dln_w), _ptr(dln_b), float(pool_scale), int(local_window),
            _ptr(conv_w), _ptr(conv_b), conv_k, _ptr(dcw), _ptr(dcb),
        )
        if rc:
            raise ValueError("fvo_layer_bwd failed: %d" % rc)
        return res


def _dir_struct(p, keep):
    arrs = [_f32(p[k]) for k in ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")]
    keep.extend(arrs)
    return _Dir(*[a.ctypes.data for a in arrs])


_lock = threading.Lock()
_default = None


def get() -> Oracle:
    """The oracle bound to ``oracle/libfastvim_oracle.so`` (built if absent)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB):
                build(force=True)
            _default = Oracle(_LIB)
    return _default


def max_threads():
    return get().max_threads()


def set_threads(n):
    get().set_threads(n)


def pool_dense(x, axis):
    return get().pool_dense(x, axis)


def mask_rows(idx, h, w, axis):
    return get().mask_rows(idx, h, w, axis)


def pool_masked(x, rows, T, P):
    return get().pool_masked(x, rows, T, P)


def xproj(u, x_proj_w):
    return get().xproj(u, x_proj_w)


def delta(v, R, dt_proj_w, dt_proj_b):
    return get().delta(v, R, dt_proj_w, dt_proj_b)


def scan(u, dlt, v, A_log, R, reverse=False, reset=None):
    return get().scan(u, dlt, v, A_log, R, reverse=reverse, reset=reset)


def layer(x, z, fwd, bwd, axis, idx=None, hw=None, stages=False, ln=None, conv=None, local_window=0,
          pool_scale=1.0):
    return get().layer(x, z, fwd, bwd, axis, idx=idx, hw=hw, stages=stages, ln=ln, conv=conv,
                       local_window=local_window, pool_scale=pool_scale)


def conv_silu(x, axis, conv):
    return get().conv_silu(x, axis, conv)


def layer_bwd(x, z, dout, fwd, bwd, axis, idx=None, hw=None, stages=False, ln=None, pool_scale=1.0,
              local_window=0, conv=None):
    return get().layer_bwd(x, z, dout, fwd, bwd, axis, idx=idx, hw=hw, stages=stages, ln=ln,
                           pool_scale=pool_scale, local_window=local_window, conv=conv)
