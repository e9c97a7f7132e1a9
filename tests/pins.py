"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees with a closed form, an invariant, a library routine, a
brute-force evaluation on tiny inputs or the hand-worked golden example.  The
same checks run against mutated builds of the oracle (``test_oracle_mutants``)
to show that a plausible slip anywhere in it (a dropped term, a flipped sign,
a wrong index or a transposed operand) fails at least one of them.

Sources: the FastVim summary page (gptget.net, arXiv 2502.00594), sections
方法详解 and 术语表; the Pith review of 2502.00594 ("key_machinery", the
pooling-invariance falsifier); the SF-Mamba article (glsqs.com), section 二
(periodic state reset).
"""
from __future__ import annotations

import os

import numpy as np
from scipy.special import expit

COLS, ROWS, NONE_ROWMAJOR, NONE_COLMAJOR = 0, 1, 2, 3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TIGHT = 1e-12


def _close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    err = np.max(np.abs(a - b)) / scale if a.size else 0.0
    assert err <= tol, "%s: rel err %.3e > %.1e" % (what, err, tol)


def rand_dir(rng, E, N, R, scale=0.3):
    """A parameter set with every entry distinct and O(1) effects."""
    return {
        "x_proj_w": (scale * rng.standard_normal((R + 2 * N, E))).astype(np.float32),
        "dt_proj_w": (scale * rng.standard_normal((E, R))).astype(np.float32),
        "dt_proj_b": rng.uniform(-3.0, -0.5, E).astype(np.float32),
        "A_log": rng.uniform(-1.0, 1.5, (E, N)).astype(np.float32),
        "D": rng.uniform(0.5, 1.5, E).astype(np.float32),
    }


def silu(z):
    return np.asarray(z, np.float64) * expit(np.asarray(z, np.float64))


def softplus(q):
    return np.logaddexp(0.0, q)


# ---------------------------------------------------------------- brute force
def bf_direction(u, p, reverse):
    """s of one direction by the matrix (convolution) form of the SSM:
    s_t = sum_tau sum_n C_t[n] exp(A[e,n] * sum of delta strictly after tau up
    to t) delta_tau B_tau[n] u_tau  (forward; mirrored for the backward scan).
    Uses numpy for the contractions; no recurrence."""
    B_, T, E = u.shape
    Wx = p["x_proj_w"].astype(np.float64)
    N = p["A_log"].shape[1]
    R = Wx.shape[0] - 2 * N
    v = u @ Wx.T
    dl = softplus(v[..., :R] @ p["dt_proj_w"].astype(np.float64).T + p["dt_proj_b"].astype(np.float64))
    Bm, Cm = v[..., R:R + N], v[..., R + N:]
    A = -np.exp(p["A_log"].astype(np.float64))  # (E, N)
    s = np.zeros((B_, T, E))
    for b in range(B_):
        cum = np.concatenate([np.zeros((1, E)), np.cumsum(dl[b], axis=0)])  # cum[k] = sum_{<k}
        for t in range(T):
            taus = range(0, t + 1) if not reverse else range(t, T)
            for tau in taus:
                if not reverse:
                    span = cum[t + 1] - cum[tau + 1]  # sum_{k=tau+1..t}
                else:
                    span = cum[tau] - cum[t]  # sum_{k=t..tau-1}
                decay = np.exp(A * span[:, None])  # (E, N)
                s[b, t] += np.sum(Cm[b, t][None, :] * decay * (dl[b, tau] * u[b, tau])[:, None]
                                  * Bm[b, tau][None, :], axis=1)
    return s, v, dl


def bf_layer(x, z, pf, pb, axis, idx=None, hw=None):
    """Whole layer from scratch in numpy (means, permutations, matrix-form SSM)."""
    x = np.asarray(x, np.float64)
    z = np.asarray(z, np.float64)
    if idx is None:
        B_, h, w, E = x.shape
        if axis == COLS:
            u = x.mean(axis=2)
        elif axis == ROWS:
            u = x.mean(axis=1)
        elif axis == NONE_ROWMAJOR:
            u = x.reshape(B_, h * w, E)
        else:
            u = x.transpose(0, 2, 1, 3).reshape(B_, h * w, E)
    else:
        B_, K, E = x.shape
        h, w = hw
        T, P = (h, w) if axis == COLS else (w, h)
        u = np.zeros((B_, T, E))
        for b in range(B_):
            for k in range(K):
                i, j = divmod(int(idx[b, k]), w)
                u[b, i if axis == COLS else j] += x[b, k]
        u /= P
    sf, _, _ = bf_direction(u, pf, False)
    sb, _, _ = bf_direction(u, pb, True)
    s = sf + sb
    D = pf["D"].astype(np.float64) + pb["D"].astype(np.float64)
    if idx is None:
        if axis == COLS:
            rep = np.repeat(s[:, :, None, :], w, axis=2)
        elif axis == ROWS:
            rep = np.repeat(s[:, None, :, :], h, axis=1)
        elif axis == NONE_ROWMAJOR:
            rep = s.reshape(B_, h, w, E)
        else:
            rep = s.reshape(B_, w, h, E).transpose(0, 2, 1, 3)
    else:
        rep = np.zeros_like(x)
        for b in range(B_):
            for k in range(K):
                i, j = divmod(int(idx[b, k]), w)
                rep[b, k] = s[b, i if axis == COLS else j]
    return (rep + D * x) * silu(z), u, sf, sb


# ----------------------------------------------------------------------- pins
def pin_golden_worked_example(O):
    """Hand-derived T=3 example (exact multiples of ln 2)."""
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example_T3.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = np.array([float(t) for t in v.split()])
    L = np.log(2.0)
    x = vals["x"].astype(np.float32).reshape(1, 3, 2, 1)
    z = vals["z"].astype(np.float32).reshape(1, 3, 2, 1)

    def d(tag):
        return {
            "x_proj_w": vals[tag + ".x_proj_w"].astype(np.float32).reshape(5, 1),
            "dt_proj_w": vals["dt_proj_w"].astype(np.float32).reshape(1, 1),
            "dt_proj_b": vals["dt_proj_b"].astype(np.float32),
            "A_log": np.log(vals[tag + ".A_log_exp"]).astype(np.float32).reshape(1, 2),
            "D": vals[tag + ".D"].astype(np.float32),
        }

    r = O.layer(x, z, d("fwd"), d("bwd"), COLS, stages=True)
    # A_log is stored in fp32, so exp(delta * A) is exact only to fp32 rounding of log 2.
    _close(r["u"].ravel(), vals["u"], what="golden u")
    _close(r["fwd"]["delta"].ravel(), vals["delta_over_ln2"] * L, what="golden delta")
    _close(r["fwd"]["s"].ravel(), vals["s_fwd_over_ln2"] * L, tol=1e-7, what="golden s_fwd")
    _close(r["bwd"]["s"].ravel(), vals["s_bwd_over_ln2"] * L, tol=1e-7, what="golden s_bwd")
    _close(r["out"].ravel(), vals["out_ln2_coef"] * L + vals["out_const"], tol=1e-7, what="golden out")


def pin_geometric_series(O):
    """Inputs constant along every pooled and scanned position: the scan is a
    geometric series, s_t = sum_n C_n delta B_n c (1 - a_n^(t+1)) / (1 - a_n)."""
    rng = np.random.default_rng(11)
    B_, h, w, E, N, R = 2, 5, 3, 6, 4, 3
    c = rng.standard_normal((B_, E)).astype(np.float32)
    x = np.broadcast_to(c[:, None, None, :], (B_, h, w, E)).copy()
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    for axis, T in ((COLS, h), (ROWS, w), (NONE_ROWMAJOR, h * w)):
        r = O.layer(x, z, pf, pb, axis, stages=True)
        for name, p, rev in (("fwd", pf, False), ("bwd", pb, True)):
            cc = c.astype(np.float64)
            v = cc @ p["x_proj_w"].astype(np.float64).T  # (B, NX)
            dl = softplus(v[:, :R] @ p["dt_proj_w"].astype(np.float64).T + p["dt_proj_b"])  # (B,E)
            A = -np.exp(p["A_log"].astype(np.float64))
            a = np.exp(dl[:, :, None] * A[None])  # (B,E,N)
            Bn, Cn = v[:, R:R + N], v[:, R + N:]
            t = np.arange(T)
            k = (T - t) if rev else (t + 1)  # number of terms in the series
            series = (1 - a[:, None, :, :] ** k[None, :, None, None]) / (1 - a[:, None, :, :])
            coef = (Cn * Bn)[:, None, None, :] * (dl * cc)[:, None, :, None]
            expect = np.sum(coef * series, axis=-1)
            _close(r[name]["s"], expect, what="geometric series %s axis %d" % (name, axis))


def pin_delta_to_zero(O):
    """With the step size driven to ~1e-26 the scan contributes nothing and
    out = (D_fwd + D_bwd) * x * silu(z)."""
    rng = np.random.default_rng(12)
    B_, h, w, E, N, R = 2, 4, 5, 8, 4, 2
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    pf["dt_proj_b"][:] = -60.0
    pb["dt_proj_b"][:] = -60.0
    pf["dt_proj_w"][:] = 0.0
    pb["dt_proj_w"][:] = 0.0
    for axis in (COLS, ROWS, NONE_COLMAJOR):
        out = O.layer(x, z, pf, pb, axis)
        expect = (pf["D"].astype(np.float64) + pb["D"]) * x * silu(z)
        _close(out, expect, tol=1e-20 * 1e6, what="delta->0 axis %d" % axis)


def pin_flip(O):
    """The backward scan is the forward scan of the time-reversed sequence."""
    rng = np.random.default_rng(13)
    B_, T, E, N, R = 2, 9, 5, 4, 3
    u = rng.standard_normal((B_, T, E))
    dl = rng.uniform(0.01, 0.5, (B_, T, E))
    v = rng.standard_normal((B_, T, R + 2 * N))
    A_log = rng.uniform(-1, 1, (E, N)).astype(np.float32)
    sb = O.scan(u, dl, v, A_log, R, reverse=True)
    sf_flipped = O.scan(u[:, ::-1], dl[:, ::-1], v[:, ::-1], A_log, R, reverse=False)
    _close(sb, sf_flipped[:, ::-1], what="flip")
    # and the two directions genuinely differ on this input
    sf = O.scan(u, dl, v, A_log, R, reverse=False)
    assert np.max(np.abs(sf - sb)) > 1e-3


def pin_width_one_pooling(O):
    """Pooling over an axis of length 1 is the identity, so the pooled layer
    equals the unpooled layer (both raster orders) on that grid."""
    rng = np.random.default_rng(14)
    B_, h, E, N, R = 2, 7, 6, 4, 3
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, 1, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, 1, E)).astype(np.float32)
    ref = O.layer(x, z, pf, pb, NONE_ROWMAJOR)
    _close(O.layer(x, z, pf, pb, COLS), ref, what="w=1 COLS")
    _close(O.layer(x, z, pf, pb, NONE_COLMAJOR), ref, what="w=1 colmajor")
    xt, zt = x.transpose(0, 2, 1, 3).copy(), z.transpose(0, 2, 1, 3).copy()  # (B,1,h,E)
    _close(O.layer(xt, zt, pf, pb, ROWS), O.layer(xt, zt, pf, pb, NONE_ROWMAJOR), what="h=1 ROWS")


def pin_reset_equals_independent(O):
    """A scan over concatenated sequences with the decay forced to zero at each
    sequence start equals independent scans of the pieces."""
    rng = np.random.default_rng(15)
    E, N, R = 4, 3, 2
    lens = [3, 5, 1, 4]
    A_log = rng.uniform(-1, 1, (E, N)).astype(np.float32)
    pieces = [(rng.standard_normal((1, L, E)), rng.uniform(0.05, 0.6, (1, L, E)),
               rng.standard_normal((1, L, R + 2 * N))) for L in lens]
    u = np.concatenate([p[0] for p in pieces], axis=1)
    dl = np.concatenate([p[1] for p in pieces], axis=1)
    v = np.concatenate([p[2] for p in pieces], axis=1)
    reset = np.zeros(sum(lens), np.uint8)
    reset[np.cumsum([0] + lens[:-1])] = 1
    s = O.scan(u, dl, v, A_log, R, reverse=False, reset=reset)
    ind = np.concatenate([O.scan(p[0], p[1], p[2], A_log, R) for p in pieces], axis=1)
    _close(s, ind, what="reset")
    assert np.max(np.abs(O.scan(u, dl, v, A_log, R) - ind)) > 1e-4  # the reset matters


def pin_brute_force_layer(O):
    """Tiny layers against a from-scratch numpy evaluation (matrix-form SSM)."""
    rng = np.random.default_rng(16)
    B_, h, w, E, N, R = 2, 4, 3, 3, 4, 2
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    for axis in (COLS, ROWS, NONE_ROWMAJOR, NONE_COLMAJOR):
        r = O.layer(x, z, pf, pb, axis, stages=True)
        out, u, sf, sb = bf_layer(x, z, pf, pb, axis)
        _close(r["u"], u, what="bf u axis %d" % axis)
        _close(r["fwd"]["s"], sf, tol=1e-11, what="bf s_fwd axis %d" % axis)
        _close(r["bwd"]["s"], sb, tol=1e-11, what="bf s_bwd axis %d" % axis)
        _close(r["out"], out, tol=1e-11, what="bf out axis %d" % axis)
    K = 5
    idx = np.stack([rng.permutation(h * w)[:K] for _ in range(B_)]).astype(np.int32)
    xm = rng.standard_normal((B_, K, E)).astype(np.float32)
    zm = rng.standard_normal((B_, K, E)).astype(np.float32)
    for axis in (COLS, ROWS):
        r = O.layer(xm, zm, pf, pb, axis, idx=idx, hw=(h, w), stages=True)
        out, u, sf, sb = bf_layer(xm, zm, pf, pb, axis, idx=idx, hw=(h, w))
        _close(r["u"], u, what="bf masked u axis %d" % axis)
        _close(r["out"], out, tol=1e-11, what="bf masked out axis %d" % axis)


def pin_pooling_invariance(O):
    """Permuting the pooled positions within every scanned row (x and z alike)
    leaves the scan unchanged and permutes out the same way (the Pith review's
    falsifier: inputs equal after pooling give equal scan outputs)."""
    rng = np.random.default_rng(17)
    B_, h, w, E, N, R = 2, 4, 6, 5, 4, 2
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    r = O.layer(x, z, pf, pb, COLS, stages=True)
    perm = [rng.permutation(w) for _ in range(h)]
    xp = np.stack([x[:, i, perm[i]] for i in range(h)], axis=1)
    zp = np.stack([z[:, i, perm[i]] for i in range(h)], axis=1)
    rp = O.layer(xp, zp, pf, pb, COLS, stages=True)
    _close(rp["fwd"]["s"] + rp["bwd"]["s"], r["fwd"]["s"] + r["bwd"]["s"], tol=1e-13, what="perm s")
    _close(rp["out"], np.stack([r["out"][:, i, perm[i]] for i in range(h)], axis=1), tol=1e-13,
           what="perm out")


def pin_transpose(O):
    """ROWS pooling is COLS pooling on the transposed grid, and column-major
    unpooled order is row-major order on the transposed grid."""
    rng = np.random.default_rng(18)
    B_, h, w, E, N, R = 2, 3, 5, 4, 4, 2
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    xt, zt = x.transpose(0, 2, 1, 3).copy(), z.transpose(0, 2, 1, 3).copy()
    for a, b in ((ROWS, COLS), (NONE_COLMAJOR, NONE_ROWMAJOR)):
        _close(O.layer(x, z, pf, pb, a), O.layer(xt, zt, pf, pb, b).transpose(0, 2, 1, 3),
               what="transpose %d/%d" % (a, b))


def pin_masked_equals_zero_filled(O):
    """Masked pooling (sum of kept tokens / fixed P) equals dense pooling of the
    grid with the dropped tokens set to zero, at every kept position."""
    rng = np.random.default_rng(19)
    B_, h, w, E, N, R, K = 3, 5, 4, 6, 4, 3, 7
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    idx = np.stack([rng.permutation(h * w)[:K] for _ in range(B_)]).astype(np.int32)
    xm = rng.standard_normal((B_, K, E)).astype(np.float32)
    zm = rng.standard_normal((B_, K, E)).astype(np.float32)
    xf = np.zeros((B_, h * w, E), np.float32)
    zf = np.zeros((B_, h * w, E), np.float32)
    for b in range(B_):
        xf[b, idx[b]] = xm[b]
        zf[b, idx[b]] = zm[b]
    xf, zf = xf.reshape(B_, h, w, E), zf.reshape(B_, h, w, E)
    for axis in (COLS, ROWS):
        dense = O.layer(xf, zf, pf, pb, axis).reshape(B_, h * w, E)
        masked = O.layer(xm, zm, pf, pb, axis, idx=idx, hw=(h, w))
        _close(masked, np.stack([dense[b, idx[b]] for b in range(B_)]), what="zero-fill axis %d" % axis)


def pin_all_kept(O):
    """With every token kept (any order) the masked layer is the dense layer."""
    rng = np.random.default_rng(20)
    B_, h, w, E, N, R = 2, 4, 3, 5, 4, 2
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    idx = np.stack([rng.permutation(h * w) for _ in range(B_)]).astype(np.int32)
    xf, zf = x.reshape(B_, h * w, E), z.reshape(B_, h * w, E)
    xm = np.stack([xf[b, idx[b]] for b in range(B_)])
    zm = np.stack([zf[b, idx[b]] for b in range(B_)])
    ln = rand_ln(rng, E)
    for axis in (COLS, ROWS):
        for norm in (None, ln):
            dense = O.layer(x, z, pf, pb, axis, ln=norm).reshape(B_, h * w, E)
            masked = O.layer(xm, zm, pf, pb, axis, idx=idx, hw=(h, w), ln=norm)
            _close(masked, np.stack([dense[b, idx[b]] for b in range(B_)]),
                   what="all kept axis %d%s" % (axis, " with LayerNorm" if norm else ""))


def pin_zero_projection(O):
    """x_proj_w = 0 gives B = C = 0, so the scan output is exactly zero."""
    rng = np.random.default_rng(21)
    B_, h, w, E, N, R = 2, 3, 4, 5, 4, 2
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    pf["x_proj_w"][:] = 0
    pb["x_proj_w"][:] = 0
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    r = O.layer(x, z, pf, pb, COLS, stages=True)
    assert np.all(r["fwd"]["s"] == 0) and np.all(r["bwd"]["s"] == 0)
    _close(r["out"], (pf["D"].astype(np.float64) + pb["D"]) * x * silu(z), what="W_x=0")


def pin_linear_in_D(O):
    """out(D) - out(D=0) = (D_fwd + D_bwd) * x * silu(z)."""
    rng = np.random.default_rng(22)
    B_, h, w, E, N, R = 2, 4, 4, 6, 4, 3
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    f0, b0 = dict(pf), dict(pb)
    f0["D"] = np.zeros(E, np.float32)
    b0["D"] = np.zeros(E, np.float32)
    for axis in (COLS, ROWS):
        diff = O.layer(x, z, pf, pb, axis) - O.layer(x, z, f0, b0, axis)
        _close(diff, (pf["D"].astype(np.float64) + pb["D"]) * x * silu(z), tol=1e-12,
               what="linear in D axis %d" % axis)


def pin_library_routines(O):
    """Stages that are textbook operations equal numpy's: the mean over an
    axis, the x_proj contraction (matmul), softplus (logaddexp)."""
    rng = np.random.default_rng(23)
    x = rng.standard_normal((2, 5, 7, 8)).astype(np.float32)
    _close(O.pool_dense(x, COLS), x.astype(np.float64).mean(axis=2), tol=1e-15, what="mean cols")
    _close(O.pool_dense(x, ROWS), x.astype(np.float64).mean(axis=1), tol=1e-15, what="mean rows")
    u = rng.standard_normal((3, 4, 8))
    W = rng.standard_normal((11, 8)).astype(np.float32)
    _close(O.xproj(u, W), u @ W.astype(np.float64).T, tol=1e-14, what="xproj")
    v = rng.standard_normal((3, 4, 11)) * 4
    Wdt = rng.standard_normal((8, 3)).astype(np.float32)
    bdt = rng.standard_normal(8).astype(np.float32) * 10
    expect = softplus(v[..., :3] @ Wdt.astype(np.float64).T + bdt)
    _close(O.delta(v, 3, Wdt, bdt), expect, tol=1e-14, what="softplus")
    # softplus at large |q| (no overflow, no cancellation)
    big = np.array([[[60.0] + [0.0] * 10]])
    got = O.delta(big, 1, np.ones((1, 1), np.float32), np.zeros(1, np.float32))
    assert abs(got.item() - 60.0) < 1e-12
    got = O.delta(-big, 1, np.ones((1, 1), np.float32), np.zeros(1, np.float32))
    assert abs(got.item() / np.exp(-60.0) - 1.0) < 1e-12


def pin_mask_rows_exact(O):
    """Kept-token rows are idx div w (COLS) or idx mod w (ROWS), exactly; masked
    pooled sums of integer-valued tokens are exact integers."""
    rng = np.random.default_rng(24)
    B_, h, w, K, E = 4, 7, 5, 12, 3
    idx = np.stack([rng.permutation(h * w)[:K] for _ in range(B_)]).astype(np.int32)
    rc = O.mask_rows(idx, h, w, COLS)
    rr = O.mask_rows(idx, h, w, ROWS)
    assert np.array_equal(rc, idx // w) and np.array_equal(rr, idx % w)
    x = np.broadcast_to((np.arange(K, dtype=np.float32) + 1)[None, :, None], (B_, K, E)).copy()
    for rows, T, P in ((rc, h, w), (rr, w, h)):
        sums = np.zeros((B_, T, E))
        for b in range(B_):
            np.add.at(sums[b], rows[b], x[b].astype(np.float64))
        u = O.pool_masked(x, rows, T, P)
        assert np.array_equal(u * P, sums)
    for bad in ([0, h * w], [3, 3], [-1, 2]):
        try:
            O.mask_rows(np.array([bad], np.int32), h, w, COLS)
        except ValueError:
            continue
        raise AssertionError("invalid mask index %s accepted" % (bad,))


def rand_ln(rng, E, eps=1e-5):
    """Post-SSM LayerNorm parameters with every entry distinct."""
    return {"weight": rng.uniform(0.5, 1.5, E).astype(np.float32),
            "bias": rng.uniform(-0.5, 0.5, E).astype(np.float32), "eps": eps}


def _ln_case(rng, B_=2, h=5, w=4, E=7, N=4, R=3):
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    # the gate bounded away from zero, so the pre-gate value can be recovered
    z = (1.0 + np.abs(rng.standard_normal((B_, h, w, E)))).astype(np.float32)
    return pf, pb, x, z


def pin_layernorm_moments(O):
    """With unit scale and zero shift, every token's normalised output (the
    output divided by the gate) has mean 0 and mean square var / (var + eps),
    var being the variance of the same token's output without the norm."""
    rng = np.random.default_rng(25)
    pf, pb, x, z = _ln_case(rng)
    E = x.shape[-1]
    eps = 0.25  # large enough that a misplaced eps shows
    ln = {"weight": np.ones(E, np.float32), "bias": np.zeros(E, np.float32), "eps": eps}
    for axis in (COLS, ROWS, NONE_ROWMAJOR):
        g = silu(z)
        y = O.layer(x, z, pf, pb, axis) / g
        yn = O.layer(x, z, pf, pb, axis, ln=ln) / g
        var = y.var(axis=-1)
        assert float(np.abs(yn.mean(axis=-1)).max()) <= 1e-12, "LayerNorm mean not zero"
        _close((yn ** 2).mean(axis=-1), var / (var + eps), what="LayerNorm mean square")


def pin_layernorm_affine(O):
    """The norm's shift enters linearly and only through the gate:
    out(w, b) - out(w, 0) = b * silu(z); its scale multiplies the output."""
    rng = np.random.default_rng(26)
    pf, pb, x, z = _ln_case(rng)
    E = x.shape[-1]
    ln = rand_ln(rng, E)
    ln0 = dict(ln, bias=np.zeros(E, np.float32))
    ln2 = dict(ln0, weight=(2.0 * ln["weight"]).astype(np.float32))
    for axis in (COLS, ROWS):
        o1 = O.layer(x, z, pf, pb, axis, ln=ln)
        o0 = O.layer(x, z, pf, pb, axis, ln=ln0)
        o2 = O.layer(x, z, pf, pb, axis, ln=ln2)
        _close(o1 - o0, np.broadcast_to(ln["bias"].astype(np.float64), x.shape) * silu(z), what="LayerNorm shift")
        _close(o2, 2.0 * o0, what="LayerNorm scale")


def pin_layernorm_library(O):
    """The normalised output equals numpy's mean / var normalisation of the
    un-normalised output, scaled and shifted, then gated."""
    rng = np.random.default_rng(27)
    pf, pb, x, z = _ln_case(rng, E=9)
    E = x.shape[-1]
    ln = rand_ln(rng, E, eps=0.1)
    for axis in (COLS, NONE_COLMAJOR):
        g = silu(z)
        y = O.layer(x, z, pf, pb, axis) / g
        ref = ((y - y.mean(-1, keepdims=True)) / np.sqrt(y.var(-1, keepdims=True) + ln["eps"])
               * ln["weight"].astype(np.float64) + ln["bias"].astype(np.float64)) * g
        _close(O.layer(x, z, pf, pb, axis, ln=ln), ref, tol=1e-11, what="LayerNorm vs numpy")


# ---------------------------------------------------------------- backward pass
def _dyadic(a, step=2.0 ** -10, lim=3.9):
    """Values on a grid of 2^-10 inside (-4, 4): a perturbation by a multiple of
    2^-14 stays exactly representable in fp32, so finite differences of the
    oracle see exactly the perturbation they ask for."""
    return (np.round(np.clip(np.asarray(a, np.float64), -lim, lim) / step) * step).astype(np.float32)


def _bwd_case(rng, axis, masked, B_=2, h=4, w=3, E=5, N=3, R=2):
    pf = {k: _dyadic(v) for k, v in rand_dir(rng, E, N, R).items()}
    pb = {k: _dyadic(v) for k, v in rand_dir(rng, E, N, R).items()}
    if masked:
        K = 7
        idx = np.stack([rng.permutation(h * w)[:K] for _ in range(B_)]).astype(np.int32)
        shape = (B_, K, E)
    else:
        idx = None
        shape = (B_, h, w, E)
    x = _dyadic(rng.standard_normal(shape))
    z = _dyadic(rng.standard_normal(shape))
    dout = rng.standard_normal(shape).astype(np.float32)
    return pf, pb, x, z, dout, idx, (h, w)


def _loss(O, x, z, dout, pf, pb, axis, idx, hw, ln=None, pool_scale=1.0, local=0, conv=None):
    return float(np.sum(dout.astype(np.float64) * O.layer(x, z, pf, pb, axis, idx=idx, hw=hw, ln=ln,
                                                          pool_scale=pool_scale, local_window=local, conv=conv)))


def _perturbed(a, V, eps):
    out = (a.astype(np.float64) + eps * V).astype(np.float32)
    assert np.array_equal(out.astype(np.float64), a.astype(np.float64) + eps * V), "perturbation not exact"
    return out


def pin_bwd_finite_differences(O):
    """Every gradient of L = sum(dout * out) (x, z, and the five parameters of
    each direction) matches the central difference of the pinned forward
    oracle along a random +-1 direction.  Inputs sit on a dyadic grid, so the
    perturbed inputs are exact and the difference quotient carries only its
    O(eps^2) truncation error (~1e-9 relative at eps = 2^-14) and the fp64
    rounding of the two losses, at most a few ulps of sum |dout out| divided
    by 2 eps (which matters only for a gradient near zero); also with the
    pooled tokens scaled by 1/4, and with LBMamba's local backward scan
    (windows of 2, 3 and 5 steps, the last one partial; the backward set's
    unused parameters then have zero gradients)."""
    eps = 2.0 ** -14
    rng = np.random.default_rng(40)
    cases = ((COLS, False, 1.0, 0), (ROWS, False, 1.0, 0), (NONE_ROWMAJOR, False, 1.0, 0),
             (NONE_COLMAJOR, False, 1.0, 0), (COLS, True, 1.0, 0), (ROWS, True, 1.0, 0), (COLS, False, 0.25, 0),
             (ROWS, True, 0.25, 0), (COLS, False, 1.0, 3), (ROWS, True, 1.0, 2), (NONE_ROWMAJOR, False, 0.25, 5))
    for axis, masked, scale, local in cases:
        pf, pb, x, z, dout, idx, hw = _bwd_case(rng, axis, masked)
        g = O.layer_bwd(x, z, dout, pf, pb, axis, idx=idx, hw=hw, pool_scale=scale, local_window=local)
        out = O.layer(x, z, pf, pb, axis, idx=idx, hw=hw, pool_scale=scale, local_window=local)
        floor = 64 * 2.0 ** -52 * float(np.sum(np.abs(dout * out))) / (2.0 * eps)
        targets = [("x", None), ("z", None)] + [(d, k) for d in ("fwd", "bwd") for k in
                                                 ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")]
        for d, k in targets:
            if k is None:
                base = x if d == "x" else z
                grad = g["dx"] if d == "x" else g["dz"]
            else:
                base = (pf if d == "fwd" else pb)[k]
                grad = g[d][k]
            V = rng.choice([-1.0, 1.0], size=base.shape)
            L = []
            for sgn in (1.0, -1.0):
                arg = {"x": x, "z": z, "pf": dict(pf), "pb": dict(pb)}
                pert = _perturbed(base, sgn * V, eps)
                if k is None:
                    arg[d] = pert
                else:
                    arg["pf" if d == "fwd" else "pb"][k] = pert
                L.append(_loss(O, arg["x"], arg["z"], dout, arg["pf"], arg["pb"], axis, idx, hw, pool_scale=scale,
                               local=local))
            fd = (L[0] - L[1]) / (2.0 * eps)
            an = float(np.sum(grad * V))
            size = max(float(np.linalg.norm(grad)), 1e-30)
            assert abs(fd - an) <= 1e-6 * size + floor, "axis %d masked %s pool scale %g local %d: d/d%s %s: " \
                "analytic %.12g, finite difference %.12g" % (axis, masked, scale, local, d, k or "", an, fd)


def pin_bwd_finite_differences_ln(O):
    """The same check for a layer with the post-SSM LayerNorm: every gradient,
    the LayerNorm's weight and bias included, matches the central difference
    of the forward oracle with the norm along a random +-1 direction."""
    eps = 2.0 ** -14
    rng = np.random.default_rng(42)
    for axis, masked, local in ((COLS, False, 0), (ROWS, False, 0), (NONE_ROWMAJOR, False, 0), (ROWS, True, 0),
                                (COLS, False, 3)):
        pf, pb, x, z, dout, idx, hw = _bwd_case(rng, axis, masked)
        E = x.shape[-1]
        ln = {k: _dyadic(v) if k != "eps" else v for k, v in rand_ln(rng, E).items()}
        g = O.layer_bwd(x, z, dout, pf, pb, axis, idx=idx, hw=hw, ln=ln, local_window=local)
        targets = [("x", None), ("z", None), ("ln", "weight"), ("ln", "bias")] + \
            [(d, k) for d in ("fwd", "bwd") for k in ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")]
        for d, k in targets:
            if k is None:
                base, grad = (x, g["dx"]) if d == "x" else (z, g["dz"])
            elif d == "ln":
                base, grad = ln[k], g["ln"][k]
            else:
                base, grad = (pf if d == "fwd" else pb)[k], g[d][k]
            V = rng.choice([-1.0, 1.0], size=base.shape)
            L = []
            for sgn in (1.0, -1.0):
                arg = {"x": x, "z": z, "pf": dict(pf), "pb": dict(pb), "ln": dict(ln)}
                pert = _perturbed(base, sgn * V, eps)
                if k is None:
                    arg[d] = pert
                else:
                    arg["ln" if d == "ln" else ("pf" if d == "fwd" else "pb")][k] = pert
                L.append(_loss(O, arg["x"], arg["z"], dout, arg["pf"], arg["pb"], axis, idx, hw, ln=arg["ln"],
                               local=local))
            fd = (L[0] - L[1]) / (2.0 * eps)
            an = float(np.sum(grad * V))
            scale = max(float(np.linalg.norm(grad)), 1e-30)
            assert abs(fd - an) <= 1e-6 * scale, "LayerNorm axis %d masked %s: d/d%s %s: analytic %.12g, " \
                "finite difference %.12g" % (axis, masked, d, k or "", an, fd)


def pin_bwd_finite_differences_conv(O):
    """The same check for a layer whose x is the producer Conv1D's input: every
    gradient, dx through the conv and the conv's weight and bias included,
    matches the central difference of the forward oracle with the conv: both
    pooling axes, the pool scale, the local backward scan, the post-SSM
    LayerNorm (the whole block: conv, pool, scans, skip, norm, gate, with the
    norm's gradients too) and masked layers (the conv along the kept tokens)."""
    eps = 2.0 ** -14
    rng = np.random.default_rng(44)
    cases = ((COLS, 1.0, 0, False, False), (ROWS, 0.25, 0, False, False), (COLS, 1.0, 3, False, False),
             (ROWS, 1.0, 2, False, False), (COLS, 1.0, 0, False, True), (ROWS, 0.25, 0, False, True),
             (COLS, 1.0, 0, True, False), (ROWS, 1.0, 2, True, True))
    for axis, scale, local, masked, with_ln in cases:
        pf, pb, x, z, dout, idx, hw = _bwd_case(rng, axis, masked)
        if not masked:
            idx = hw = None
        E = x.shape[-1]
        conv = {k: _dyadic(v) for k, v in rand_conv(rng, E).items()}
        ln = {"weight": _dyadic(rng.uniform(0.5, 1.5, E)), "bias": _dyadic(rng.uniform(-0.5, 0.5, E)),
              "eps": 2.0 ** -6} if with_ln else None
        g = O.layer_bwd(x, z, dout, pf, pb, axis, idx=idx, hw=hw, pool_scale=scale, local_window=local, conv=conv,
                        ln=ln)
        out = O.layer(x, z, pf, pb, axis, idx=idx, hw=hw, pool_scale=scale, local_window=local, conv=conv, ln=ln)
        floor = 64 * 2.0 ** -52 * float(np.sum(np.abs(dout * out))) / (2.0 * eps)
        targets = [("x", None), ("z", None), ("conv", "weight"), ("conv", "bias")] + \
            [(d, k) for d in ("fwd", "bwd") for k in ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D")]
        if with_ln:
            targets += [("ln", "weight"), ("ln", "bias")]
        for d, k in targets:
            if k is None:
                base, grad = (x, g["dx"]) if d == "x" else (z, g["dz"])
            elif d in ("conv", "ln"):
                base, grad = (conv if d == "conv" else ln)[k], g[d][k]
            else:
                base, grad = (pf if d == "fwd" else pb)[k], g[d][k]
            V = rng.choice([-1.0, 1.0], size=base.shape)
            L = []
            for sgn in (1.0, -1.0):
                arg = {"x": x, "z": z, "pf": dict(pf), "pb": dict(pb), "conv": dict(conv),
                       "ln": dict(ln) if ln else None}
                pert = _perturbed(base, sgn * V, eps)
                if k is None:
                    arg[d] = pert
                else:
                    arg[d if d in ("conv", "ln") else ("pf" if d == "fwd" else "pb")][k] = pert
                L.append(_loss(O, arg["x"], arg["z"], dout, arg["pf"], arg["pb"], axis, idx, hw, ln=arg["ln"],
                               pool_scale=scale, local=local, conv=arg["conv"]))
            fd = (L[0] - L[1]) / (2.0 * eps)
            an = float(np.sum(grad * V))
            size = max(float(np.linalg.norm(grad)), 1e-30)
            assert abs(fd - an) <= 1e-6 * size + floor, "Conv1D axis %d scale %g local %d masked %s norm %s: " \
                "d/d%s %s: analytic %.12g, finite difference %.12g" % (axis, scale, local, masked, with_ln, d,
                                                                     k or "", an, fd)


def pin_pool_scale_is_a_scaled_input(O):
    """Scaling the pooled tokens by s equals running the layer on s x with the
    skip weights divided by s: the pooled tokens are then s times the row
    means and the skip term (D / s)(s x) is unchanged.  With s = 1/4 both
    rescalings are exact in fp32, so the two agree to fp64 rounding; dense
    COLS and ROWS, masked, with the post-SSM LayerNorm and with the local
    backward scan."""
    rng = np.random.default_rng(43)
    s = 0.25
    for axis, masked, norm, local in ((COLS, False, False, 0), (ROWS, False, True, 0), (COLS, True, False, 0),
                                      (ROWS, True, True, 0), (COLS, False, False, 4)):
        pf, pb, x, z, dout, idx, hw = _bwd_case(rng, axis, masked)
        ln = rand_ln(rng, x.shape[-1]) if norm else None
        got = O.layer(x, z, pf, pb, axis, idx=idx, hw=hw, ln=ln, local_window=local, pool_scale=s)
        qf, qb = dict(pf), dict(pb)
        qf["D"] = (pf["D"].astype(np.float64) / s).astype(np.float32)
        qb["D"] = (pb["D"].astype(np.float64) / s).astype(np.float32)
        want = O.layer((x.astype(np.float64) * s).astype(np.float32), z, qf, qb, axis, idx=idx, hw=hw, ln=ln,
                       local_window=local)
        _close(got, want, tol=1e-12, what="pool scale axis %d masked %s norm %s local %d" % (axis, masked, norm,
                                                                                             local))
        plain = O.layer(x, z, pf, pb, axis, idx=idx, hw=hw, ln=ln, local_window=local)
        assert np.max(np.abs(got - plain)) > 1e-6 * np.max(np.abs(plain)), "the pool scale changed nothing"


def pin_bwd_masked_equals_zero_filled(O):
    """The masked backward pass equals the dense one on the zero-filled grid
    (x, z and dout scattered into zeros): every parameter gradient agrees, and
    dx, dz agree at the kept cells (an unkept cell has z = 0, so silu(0) = 0
    removes it from the pooled adjoint and from dD); also with the post-SSM
    LayerNorm, whose statistics are per token."""
    rng = np.random.default_rng(41)
    for axis, norm in ((COLS, False), (ROWS, False), (COLS, True)):
        pf, pb, x, z, dout, idx, (h, w) = _bwd_case(rng, axis, True)
        B_, K, E = x.shape
        ln = rand_ln(rng, E) if norm else None
        dense = [np.zeros((B_, h * w, E), np.float32) for _ in range(3)]
        for b in range(B_):
            for arr, src in zip(dense, (x, z, dout)):
                arr[b, idx[b]] = src[b]
        xd, zd, dd = (a.reshape(B_, h, w, E) for a in dense)
        gm = O.layer_bwd(x, z, dout, pf, pb, axis, idx=idx, hw=(h, w), ln=ln)
        gd = O.layer_bwd(xd, zd, dd, pf, pb, axis, ln=ln)
        for d in ("fwd", "bwd") + (("ln",) if norm else ()):
            for k in gm[d]:
                _close(gm[d][k], gd[d][k], tol=1e-12, what="masked %s %s" % (d, k))
        for name in ("dx", "dz"):
            flat = gd[name].reshape(B_, h * w, E)
            _close(gm[name], np.stack([flat[b, idx[b]] for b in range(B_)]), tol=1e-12, what="masked " + name)


# ---------------------------------------------------------------- producer Conv1D
def rand_conv(rng, E, KC=4):
    return {"weight": rng.uniform(-0.8, 0.8, (E, KC)).astype(np.float32),
            "bias": rng.uniform(-0.3, 0.3, E).astype(np.float32)}


def _oriented_seq(x, axis):
    """(B, h*w, E) view of x in the oriented grid's sequence order."""
    B, h, w, E = x.shape
    if axis in (ROWS, NONE_COLMAJOR):
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(B, h * w, E)
    return x.reshape(B, h * w, E)


def pin_conv_library(O):
    """The producer's causal depthwise Conv1D + SiLU equals numpy's full
    convolution truncated to the sequence (taps reversed, oldest first), then
    x * sigmoid(x), along the oriented grid's sequence (both orders)."""
    rng = np.random.default_rng(50)
    B_, h, w, E = 2, 5, 3, 6
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    for KC in (4, 2):
        conv = rand_conv(rng, E, KC)
        for axis in (COLS, ROWS, NONE_ROWMAJOR, NONE_COLMAJOR):
            xc = O.conv_silu(x, axis, conv)
            seq = _oriented_seq(x.astype(np.float64), axis)
            got = _oriented_seq(xc, axis)
            for b in range(B_):
                for e in range(E):
                    a = np.convolve(seq[b, :, e], conv["weight"][e, ::-1].astype(np.float64))[: h * w]
                    a = a + float(conv["bias"][e])
                    _close(got[b, :, e], a * expit(a), what="conv KC=%d axis %d" % (KC, axis))


def pin_conv_closed_forms(O):
    """Identity taps (only the newest, weight 1, bias 0) pool silu(x); with
    x_proj_w = 0 the scan is zero and out = (D_fwd + D_bwd) silu(x) silu(z)
    exactly, for any taps."""
    rng = np.random.default_rng(51)
    B_, h, w, E, N, R = 2, 4, 5, 7, 4, 3
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    ident = {"weight": np.zeros((E, 4), np.float32), "bias": np.zeros(E, np.float32)}
    ident["weight"][:, 3] = 1.0
    for axis in (COLS, ROWS):
        st = O.layer(x, z, pf, pb, axis, stages=True, conv=ident)
        sx = silu(x)
        ref_u = sx.mean(axis=2) if axis == COLS else sx.mean(axis=1)
        _close(st["u"], ref_u, what="identity-tap pooled tokens")
        conv = rand_conv(rng, E)
        pf0, pb0 = dict(pf), dict(pb)
        pf0["x_proj_w"] = np.zeros_like(pf["x_proj_w"])
        pb0["x_proj_w"] = np.zeros_like(pb["x_proj_w"])
        out = O.layer(x, z, pf0, pb0, axis, conv=conv)
        Ds = pf["D"].astype(np.float64) + pb["D"].astype(np.float64)
        _close(out, Ds * O.conv_silu(x, axis, conv) * silu(z), what="conv with zero projection")


def pin_conv_transpose(O):
    """With the Conv1D, ROWS is COLS on the transposed grid (the conv follows
    the orientation, as the scan does)."""
    rng = np.random.default_rng(52)
    B_, h, w, E, N, R = 2, 4, 6, 5, 4, 2
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    conv = rand_conv(rng, E)
    r = O.layer(x, z, pf, pb, ROWS, conv=conv)
    xt, zt = (np.ascontiguousarray(a.transpose(0, 2, 1, 3)) for a in (x, z))
    c = O.layer(xt, zt, pf, pb, COLS, conv=conv)
    _close(r, c.transpose(0, 2, 1, 3), what="conv ROWS = COLS transposed")


def pin_conv_causal(O):
    """Changing x at one position of the sequence changes the conv output at
    that position and the next KC - 1 only, in every channel."""
    rng = np.random.default_rng(53)
    B_, h, w, E, KC = 1, 4, 5, 3, 4
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    conv = rand_conv(rng, E, KC)
    for axis in (COLS, ROWS):
        base = _oriented_seq(O.conv_silu(x, axis, conv), axis)
        for r0 in (0, 6, h * w - 2):
            seq = _oriented_seq(x, axis).copy()
            seq[:, r0] += 1.0
            if axis == ROWS:
                x2 = np.ascontiguousarray(seq.reshape(B_, w, h, E).transpose(0, 2, 1, 3))
            else:
                x2 = seq.reshape(B_, h, w, E)
            diff = np.abs(_oriented_seq(O.conv_silu(x2, axis, conv), axis) - base).max(axis=(0, 2))
            changed = set(np.nonzero(diff > 0)[0].tolist())
            assert changed == set(range(r0, min(r0 + KC, h * w))), (axis, r0, sorted(changed))


def _np_conv_silu_seq(seq, conv):
    """numpy: causal depthwise conv + SiLU along axis 1 of seq (B, n, E)."""
    B_, n, E = seq.shape
    out = np.empty(seq.shape)
    for b in range(B_):
        for e in range(E):
            a = np.convolve(seq[b, :, e].astype(np.float64), conv["weight"][e, ::-1].astype(np.float64))[:n]
            a = a + float(conv["bias"][e])
            out[b, :, e] = a * expit(a)
    return out


def _np_layernorm(y, ln):
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    return (y - mu) / np.sqrt(var + ln["eps"]) * ln["weight"].astype(np.float64) + ln["bias"].astype(np.float64)


def pin_conv_masked_sequence(O):
    """A masked layer's Conv1D runs along its kept tokens in the given order:
    its pooled tokens are the fixed-width row means of numpy's causal
    convolution + SiLU along k, and with x_proj_w = 0 out is (D_fwd + D_bwd)
    x_conv silu(z) exactly -- with the post-SSM LayerNorm, numpy's
    normalisation of (D_fwd + D_bwd) x_conv, gated."""
    rng = np.random.default_rng(54)
    B_, h, w, K, E, N, R = 3, 5, 4, 9, 6, 4, 3
    x = rng.standard_normal((B_, K, E)).astype(np.float32)
    z = rng.standard_normal((B_, K, E)).astype(np.float32)
    idx = np.stack([rng.permutation(h * w)[:K] for _ in range(B_)]).astype(np.int32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    conv = rand_conv(rng, E)
    xc = _np_conv_silu_seq(x, conv)
    Ds = pf["D"].astype(np.float64) + pb["D"].astype(np.float64)
    for axis, T, P in ((COLS, h, w), (ROWS, w, h)):
        st = O.layer(x, z, pf, pb, axis, idx=idx, hw=(h, w), stages=True, conv=conv)
        rows = idx // w if axis == COLS else idx % w
        u = np.zeros((B_, T, E))
        for b in range(B_):
            for k in range(K):
                u[b, rows[b, k]] += xc[b, k]
        _close(st["u"], u / P, what="masked conv pooled tokens axis %d" % axis)
        pf0, pb0 = dict(pf), dict(pb)
        pf0["x_proj_w"] = np.zeros_like(pf["x_proj_w"])
        pb0["x_proj_w"] = np.zeros_like(pb["x_proj_w"])
        out = O.layer(x, z, pf0, pb0, axis, idx=idx, hw=(h, w), conv=conv)
        _close(out, Ds * xc * silu(z), what="masked conv with zero projection axis %d" % axis)
        ln = rand_ln(rng, E)
        out = O.layer(x, z, pf0, pb0, axis, idx=idx, hw=(h, w), conv=conv, ln=ln)
        _close(out, _np_layernorm(Ds * xc, ln) * silu(z), what="masked conv + norm, zero projection")


def pin_conv_masked_all_kept(O):
    """Every token kept, in the oriented grid's sequence order (row-major for
    COLS, column-major for ROWS): the masked layer with the Conv1D (and with
    the LayerNorm) equals the dense one, forward and backward."""
    rng = np.random.default_rng(55)
    B_, h, w, E, N, R = 2, 4, 3, 5, 3, 2
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    dout = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    conv = rand_conv(rng, E)
    for axis in (COLS, ROWS):
        order = np.arange(h * w) if axis == COLS else np.array([i * w + j for j in range(w) for i in range(h)])
        idx = np.broadcast_to(order.astype(np.int32), (B_, h * w)).copy()
        for ln in (None, rand_ln(rng, E)):
            take = lambda a: a.reshape(B_, h * w, E)[:, order]
            dense = O.layer(x, z, pf, pb, axis, conv=conv, ln=ln)
            masked = O.layer(take(x), take(z), pf, pb, axis, idx=idx, hw=(h, w), conv=conv, ln=ln)
            _close(masked, take(dense), what="all kept, conv, axis %d" % axis)
            gd = O.layer_bwd(x, z, dout, pf, pb, axis, conv=conv, ln=ln)
            gm = O.layer_bwd(take(x), take(z), take(dout), pf, pb, axis, idx=idx, hw=(h, w), conv=conv, ln=ln)
            _close(gm["dx"], take(gd["dx"]), what="all kept, conv, dx")
            _close(gm["dz"], take(gd["dz"]), what="all kept, conv, dz")
            for k in ("weight", "bias"):
                _close(gm["conv"][k], gd["conv"][k], what="all kept, conv, d conv " + k)
            for d in ("fwd", "bwd"):
                for k in ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "D"):
                    _close(gm[d][k], gd[d][k], what="all kept, conv, d%s.%s" % (d, k))


def pin_conv_norm_zero_projection(O):
    """The whole block (Conv1D, pool, scans, skip, LayerNorm, gate) with
    x_proj_w = 0: the scans give zero, so out is numpy's LayerNorm of
    (D_fwd + D_bwd) x_conv times silu(z), x_conv from numpy's convolution
    along the oriented sequence (both axes)."""
    rng = np.random.default_rng(56)
    B_, h, w, E, N, R = 2, 3, 4, 6, 4, 3
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    pf["x_proj_w"] = np.zeros_like(pf["x_proj_w"])
    pb["x_proj_w"] = np.zeros_like(pb["x_proj_w"])
    conv, ln = rand_conv(rng, E), rand_ln(rng, E)
    Ds = pf["D"].astype(np.float64) + pb["D"].astype(np.float64)
    for axis in (COLS, ROWS):
        seq = _oriented_seq(x, axis)
        xc_seq = _np_conv_silu_seq(seq, conv)
        if axis == ROWS:
            xc = xc_seq.reshape(B_, w, h, E).transpose(0, 2, 1, 3)
        else:
            xc = xc_seq.reshape(B_, h, w, E)
        out = O.layer(x, z, pf, pb, axis, conv=conv, ln=ln)
        _close(out, _np_layernorm(Ds * xc, ln) * silu(z), what="conv + norm, zero projection, axis %d" % axis)


# ---------------------------------------------------------------- LBMamba local backward scan
def _local_case(rng, B_=2, h=10, w=3, E=5, N=4, R=3):
    pf, pb = rand_dir(rng, E, N, R), rand_dir(rng, E, N, R)
    x = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    z = rng.standard_normal((B_, h, w, E)).astype(np.float32)
    return pf, pb, x, z


def pin_local_window_covers_sequence(O):
    """A window as long as the sequence is the global backward scan run with
    the forward direction's projection, step size and decay."""
    rng = np.random.default_rng(60)
    pf, pb, x, z = _local_case(rng)
    shared = dict(pf, D=pb["D"])
    for axis, L in ((COLS, 10), (COLS, 64), (ROWS, 3), (NONE_ROWMAJOR, 30)):
        _close(O.layer(x, z, pf, pb, axis, local_window=L), O.layer(x, z, pf, shared, axis),
               what="local window %d axis %d" % (L, axis))


def pin_local_window_one(O):
    """Windows of one step: s_bwd[t] = sum_n C_t[n] Delta_t B_t[n] u_t."""
    rng = np.random.default_rng(61)
    pf, pb, x, z = _local_case(rng)
    N = pf["A_log"].shape[1]
    R = pf["x_proj_w"].shape[0] - 2 * N
    st = O.layer(x, z, pf, pb, COLS, stages=True, local_window=1)
    v, dl, u = st["fwd"]["v"], st["fwd"]["delta"], st["u"]
    Bt, Ct = v[..., R:R + N], v[..., R + N:]
    ref = dl * u * np.sum(Bt * Ct, axis=-1, keepdims=True)
    _close(st["bwd"]["s"], ref, what="local window 1")


def pin_local_windows_independent(O):
    """Each window [a, a + L) (aligned at t = 0, the last one partial) is the
    reverse scan of that window's inputs alone."""
    rng = np.random.default_rng(62)
    pf, pb, x, z = _local_case(rng)
    N = pf["A_log"].shape[1]
    R = pf["x_proj_w"].shape[0] - 2 * N
    for axis, L in ((COLS, 4), (ROWS, 2), (COLS, 3)):
        st = O.layer(x, z, pf, pb, axis, stages=True, local_window=L)
        T = st["u"].shape[1]
        v, dl, u = st["fwd"]["v"], st["fwd"]["delta"], st["u"]
        for a in range(0, T, L):
            sl = slice(a, min(a + L, T))
            ref = O.scan(u[:, sl], dl[:, sl], v[:, sl], pf["A_log"], R, reverse=True)
            _close(st["bwd"]["s"][:, sl], ref, what="local window [%d, %d) axis %d" % (a, sl.stop, axis))


ALL_PINS = [
    pin_golden_worked_example,
    pin_geometric_series,
    pin_delta_to_zero,
    pin_flip,
    pin_width_one_pooling,
    pin_reset_equals_independent,
    pin_brute_force_layer,
    pin_pooling_invariance,
    pin_transpose,
    pin_masked_equals_zero_filled,
    pin_all_kept,
    pin_zero_projection,
    pin_linear_in_D,
    pin_library_routines,
    pin_mask_rows_exact,
    pin_layernorm_moments,
    pin_layernorm_affine,
    pin_layernorm_library,
    pin_bwd_finite_differences,
    pin_bwd_finite_differences_ln,
    pin_pool_scale_is_a_scaled_input,
    pin_bwd_finite_differences_conv,
    pin_bwd_masked_equals_zero_filled,
    pin_conv_library,
    pin_conv_closed_forms,
    pin_conv_transpose,
    pin_conv_causal,
    pin_conv_masked_sequence,
    pin_conv_masked_all_kept,
    pin_conv_norm_zero_projection,
    pin_local_window_covers_sequence,
    pin_local_window_one,
    pin_local_windows_independent,
]
