"""The C-ABI library loads, exports every function ``include/fastvim.h``
declares, and rejects bad arguments on the host before touching the GPU.

No test here launches a kernel: every call below fails validation, which
happens before any HIP call, so these run on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

import pooled_selective_state_amd as P
from pooled_selective_state_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fastvim.h")

OK, ENULL, EDIMS, EUNSUP, EALIGN, EOVERLAP, EWS, EHIP, EARG, EBADIDX, EWAIT, ESCRATCH = (0, -1, -2, -3, -4, -5, -6, -7, -8,
                                                                     -9, -10, -11)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fastvim_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = P.lib()
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(Bd.EXPORTED_SYMBOLS)
    assert lib.fastvim_abi_version() == 13


def test_status_strings():
    lib = P.lib()
    for code in (OK, ENULL, EDIMS, EUNSUP, EALIGN, EOVERLAP, EWS, EHIP, EARG, EBADIDX, EWAIT, ESCRATCH):
        assert lib.fastvim_status_string(code)
    assert lib.fastvim_status_string(123) == b"unknown status"


def test_struct_layout_matches_header():
    # int64 x 7 + int32 x 2; five pointers; two dir structs + ptr + size_t + 2 x u32 + 2 ptrs + f32 + u32
    # + 2 conv ptrs + saved_u
    assert ctypes.sizeof(Bd.Dims) == 64
    assert ctypes.sizeof(Bd.DirParams) == 40
    assert ctypes.sizeof(Bd.Params) == 2 * 40 + 8 + 8 + 8 + 8 + 8 + 4 + 4 + 8 + 8 + 8
    assert Bd.Params.saved_u.offset == ctypes.sizeof(Bd.Params) - 8
    assert Bd.Params.pool_scale.offset == Bd.Params.ln_eps.offset + 4
    assert ctypes.sizeof(Bd.DirGrads) == 40 and ctypes.sizeof(Bd.Grads) == 112
    assert Bd.Grads.ln_weight.offset == 80 and Bd.Grads.ln_bias.offset == 88
    assert Bd.Grads.conv_w.offset == 96 and Bd.Grads.conv_b.offset == 104


def _ws(dims, axis):
    return P.workspace_bytes(dims, axis)


def test_workspace_bytes():
    def al(n):
        return (n + 255) // 256 * 256
    def sync(B):
        return al(4 * (2 + 2 * B))
    d = P.make_dims(128, 128, 128, 384, 16, 12)
    B, T, E, NX = 128, 128, 384, 44
    assert _ws(d, P.POOL_COLS) == 3 * al(B * T * E * 4) + al(B * T * 2 * NX * 4) + sync(B)
    d2 = P.make_dims(128, 128, 64, 384, 16, 12)
    assert _ws(d2, P.POOL_ROWS) == 3 * al(128 * 64 * E * 4) + al(128 * 64 * 2 * NX * 4) + sync(B)
    T2 = 128 * 128
    assert _ws(d, P.POOL_NONE_ROWMAJOR) == 2 * al(B * T2 * E * 4) + al(B * T2 * 2 * NX * 4) + sync(B)
    dm = P.make_dims(256, 14, 14, 1536, 16, 48, 49, P.BF16)
    expect = (3 * al(256 * 14 * 1536 * 4) + al(256 * 14 * 2 * 80 * 4) + al(256 * 49 * 4) + al(256 * 4)
              + sync(256))
    assert _ws(dm, P.POOL_COLS) == expect
    # invalid sizes report 0
    assert _ws(P.make_dims(1, 2, 2, 8, 15, 4), P.POOL_COLS) == 0
    assert _ws(dm, P.POOL_NONE_ROWMAJOR) == 0


class FakeCall:
    """Arguments with fake (never dereferenced) device addresses."""

    def __init__(self, B=2, h=4, w=5, E=16, N=16, R=4, K=0, io=P.F32, axis=P.POOL_COLS):
        self.dims = P.make_dims(B, h, w, E, N, R, K, io)
        self.axis = axis
        base = 1 << 40
        esz = 4 if io == P.F32 else 2
        n = B * (K if K else h * w) * E * esz
        span = (n + 4096) // 4096 * 4096
        self.x, self.z, self.out = base, base + span, base + 2 * span
        self.idx = base + 3 * span if K else None
        pbase = base + 4 * span
        dirs = [Bd.DirParams(*[pbase + (4 * i + j) * 4096 for j in range(5)]) for i in range(2)]
        wsb = max(_ws(self.dims, axis), 256)
        self.params = Bd.Params(dirs[0], dirs[1], pbase + 16 * 4096, wsb, 0, 0)

    def fwd(self):
        return P.lib().fastvim_ssm_fwd(self.x, self.z, ctypes.byref(self.params), ctypes.byref(self.dims),
                                       self.axis, self.idx, self.out, None)


def expect(call, code):
    assert call.fwd() == code


def test_null_pointers():
    lib = P.lib()
    c = FakeCall()
    assert lib.fastvim_ssm_fwd(c.x, c.z, None, ctypes.byref(c.dims), 0, None, c.out, None) == ENULL
    assert lib.fastvim_ssm_fwd(c.x, c.z, ctypes.byref(c.params), None, 0, None, c.out, None) == ENULL
    for attr in ("x", "z", "out"):
        c = FakeCall()
        setattr(c, attr, None)
        expect(c, ENULL)
    for d in ("fwd", "bwd"):
        for f in Bd.DIR_FIELDS:
            c = FakeCall()
            setattr(getattr(c.params, d), f, None)
            expect(c, ENULL)
    c = FakeCall(K=3)
    c.idx = None
    expect(c, ENULL)


def test_bad_dims():
    for kw in (dict(h=0), dict(w=-1), dict(E=0), dict(R=0), dict(B=-1), dict(K=-2)):
        expect(FakeCall(**kw), EDIMS)
    expect(FakeCall(K=21), EDIMS)  # K > h*w
    c = FakeCall(K=4)
    c.axis = P.POOL_NONE_ROWMAJOR
    expect(c, EDIMS)  # masked needs a pooled axis


def test_unsupported():
    expect(FakeCall(N=8), EUNSUP)
    expect(FakeCall(R=65), EUNSUP)
    expect(FakeCall(E=4100), EUNSUP)
    expect(FakeCall(E=18), EUNSUP)  # fp32 needs E % 4 == 0
    expect(FakeCall(E=20, io=P.BF16), EUNSUP)  # bf16 needs E % 8 == 0
    expect(FakeCall(h=200, w=100, K=5), EUNSUP)  # masked grid > 16384 cells
    expect(FakeCall(B=1, h=1 << 14, w=1 << 14, E=8), EUNSUP)  # an image of 2^31 elements


def test_bad_enums():
    expect(FakeCall(axis=4), EARG)
    expect(FakeCall(axis=-1), EARG)
    expect(FakeCall(io=2), EARG)
    c = FakeCall()
    c.idx = c.out + (1 << 30)
    expect(c, EARG)  # mask_idx with K = 0
    lib = P.lib()
    c = FakeCall()
    assert lib.fastvim_ssm_stage(5, c.x, c.z, ctypes.byref(c.params), ctypes.byref(c.dims), 0, None, c.out,
                                 None) == EARG
    for flags in (P.FLAG_STAGED | P.FLAG_FUSED, 128, 1 << 31):  # conflicting or unknown flags
        c = FakeCall()
        c.params.flags = flags
        expect(c, EARG)
    for tuning in (1 << 17, 1 << 31):  # unknown tuning bits
        c = FakeCall()
        c.params.tuning = tuning
        expect(c, EARG)


def test_alignment():
    for attr, off in (("x", 4), ("z", 8), ("out", 12)):
        c = FakeCall()
        setattr(c, attr, getattr(c, attr) + off)
        expect(c, EALIGN)
    c = FakeCall()
    c.params.workspace += 128
    expect(c, EALIGN)
    c = FakeCall()
    c.params.fwd.D += 2
    expect(c, EALIGN)
    c = FakeCall()
    c.params.bwd.x_proj_w += 8
    expect(c, EALIGN)
    c = FakeCall()
    c.params.bwd.A_log += 4  # scalar-read parameters need only 4 bytes ...
    c.params.workspace_bytes -= 1  # ... so the later workspace check is what fails (nothing launches)
    expect(c, EWS)
    c = FakeCall(K=3)
    c.idx += 2
    expect(c, EALIGN)


def test_overlap():
    c = FakeCall()
    c.out = c.x + 64
    expect(c, EOVERLAP)
    c = FakeCall()
    c.out = c.z
    expect(c, EOVERLAP)
    c = FakeCall()
    c.params.workspace = c.out
    expect(c, EOVERLAP)


def test_workspace_checks():
    c = FakeCall()
    c.params.workspace_bytes -= 1
    expect(c, EWS)
    c = FakeCall()
    c.params.workspace = c.params.workspace + 64
    expect(c, EALIGN)
    # a NULL workspace is the stream-ordered allocator's: every argument is
    # still checked first, before anything is allocated
    c = FakeCall()
    c.params.workspace = None
    c.x += 4
    expect(c, EALIGN)
    c = FakeCall()
    c.params.workspace = None
    c.out = c.x
    expect(c, EOVERLAP)
    # calls that need the caller's workspace
    lib = P.lib()
    c = FakeCall()
    c.params.workspace = None
    assert lib.fastvim_ssm_stage(P.STAGE_POOL, c.x, c.z, ctypes.byref(c.params), ctypes.byref(c.dims), c.axis,
                                 None, c.out, None) == EWS
    assert lib.fastvim_ssm_export(ctypes.byref(c.params), ctypes.byref(c.dims), c.axis, P.EXPORT_U, c.out,
                                  1 << 20, None) == EWS
    assert lib.fastvim_get_device_error(ctypes.byref(c.params), None) == EWS
    assert lib.fastvim_get_device_error(None, None) == ENULL


class FakeStages(FakeCall):
    """fastvim_ssm_fwd_stages with fake destinations far from the other arguments."""

    def __init__(self, **kw):
        super().__init__(**kw)
        far = 1 << 43
        self.u, self.sf, self.sb, self.rows = far, far + (1 << 30), far + (2 << 30), far + (3 << 30)

    def fwd(self):
        return P.lib().fastvim_ssm_fwd_stages(self.x, self.z, ctypes.byref(self.params), ctypes.byref(self.dims),
                                              self.axis, self.idx, self.out, None, self.u, self.sf, self.sb,
                                              self.rows)


def test_fwd_stages_validation():
    c = FakeStages()
    expect(c, EARG)  # row ids of a dense layer
    c = FakeStages(axis=P.POOL_NONE_ROWMAJOR)
    c.rows = None
    expect(c, EARG)  # pooled tokens of an unpooled layer
    c = FakeStages()
    c.rows = None
    c.sf += 2
    expect(c, EALIGN)
    c = FakeStages()
    c.rows = None
    c.sb = c.x
    expect(c, EOVERLAP)  # a destination over an input
    c = FakeStages()
    c.rows = None
    c.sb = c.sf + 64
    expect(c, EOVERLAP)  # two destinations over each other
    c = FakeStages()
    c.rows = None
    c.u = c.params.workspace
    expect(c, EOVERLAP)  # a destination over the workspace
    c = FakeStages()
    c.rows = None
    c.x += 4
    expect(c, EALIGN)  # the layer's own arguments as fastvim_ssm_fwd
    c = FakeStages(B=0)
    c.rows = None
    expect(c, OK)  # nothing to run or copy


def test_empty_batch_is_a_noop():
    c = FakeCall(B=0)
    c.x = c.z = c.out = None
    expect(c, OK)


def test_export_arguments():
    lib = P.lib()
    c = FakeCall()
    assert lib.fastvim_ssm_export(ctypes.byref(c.params), ctypes.byref(c.dims), 0, 9, c.out, 1 << 20, None) == EARG
    assert lib.fastvim_ssm_export(ctypes.byref(c.params), ctypes.byref(c.dims), 0, -1, c.out, 1 << 20, None) == EARG
    assert lib.fastvim_ssm_export(ctypes.byref(c.params), ctypes.byref(c.dims), 0, P.EXPORT_ROWS, c.out, 1 << 20,
                                  None) == EARG  # dense layer has no rows
    assert lib.fastvim_ssm_export(ctypes.byref(c.params), ctypes.byref(c.dims), 0, P.EXPORT_U, c.out, 16,
                                  None) == EDIMS  # destination too small
    assert lib.fastvim_ssm_export_bytes(ctypes.byref(c.dims), 0, P.EXPORT_U) == 2 * 4 * 16 * 4
    assert lib.fastvim_ssm_export_bytes(ctypes.byref(c.dims), P.POOL_NONE_ROWMAJOR, P.EXPORT_U) == 0


@pytest.mark.parametrize("what", range(7))
def test_export_bytes_masked(what):
    lib = P.lib()
    d = P.make_dims(3, 4, 5, 16, 16, 4, 7, P.BF16)
    n = lib.fastvim_ssm_export_bytes(ctypes.byref(d), P.POOL_ROWS, what)
    T = 5
    expect_n = {0: 3 * T * 16 * 4, 1: 3 * T * 2 * 36 * 4, 2: 3 * T * 16 * 4, 3: 3 * T * 16 * 4, 4: 3 * 7 * 4, 5: 12,
                6: 4}
    assert n == expect_n[what]


def test_calib_copy_validation():
    """The calibration copy rejects bad arguments before launching anything."""
    lib = P.lib()
    a, b = 0x10000, 0x20000
    assert lib.fastvim_calib_copy(None, None, 0, None) == OK  # nothing to do
    assert lib.fastvim_calib_copy(None, b, 64, None) == ENULL
    assert lib.fastvim_calib_copy(a, None, 64, None) == ENULL
    assert lib.fastvim_calib_copy(a + 4, b, 64, None) == EALIGN
    assert lib.fastvim_calib_copy(a, b + 8, 64, None) == EALIGN
    assert lib.fastvim_calib_copy(a, b, 60, None) == EALIGN
    assert lib.fastvim_calib_copy(a, a + 32, 64, None) == EOVERLAP
    assert lib.fastvim_calib_copy(a + 32, a, 64, None) == EOVERLAP


def test_post_norm_validation():
    """The post-SSM LayerNorm's parameters are checked before any launch."""
    base = 0x40000
    for (w, b, eps, code) in ((None, base, 1e-5, ENULL), (base, None, 1e-5, ENULL), (base + 4, base, 1e-5, EALIGN),
                              (base, base + 8, 1e-5, EALIGN), (base, base, 0.0, EARG), (base, base, -1.0, EARG),
                              (base, base, float("nan"), EARG), (base, base, float("inf"), EARG)):
        c = FakeCall()
        c.params.flags = P.FLAG_POST_NORM
        c.params.ln_weight, c.params.ln_bias, c.params.ln_eps = w, b, eps
        expect(c, code)


# ------------------------------------------------------------------ backward
class FakeBwd:
    """Backward-call arguments with fake (never dereferenced) device addresses."""

    def __init__(self, B=2, h=4, w=5, E=16, N=16, R=4, K=0, io=P.F32, axis=P.POOL_COLS):
        self.dims = P.make_dims(B, h, w, E, N, R, K, io)
        self.axis = axis
        base = 1 << 41
        esz = 4 if io == P.F32 else 2
        n = B * (K if K else h * w) * E * esz
        span = (n + 4096) // 4096 * 4096
        self.x, self.z, self.dout, self.dx, self.dz = (base + i * span for i in range(5))
        self.idx = base + 5 * span if K else None
        pbase = base + 6 * span
        dirs = [Bd.DirParams(*[pbase + (5 * i + j) * 65536 for j in range(5)]) for i in range(2)]
        gbase = pbase + 10 * 65536
        self.grads = Bd.Grads(*[Bd.DirGrads(*[gbase + (5 * i + j) * 65536 for j in range(5)]) for i in range(2)])
        wsb = max(P.bwd_workspace_bytes(self.dims, axis), 256)
        self.params = Bd.Params(dirs[0], dirs[1], gbase + 10 * 65536, wsb, 0, 0)

    def bwd(self):
        return P.lib().fastvim_ssm_bwd(self.x, self.z, self.dout, ctypes.byref(self.params), ctypes.byref(self.dims),
                                       self.axis, self.idx, self.dx, self.dz, ctypes.byref(self.grads), None)


def test_saved_u_checks_forward():
    far = 1 << 44  # an address far from every other argument
    c = FakeCall(axis=P.POOL_NONE_ROWMAJOR)
    c.params.saved_u = far
    expect(c, EARG)  # unpooled: no pooled tokens to keep
    c = FakeCall()
    c.params.saved_u = far + 4
    expect(c, EALIGN)
    for target in ("x", "z", "out"):
        c = FakeCall()
        c.params.saved_u = getattr(c, target)
        expect(c, EOVERLAP)
    c = FakeCall()
    c.params.saved_u = c.params.workspace + 256
    expect(c, EOVERLAP)


def test_saved_u_checks_backward():
    far = 1 << 44
    c = FakeBwd()
    c.params.saved_u = far + 8
    assert c.bwd() == EALIGN
    for target in ("dx", "dz"):
        c = FakeBwd()
        c.params.saved_u = getattr(c, target)
        assert c.bwd() == EOVERLAP, target
    c = FakeBwd()
    c.params.saved_u = c.params.workspace
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.params.saved_u = c.grads.fwd.D
    assert c.bwd() == EOVERLAP


def test_bwd_workspace_bytes():
    d = P.make_dims(2, 4, 5, 16, 16, 4)
    assert P.bwd_workspace_bytes(d, P.POOL_COLS) > P.workspace_bytes(d, P.POOL_COLS) > 0
    assert P.bwd_workspace_bytes(d, P.POOL_NONE_ROWMAJOR) == 0  # unpooled: no backward pass
    assert P.bwd_workspace_bytes(P.make_dims(2, 721, 4, 16), P.POOL_COLS) == 0  # scan of 721 steps
    assert P.bwd_workspace_bytes(P.make_dims(2, 721, 4, 16), P.POOL_ROWS) > 0   # ... but 4 steps over columns
    # scans longer than 128 steps: the checkpoint region grows with T
    small, big = (P.bwd_workspace_bytes(P.make_dims(2, h, 4, 16), P.POOL_COLS) for h in (128, 720))
    assert big > small > 0
    assert P.bwd_workspace_bytes(P.make_dims(2, 4, 5, 16, 8), P.POOL_COLS) == 0  # N != 16


def test_bwd_null_pointers():
    lib = P.lib()
    c = FakeBwd()
    assert lib.fastvim_ssm_bwd(c.x, c.z, c.dout, None, ctypes.byref(c.dims), 0, None, c.dx, c.dz,
                               ctypes.byref(c.grads), None) == ENULL
    assert lib.fastvim_ssm_bwd(c.x, c.z, c.dout, ctypes.byref(c.params), None, 0, None, c.dx, c.dz,
                               ctypes.byref(c.grads), None) == ENULL
    assert lib.fastvim_ssm_bwd(c.x, c.z, c.dout, ctypes.byref(c.params), ctypes.byref(c.dims), 0, None, c.dx, c.dz,
                               None, None) == ENULL
    for attr in ("x", "z", "dout", "dx", "dz"):
        c = FakeBwd()
        setattr(c, attr, None)
        assert c.bwd() == ENULL, attr
    for d in ("fwd", "bwd"):
        for f in Bd.DIR_FIELDS:
            c = FakeBwd()
            setattr(getattr(c.params, d), f, None)
            assert c.bwd() == ENULL
            c = FakeBwd()
            setattr(getattr(c.grads, d), f, None)
            assert c.bwd() == ENULL
    c = FakeBwd(K=3)
    c.idx = None
    assert c.bwd() == ENULL


def test_bwd_unsupported_and_bad_flags():
    for axis in (P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR):
        assert FakeBwd(axis=axis).bwd() == EUNSUP
    assert FakeBwd(h=721, R=12).bwd() == EUNSUP  # longer than the scan adjoint's LDS holds (720 at rank 16)
    assert FakeBwd(h=513, R=20).bwd() == EUNSUP  # 512 at rank 32
    assert FakeBwd(N=8).bwd() == EUNSUP
    for flags, code in ((P.FLAG_FUSED, EUNSUP), (128, EARG),
                        (P.FLAG_STAGED, OK)):
        c = FakeBwd()
        c.params.flags = flags
        if code != OK:
            assert c.bwd() == code, flags
    c = FakeBwd()
    c.idx = c.dx + (1 << 30)
    assert c.bwd() == EARG  # mask_idx with a dense layer
    c = FakeBwd()
    c.params.tuning = 1
    assert c.bwd() == EARG  # no single launch to tune
    for tuning in (P.TUNING_POLL1, P.tuning_bwd_groups(33), P.tuning_bwd_groups(63), 1 << 26):
        c = FakeBwd()
        c.params.tuning = tuning
        assert c.bwd() == EARG, hex(tuning)  # only the image groups, at most 32
    for groups in (0, 1, 4, 32):
        # accepted: the call goes on to the next check (a misaligned dx here)
        c = FakeBwd()
        c.params.tuning = P.tuning_bwd_groups(groups)
        c.dx += 4
        assert c.bwd() == EALIGN, groups


def test_forward_accepts_the_backward_groups():
    """A params struct shared by the forward and backward calls may carry the
    backward's image groups: the forward calls ignore them."""
    c = FakeCall()
    c.params.tuning = P.tuning_bwd_groups(8) | P.tuning_lags(3, 7)
    c.x += 4
    expect(c, EALIGN)
    for bad in (P.tuning_bwd_groups(8) | (1 << 28), 1 << 17, P.tuning_scan_out(3)):
        c = FakeCall()
        c.params.tuning = bad
        expect(c, EARG)


def test_forward_scan_out_tuning():
    """Bits 26-27 choose how short stage-kernel layers run their scan and
    output stages: 0, 1 and 2 are accepted (the call goes on to its next
    check, a misaligned x here), 3 is ARG."""
    for n in (P.SCAN_OUT_AUTO, P.SCAN_OUT_TWO, P.SCAN_OUT_ONE):
        c = FakeCall()
        c.params.tuning = P.tuning_scan_out(n) | P.tuning_lags(3, 7)
        c.x += 4
        expect(c, EALIGN)
    c = FakeCall()
    c.params.tuning = P.tuning_scan_out(3)
    expect(c, EARG)


def test_bwd_workspace_covers_every_grouping():
    """The backward workspace size does not depend on the tuning word, so it
    covers the largest of the groupings a call may ask for: never smaller
    than for fewer images, and growing about linearly in B."""
    sizes = [P.bwd_workspace_bytes(P.make_dims(B, 128, 128, 384, 16, 12), P.POOL_COLS) for B in (1, 16, 128)]
    assert 0 < sizes[0] < sizes[1] < sizes[2]
    assert sizes[2] < 9 * sizes[1]


def _norm_bwd(**kw):
    """A backward call with the post-SSM LayerNorm (fake addresses)."""
    c = FakeBwd(**kw)
    far = 1 << 45
    c.params.flags = P.FLAG_POST_NORM
    c.params.ln_weight, c.params.ln_bias, c.params.ln_eps = far, far + 65536, 1e-5
    c.grads.ln_weight, c.grads.ln_bias = far + 2 * 65536, far + 3 * 65536
    return c


def test_pool_scale_validation():
    """The pool scale needs a pooled layer and a finite value, in both calls;
    a valid one passes every check (the call then stops at the workspace)."""
    for axis in (P.POOL_NONE_ROWMAJOR, P.POOL_NONE_COLMAJOR):
        c = FakeCall(axis=axis)
        c.params.flags, c.params.pool_scale = P.FLAG_POOL_SCALE, 0.25
        expect(c, EARG)
    for v in (float("nan"), float("inf"), -float("inf")):
        c = FakeCall()
        c.params.flags, c.params.pool_scale = P.FLAG_POOL_SCALE, v
        expect(c, EARG)
        c = FakeBwd()
        c.params.flags, c.params.pool_scale = P.FLAG_POOL_SCALE, v
        assert c.bwd() == EARG
    for v in (0.25, -3.0, 0.0):
        c = FakeCall(K=3)
        c.params.flags, c.params.pool_scale = P.FLAG_POOL_SCALE, v
        c.params.workspace_bytes -= 1
        expect(c, EWS)
        c = FakeBwd()
        c.params.flags, c.params.pool_scale = P.FLAG_POOL_SCALE, v
        c.params.workspace_bytes -= 1
        assert c.bwd() == EWS
    # without the flag the field is not looked at
    c = FakeCall()
    c.params.pool_scale = float("nan")
    c.params.workspace_bytes -= 1
    expect(c, EWS)


def test_bwd_post_norm_validation():
    """The LayerNorm's parameters and gradient buffers of a backward call are
    checked before any launch; E > 2048 is not supported with the norm."""
    for attr in ("ln_weight", "ln_bias"):
        c = _norm_bwd()
        setattr(c.params, attr, None)
        assert c.bwd() == ENULL, attr
        c = _norm_bwd()
        setattr(c.grads, attr, None)
        assert c.bwd() == ENULL, "grad " + attr
    c = _norm_bwd()
    c.params.ln_bias += 4
    assert c.bwd() == EALIGN
    c = _norm_bwd()
    c.grads.ln_weight += 2
    assert c.bwd() == EALIGN
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        c = _norm_bwd()
        c.params.ln_eps = eps
        assert c.bwd() == EARG, eps
    c = _norm_bwd()
    c.grads.ln_bias = c.grads.ln_weight + 32  # the two gradients overlap
    assert c.bwd() == EOVERLAP
    c = _norm_bwd()
    c.grads.ln_weight = c.params.ln_weight  # gradient over its parameter
    assert c.bwd() == EOVERLAP
    c = _norm_bwd()
    c.grads.ln_bias = c.dz + 64
    assert c.bwd() == EOVERLAP
    c = _norm_bwd()
    c.grads.ln_weight = c.grads.fwd.D
    assert c.bwd() == EOVERLAP
    assert _norm_bwd(E=2056).bwd() == EUNSUP
    # without the flag the norm's pointers are not looked at
    c = FakeBwd()
    c.grads.ln_weight = c.grads.ln_bias = c.dx
    c.params.workspace_bytes -= 1
    assert c.bwd() == EWS  # the call got past every other check


def test_bwd_local_scan_validation():
    """With the local backward scan the backward set's x_proj_w, dt_proj_w,
    dt_proj_b and A_log may be NULL (the call then gets past every check),
    while its D and every gradient buffer stay required."""
    c = FakeBwd()
    c.params.flags = P.FLAG_LOCAL_BWD
    for f in ("x_proj_w", "dt_proj_w", "dt_proj_b", "A_log"):
        setattr(c.params.bwd, f, None)
    c.params.workspace_bytes -= 1
    assert c.bwd() == EWS
    c = FakeBwd()
    c.params.flags = P.FLAG_LOCAL_BWD
    c.params.bwd.D = None
    assert c.bwd() == ENULL
    c = FakeBwd()
    c.params.flags = P.FLAG_LOCAL_BWD
    c.grads.bwd.A_log = None
    assert c.bwd() == ENULL


def _conv_bwd(**kw):
    """A backward call with the producer Conv1D (fake addresses)."""
    c = FakeBwd(**kw)
    far = 1 << 45
    c.params.flags = P.FLAG_CONV
    c.params.conv_w, c.params.conv_b = far, far + 65536
    c.grads.conv_w, c.grads.conv_b = far + 2 * 65536, far + 3 * 65536
    return c


def test_bwd_conv_validation():
    """The Conv1D's parameters and gradient buffers of a backward call are
    checked before any launch, also with masked layers and the LayerNorm
    (whose conv is written out), where the two gradient pairs must not
    overlap either."""
    for attr in ("conv_w", "conv_b"):
        c = _conv_bwd()
        setattr(c.params, attr, None)
        assert c.bwd() == ENULL, attr
        c = _conv_bwd()
        setattr(c.grads, attr, None)
        assert c.bwd() == ENULL, "grad " + attr
    c = _conv_bwd()
    c.params.conv_w += 4
    assert c.bwd() == EALIGN
    c = _conv_bwd()
    c.grads.conv_b += 2
    assert c.bwd() == EALIGN
    c = _conv_bwd()
    c.grads.conv_b = c.grads.conv_w + 16  # the two gradients overlap
    assert c.bwd() == EOVERLAP
    c = _conv_bwd()
    c.grads.conv_w = c.params.conv_w
    assert c.bwd() == EOVERLAP
    c = _conv_bwd()
    c.grads.conv_b = c.dx + 32
    assert c.bwd() == EOVERLAP
    c = _conv_bwd(K=3)
    c.grads.conv_b += 2
    assert c.bwd() == EALIGN
    c = _conv_bwd()
    c.params.flags |= P.FLAG_POST_NORM
    far = 1 << 45
    c.params.ln_weight, c.params.ln_bias, c.params.ln_eps = far, far + 65536, 1e-5
    c.grads.ln_weight, c.grads.ln_bias = far + 2 * 65536, c.grads.conv_w + 8  # over the conv's gradient
    assert c.bwd() == EOVERLAP
    c = _conv_bwd()
    c.params.workspace_bytes -= 1
    assert c.bwd() == EWS  # past every other check


def test_bwd_alignment():
    for attr, off in (("dx", 4), ("dz", 8), ("dout", 4), ("x", 2)):
        c = FakeBwd()
        setattr(c, attr, getattr(c, attr) + off)
        assert c.bwd() == EALIGN, attr
    c = FakeBwd()
    c.grads.fwd.A_log += 2
    assert c.bwd() == EALIGN
    c = FakeBwd()
    c.params.workspace += 64
    c.params.workspace_bytes += 256
    assert c.bwd() == EALIGN


def test_bwd_overlap():
    c = FakeBwd()
    c.dx = c.x
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.dz = c.dx + 64
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.params.workspace = c.dout
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.grads.bwd.D = c.grads.fwd.D
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.grads.fwd.x_proj_w = c.params.fwd.x_proj_w
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.grads.fwd.D = c.params.workspace + 512
    assert c.bwd() == EOVERLAP


def test_bwd_workspace_checks():
    c = FakeBwd()
    c.params.workspace_bytes -= 1
    assert c.bwd() == EWS
    # NULL: the stream-ordered allocator's; the other arguments are checked first
    c = FakeBwd()
    c.params.workspace = None
    c.dz = c.dx
    assert c.bwd() == EOVERLAP
    c = FakeBwd()
    c.params.workspace = None
    c.grads.fwd.D = None
    assert c.bwd() == ENULL


def test_conv_validation():
    """The producer Conv1D's arguments and scope are checked before any launch."""
    base = 0x80000
    for (cw, cb, code) in ((None, base, ENULL), (base, None, ENULL), (base + 4, base, EALIGN),
                           (base, base + 2, EALIGN)):
        c = FakeCall()
        c.params.flags = P.FLAG_CONV
        c.params.conv_w, c.params.conv_b = cw, cb
        expect(c, code)
    # masked, unpooled and LayerNorm layers take the conv (written out first);
    # their other arguments are still checked
    for kw, axis in ((dict(K=3), P.POOL_COLS), (dict(), P.POOL_NONE_ROWMAJOR), (dict(), P.POOL_NONE_COLMAJOR)):
        c = FakeCall(axis=axis, **kw)
        c.params.flags = P.FLAG_CONV
        c.params.conv_w, c.params.conv_b = base + 4, base
        expect(c, EALIGN)
    c = FakeCall()
    c.params.flags = P.FLAG_CONV | P.FLAG_POST_NORM
    c.params.conv_w = c.params.conv_b = c.params.ln_weight = c.params.ln_bias = base
    c.params.ln_eps = 1e-5
    c.params.workspace_bytes -= 1
    expect(c, EWS)
    c = FakeCall(K=3)
    c.params.flags = P.FLAG_CONV
    c.params.conv_w, c.params.conv_b = base, base
    lib = P.lib()
    assert lib.fastvim_ssm_stage(P.STAGE_POOL, c.x, c.z, ctypes.byref(c.params), ctypes.byref(c.dims), c.axis,
                                 c.idx, c.out, None) == EUNSUP  # the written-out conv is a step of its own
    c = FakeBwd()
    c.params.flags = P.FLAG_CONV
    assert c.bwd() == ENULL  # the backward pass takes the conv, and needs its parameters
    c = FakeCall()
    c.params.flags = 128
    expect(c, EARG)


def test_local_bwd_validation():
    """LBMamba's local backward scan reads only D of the backward parameters:
    a NULL backward D is an error, misaligned D too."""
    c = FakeCall()
    c.params.flags = P.FLAG_LOCAL_BWD
    c.params.bwd.D = None
    expect(c, ENULL)
    c = FakeCall()
    c.params.flags = P.FLAG_LOCAL_BWD
    c.params.bwd.D += 2
    expect(c, EALIGN)
    c = FakeCall()
    c.params.flags = P.FLAG_LOCAL_BWD
    c.params.fwd.A_log = None  # the forward set is still read
    expect(c, ENULL)


class FakeNoalloc(FakeCall):
    def fwd(self):
        return P.lib().fastvim_ssm_fwd_noalloc(self.x, self.z, ctypes.byref(self.params), ctypes.byref(self.dims),
                                               self.axis, self.idx, self.out, None)


def test_noalloc_validation():
    """fastvim_ssm_fwd_noalloc checks its arguments as fastvim_ssm_fwd does
    (the workspace fields are not read), and rejects a layer whose scratch
    exceeds its fixed buffer, before touching the GPU."""
    c = FakeNoalloc()
    c.params.workspace = None
    c.x += 4
    expect(c, EALIGN)
    c = FakeNoalloc(K=3)
    c.idx = None
    expect(c, ENULL)
    c = FakeNoalloc(B=0)
    c.x = c.z = c.out = None
    expect(c, OK)
    big = FakeNoalloc(B=4, h=128, w=128, E=256, axis=P.POOL_NONE_ROWMAJOR)
    assert _ws(big.dims, big.axis) > Bd.NOALLOC_SCRATCH_BYTES
    expect(big, ESCRATCH)
    for cfg_dims, axis in ((P.make_dims(128, 128, 128, 384, 16, 12), P.POOL_COLS),
                           (P.make_dims(128, 128, 128, 384, 16, 12), P.POOL_ROWS),
                           (P.make_dims(256, 14, 14, 1536, 16, 48, 49, P.BF16), P.POOL_COLS)):
        assert _ws(cfg_dims, axis) <= Bd.NOALLOC_SCRATCH_BYTES  # the pooled workloads fit
