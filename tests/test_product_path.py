"""The product path runs the HIP library or fails loudly (CPU checks): a
missing libfastvim.so raises instead of falling back, the package never
imports the oracle, and the autograd front end rejects what the backward
pass does not take before touching any tensor."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import pooled_selective_state_amd as P
from pooled_selective_state_amd import binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(Bd, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libfastvim.so"))
    monkeypatch.setattr(Bd, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        Bd.lib()
    with pytest.raises(RuntimeError, match="not built"):
        P.workspace_bytes(P.make_dims(1, 2, 2, 8), P.POOL_COLS)


def test_package_does_not_import_the_oracle():
    code = "import sys, pooled_selective_state_amd as P; P.lib(); print('oracle' in sys.modules)"
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "False"
    pkg = os.path.join(ROOT, "pooled_selective_state_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "fastvim_oracle" not in text, f


def test_autograd_rejects_unpooled_layers():
    with pytest.raises(ValueError, match="pooled layers"):
        P.pooled_ssm(None, None, {}, P.POOL_NONE_ROWMAJOR)
