"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle's C source is compiled with ``-fsanitize=address,undefined`` into a
temporary directory and the whole pin suite runs against it in a child
process (the sanitizer runtimes preloaded, as the Python interpreter itself is
not instrumented): an out-of-bounds access, a use after free or undefined
arithmetic anywhere on the pins' paths aborts the child.  One planted mistake
that indexes past a buffer must then be stopped, by a pin or by the
sanitizer.  The real oracle library is not touched.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "fastvim_oracle.c")
ROOT = os.path.dirname(os.path.dirname(SRC))


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
pytestmark = pytest.mark.skipif(not (ASAN and UBSAN), reason="gcc's sanitizer runtimes are not installed")

_CHILD = """
import sys
sys.path[:0] = ['.', 'tests']
import oracle, pins
O = oracle.Oracle(sys.argv[1])
O.set_threads(2)
failed = []
for pin in pins.ALL_PINS:
    try:
        pin(O)
        print('PASS', pin.__name__, flush=True)
    except (AssertionError, ValueError, FloatingPointError) as e:
        print('CAUGHT', pin.__name__, str(e)[:200], flush=True)
"""


def _build(src_text, tmp_path, name):
    src = tmp_path / (name + ".c")
    src.write_text(src_text)
    out = str(tmp_path / ("lib%s.so" % name))
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", str(src), "-o", out, "-lm"])
    return out


def _run(lib):
    env = dict(os.environ, LD_PRELOAD=ASAN + ":" + UBSAN, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-c", _CHILD, lib], capture_output=True, text=True, timeout=600,
                          cwd=ROOT, env=env)


def test_pins_clean_under_sanitizers(tmp_path):
    with open(SRC) as f:
        lib = _build(f.read(), tmp_path, "oracle_san")
    proc = _run(lib)
    report = proc.stdout + proc.stderr
    assert proc.returncode == 0, report[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    passed = [ln for ln in proc.stdout.splitlines() if ln.startswith("PASS ")]
    caught = [ln for ln in proc.stdout.splitlines() if ln.startswith("CAUGHT ")]
    assert not caught, caught
    assert len(passed) >= 30, proc.stdout[-2000:]


def test_out_of_bounds_mutant_is_stopped(tmp_path):
    """The column-major scan order with w in place of h walks past the grid
    when w > h: the sanitizer aborts the child, or a pin fails first."""
    with open(SRC) as f:
        source = f.read()
    old, new = "default: return j * h + i;", "default: return j * w + i;"
    assert source.count(old) == 1
    lib = _build(source.replace(old, new), tmp_path, "mutant_san")
    proc = _run(lib)
    caught = [ln for ln in proc.stdout.splitlines() if ln.startswith("CAUGHT ")]
    assert proc.returncode != 0 or caught, "out-of-bounds mutant passed every pin under the sanitizers"
