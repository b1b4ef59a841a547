"""The oracle's pins again, on a build of the oracle instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (every finding fatal), in a
child process that loads the ASan runtime first.  An out-of-bounds index into
the flat arrays the oracle walks (by T, k, E, H, I and the group count), a
use after free or undefined arithmetic makes the child fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import build as ob

    lib = ob.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, MOE_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
