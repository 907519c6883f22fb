"""CPU: the oracle's pins again, against an AddressSanitizer +
UndefinedBehaviorSanitizer build of oracle.c (every finding fatal), so an
out-of-bounds access, a use after free or undefined arithmetic in the oracle
fails the suite even where the pins' values would still come out right."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _libasan():
    if shutil.which("gcc") is None:
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not available")
    lib = oracle.build(path=str(tmp_path / "liboracle_sanitized.so"), sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ORACLE_LIBRARY=lib, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           "-m", "not gpu", os.path.join(HERE, "test_oracle.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
