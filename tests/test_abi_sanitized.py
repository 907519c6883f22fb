"""CPU: the host tests of the C ABI again, against a build whose host code
(abi.cpp: argument checks, workspace sizing, dispatch) carries
AddressSanitizer and UndefinedBehaviorSanitizer, every finding fatal.  The
sanitized library is removed afterwards."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_abi_host_tests_under_asan_and_ubsan():
    from paged_kv_attention_24_amd import _build

    if not os.path.exists(_build.HIPCC) or shutil.which("gcc") is None:
        pytest.skip("hipcc is not available")
    rt = _build.asan_runtime()
    if not rt:
        pytest.skip("clang's ASan runtime is not available")
    lib = _build.build_sanitized()
    try:
        env = dict(os.environ)
        env.update(PKA_LIBRARY=os.path.basename(lib), LD_PRELOAD=rt,
                   ASAN_OPTIONS="detect_leaks=0:exitcode=86",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
        cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
               "-m", "not gpu", os.path.join(HERE, "test_abi_host.py")]
        r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        tail = (r.stdout + r.stderr)[-4000:]
        assert r.returncode == 0, tail
        assert " passed" in r.stdout, tail
    finally:
        os.remove(lib)
