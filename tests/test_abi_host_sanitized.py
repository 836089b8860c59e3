"""The host ABI tests (tests/test_abi_host.py) once more, against the build of
the library whose host code -- argument validation, size queries, buffer
layouts and launch sequences -- is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (libmtnlg_hostsan.so, made by build()). They run in
a child process with the sanitizer runtime preloaded; any report fails the
child. No GPU is needed: those tests only reach validation paths.
"""
import os
import subprocess
import sys

import pytest

from tensor_sliced_transformer_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(B.SAN_LIB), reason="libmtnlg_hostsan.so not built (__graft_entry__.build())")
def test_host_abi_under_address_and_undefined_behaviour_sanitizers():
    env = dict(os.environ)
    env["MTNLG_LIBRARY"] = B.SAN_LIB
    env["LD_PRELOAD"] = B.sanitizer_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
