"""The CPU checks of the C ABI (test_abi.py) rerun against a build of the
library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer.

The run happens in a child process that preloads the ASan runtime (Python
itself is not instrumented, so the runtime has to come first in the process)
and points the binding at the sanitized library. Any heap or stack overflow,
use after free, signed overflow, bad shift, misaligned access or other
undefined behaviour in the boundary's host code then ends the child with a
report, which fails this test. No GPU is used: every call in test_abi.py is
rejected, or is an empty no-op, before a HIP call is made."""
import os
import subprocess
import sys

import pytest

from exact_attention_122_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_library():
    try:
        runtime = build.asan_runtime()
        lib = build.build_host_sanitized()
    except RuntimeError as e:
        pytest.skip(f"no sanitized build: {e}")
    return lib, runtime


def test_sanitized_library_is_instrumented(sanitized_library):
    lib, _ = sanitized_library
    blob = open(lib, "rb").read()
    assert b"__asan_report" in blob and b"__ubsan_handle" in blob


def test_abi_checks_pass_under_asan_and_ubsan(sanitized_library):
    lib, runtime = sanitized_library
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "FA_TEST_LIBRARY": lib,
        # Python's own allocations are not freed at exit; leaks are not what is checked
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
           "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert f"[library] {lib}" in out, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, out[-4000:]
