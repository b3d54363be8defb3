"""The host-side C-ABI tests (tests/test_abi.py) run again against the host
sanitizer build of the library (AddressSanitizer + UndefinedBehaviorSanitizer
on the host code, `python -m packed_varlen_attention_amd.build --sanitize`),
in a child process with the ASan runtime preloaded.  Any report (an
out-of-bounds host access, a misaligned load, an invalid enum value, signed
overflow, ...) aborts the child and fails this test.  CPU only: none of these
calls reaches the GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_tests_clean_under_host_sanitizers():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    from packed_varlen_attention_amd import build
    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env.update(H3_LIBRARY=lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "Sanitizer" not in out, out[-4000:]
    assert " passed" in out
