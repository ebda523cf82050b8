"""Host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every library source together with tests/host_sanitize/abi_checks.cpp
(hipcc; the sanitizers instrument the host code only) and runs the program on
the CPU: each entry point is called with invalid arguments, empty shapes and
sizes beyond the documented launch limits, and must return its documented
status from the host checks with no sanitizer report.  No kernel is launched.
"""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "precision_mxfp4_producers_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_checks_clean_under_asan_ubsan():
    from precision_mxfp4_producers_amd.build import SOURCES
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests", "host_sanitize", "abi_checks.cpp")]
    tmp = tempfile.mkdtemp(prefix="mxfp4_san_")
    try:
        exe = os.path.join(tmp, "abi_checks")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer"] + srcs + ["-o", exe]
        b = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
        assert b.returncode == 0, b.stdout.decode()[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env, timeout=120)
        out = r.stdout.decode()
        assert r.returncode == 0, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
        assert "abi_checks: 0 failure(s)" in out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
