"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The argument validation of cca_api.hip is built with both sanitizers on its
host code (sparse_long_context_cca_amd.build.build_sanitized) and the ABI and
binding tests run against that build in a child process with the ASan runtime
preloaded (Python itself is not instrumented).  Any report -- an out-of-bounds
access, a load of an invalid enum value, a signed overflow -- stops the child
and fails this test; the reports go to log files under a temporary directory.
No kernel is launched: every call in those tests fails validation or stops
before the GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from sparse_long_context_cca_amd import build as cca_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_is_clean_under_host_sanitizers(tmp_path):
    if not os.path.exists(cca_build.HIPCC):
        pytest.skip("hipcc is not available")
    lib = cca_build.SAN_LIB
    if not os.path.exists(lib):
        lib = cca_build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": cca_build.sanitizer_runtime(),
        "ASAN_OPTIONS": f"detect_leaks=0:halt_on_error=1:log_path={tmp_path}/asan",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan",
        "CCA_LIB_PATH": lib,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_binding.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(glob.glob(f"{tmp_path}/asan*") + glob.glob(f"{tmp_path}/ubsan*"))
    text = "".join(open(p).read() for p in reports)
    assert not reports, f"sanitizer reports:\n{text[:4000]}"
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
