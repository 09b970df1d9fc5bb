"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host side of the library with both sanitizers
(reverse_selective_scan_amd/build_sanitized.py: argument checks, workspace
planning and launch code; the device code is the usual one) and runs the host API tests
(tests/test_api_host.py: every entry point's error paths, the workspace
queries, the exported symbols) against that build in a child process with the
ASan runtime preloaded.  Any sanitizer report aborts the child and fails this
test.  (The oracle is numpy and Python only: it has no native code of its
own to instrument.)"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None, reason="hipcc not found")
def test_host_api_under_asan_and_ubsan():
    from reverse_selective_scan_amd import build_sanitized as S

    lib = S.build(verbose=False)
    env = dict(os.environ)
    env.update({
        "R2L_LIB": lib,
        "LD_PRELOAD": S.asan_runtime(),
        # leaks: the interpreter and torch allocate for the whole process
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "HIP_VISIBLE_DEVICES": "",   # host paths only, also on a machine with a GPU
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_api_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out
