"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(tests/sanitize/sa_host_check.cpp, built by sketch_attention_amd/build.py with
the host translation units instrumented): argument validation, status
strings and the error paths of every entry point, without a GPU.  A
sanitizer report aborts the program, so a zero exit status is the check."""
import os
import subprocess

import pytest

from sketch_attention_amd import build as B


def _exe():
    if not os.path.exists(B.HOST_CHECK):
        try:
            B.build_host_check()
        except RuntimeError as e:  # the library's device objects are not built here
            pytest.skip(f"host check not built: {e}")
    return B.HOST_CHECK


def test_host_code_under_sanitizers_validation_paths():
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([_exe(), "validate"], capture_output=True, text=True, timeout=300, env=env)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "0 failure(s)" in res.stdout
