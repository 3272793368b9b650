"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
on a GPU (tests/sanitize/sa_host_check.cpp in `full` mode): create, compute and
destroy through the compression (both entry points, ragged batches with empty
users, more users than one launch, the two-phase prototype counts) and the
backward, checking statuses and the mass identity, then the float32
comparator, backward and action fusion; the device code is the library's
own.  A sanitizer report aborts the program."""
import os
import subprocess

import pytest

from sketch_attention_amd import build as B

pytestmark = pytest.mark.gpu


def test_host_code_under_sanitizers_on_device():
    assert os.path.exists(B.HOST_CHECK), "build the host check first (__graft_entry__.build())"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([B.HOST_CHECK, "full"], capture_output=True, text=True, timeout=600, env=env)
    print(res.stdout, res.stderr[-4000:])
    assert res.returncode == 0, res.stderr[-4000:]
    assert "0 failure(s)" in res.stdout
