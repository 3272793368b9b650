"""The C ABI library on the CPU: it loads, exports what include/sa.h declares,
and its host-only validation behaves as documented.  No compute calls."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

from sketch_attention_amd import binding as B
from sketch_attention_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


def test_library_is_built_and_loads():
    assert os.path.exists(LIB_PATH), "run __graft_entry__.build() first"
    B.library()


def test_every_declared_symbol_is_exported():
    decl = _declared()
    assert {"sa_create", "sa_compress_batch", "sa_destroy"} <= set(decl)
    lib = ctypes.CDLL(LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name
    assert set(decl) == set(B.EXPORTED)
    # nothing else leaks out of the library under an sa_ name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {s for s in exported if s.startswith("sa_")} == set(decl)


def test_status_strings():
    assert B.sa_status_string(0) == "success"
    assert "invalid" in B.sa_status_string(1)
    assert "unsupported" in B.sa_status_string(2)
    assert "memory" in B.sa_status_string(3)
    assert "device" in B.sa_status_string(4).lower()
    assert B.sa_status_string(77) == "unknown status"


@pytest.mark.parametrize("d,k,tau,dtype,want", [
    (128, 256, 0.088, "bf16", B.SA_OK),
    (64, 1024, 0.125, "bf16", B.SA_OK),
    (64, 16, 0.125, "f32", B.SA_OK),
    (128, 1, 0.0, "bf16", B.SA_OK),
    (128, 512, -3.0, "bf16", B.SA_OK),
    (64, 256, 1.0, "f32", B.SA_OK),
    (128, 1024, 0.1, "bf16", B.SA_OK),                # two-phase pass (blocks of 256 prototypes)
    (128, 513, 0.1, "bf16", B.SA_OK),
    (128, 1025, 0.1, "bf16", B.SA_ERR_UNSUPPORTED),
    (64, 1025, 0.1, "bf16", B.SA_ERR_UNSUPPORTED),
    (64, 257, 0.1, "f32", B.SA_OK),                   # float32 in two phases beyond 256 prototypes
    (128, 1024, 0.1, "f32", B.SA_OK),
    (128, 1025, 0.1, "f32", B.SA_ERR_UNSUPPORTED),
    (96, 16, 0.1, "bf16", B.SA_ERR_UNSUPPORTED),
    (256, 16, 0.1, "bf16", B.SA_ERR_UNSUPPORTED),
    (128, 0, 0.1, "bf16", B.SA_ERR_INVALID_ARG),
    (0, 4, 0.1, "bf16", B.SA_ERR_INVALID_ARG),
    (128, 4, math.inf, "bf16", B.SA_ERR_INVALID_ARG),
    (128, 4, math.nan, "bf16", B.SA_ERR_INVALID_ARG),
    (128, 4, 0.1, "f16", B.SA_ERR_INVALID_ARG),
])
def test_check_config(d, k, tau, dtype, want):
    assert B.sa_check_config(d, k, tau, dtype) == want


@pytest.mark.parametrize("offsets,want", [
    ([0], B.SA_OK),
    ([0, 0, 0], B.SA_OK),
    ([0, 5, 5, 100000], B.SA_OK),
    ([1, 5], B.SA_ERR_INVALID_ARG),
    ([0, 5, 4], B.SA_ERR_INVALID_ARG),
    ([0, -1], B.SA_ERR_INVALID_ARG),
    ([0, 2 ** 41], B.SA_ERR_INVALID_ARG),
    ([0, 2 ** 31 - 1], B.SA_OK),                 # the largest batch (a work group's rows in 32-bit offsets)
    ([0, 2 ** 30, 2 ** 31], B.SA_ERR_INVALID_ARG),
])
def test_check_batch(offsets, want):
    assert B.sa_check_batch(16, np.array(offsets, dtype=np.int64)) == want


def test_check_batch_rejects_bad_k_and_negative_users():
    lib = B.library()
    offs = np.zeros(1, dtype=np.int64)
    assert lib.sa_check_batch(0, B._i64_ptr(offs), 0) == B.SA_ERR_INVALID_ARG
    assert lib.sa_check_batch(4, B._i64_ptr(offs), -1) == B.SA_ERR_INVALID_ARG
    assert lib.sa_check_batch(4, None, 3) == B.SA_ERR_INVALID_ARG


def test_null_handle_paths_return_errors_without_device_work():
    lib = B.library()
    offs = np.array([0, 4], dtype=np.int64)
    assert lib.sa_compress_batch(None, None, B._i64_ptr(offs), 1, None, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_create(None, 128, 16, ctypes.c_float(0.1), 1, None, None, None, None) == B.SA_ERR_INVALID_ARG
    h = ctypes.c_void_p(1234)
    # config errors are reported before any pointer is touched, and the handle is cleared
    assert lib.sa_create(ctypes.byref(h), 96, 16, ctypes.c_float(0.1), 1, None, None, None, None) == B.SA_ERR_UNSUPPORTED
    assert h.value is None
    assert lib.sa_create(ctypes.byref(h), 128, 16, ctypes.c_float(0.1), 1, None, None, None, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_set_kernel_timing(None, 1) == B.SA_ERR_INVALID_ARG
    assert lib.sa_get_folded(None, None, None) == B.SA_ERR_INVALID_ARG
    lib.sa_destroy(None)  # NULL-safe


def test_create_ex_validates_before_device_work():
    lib = B.library()
    f = ctypes.c_float(0.1)
    h = ctypes.c_void_p(77)
    assert lib.sa_create_ex(None, 128, 16, f, 1, None, None, None, 1, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_create_ex(ctypes.byref(h), 128, 16, f, 1, None, None, None, 7, None) == B.SA_ERR_INVALID_ARG
    assert h.value is None
    # the comparator takes both dtypes: with null weights, float32 fails on the arguments, not the dtype
    assert lib.sa_create_ex(ctypes.byref(h), 128, 16, f, 0, None, None, None, 1, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_create_ex(ctypes.byref(h), 96, 16, f, 1, None, None, None, 1, None) == B.SA_ERR_UNSUPPORTED


def test_stack_entry_points_validate_before_device_work():
    lib = B.library()
    f = ctypes.c_float(0.1)
    h = ctypes.c_void_p(99)
    params = (B.sa_layer_params * 2)()
    assert lib.sa_stack_create(None, 128, 16, 256, 2, f, 1, None, params, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_stack_create(ctypes.byref(h), 96, 16, 256, 2, f, 1, None, params, None) == B.SA_ERR_UNSUPPORTED
    assert h.value is None
    assert lib.sa_stack_create(ctypes.byref(h), 128, 16, 256, 0, f, 1, ctypes.c_void_p(16), params, None) == \
        B.SA_ERR_INVALID_ARG
    assert lib.sa_stack_create(ctypes.byref(h), 128, 16, 256, 2, f, 1, ctypes.c_void_p(16), None, None) == \
        B.SA_ERR_INVALID_ARG
    assert lib.sa_stack_create(ctypes.byref(h), 128, 16, 100, 2, f, 1, ctypes.c_void_p(16), params, None) == \
        B.SA_ERR_UNSUPPORTED
    # null layer pointers are rejected before anything is allocated
    assert lib.sa_stack_create(ctypes.byref(h), 128, 16, 256, 2, f, 1, ctypes.c_void_p(16), params, None) == \
        B.SA_ERR_INVALID_ARG
    offs = np.array([0, 4], dtype=np.int64)
    assert lib.sa_stack_compress_batch(None, None, offs.ctypes.data, 1, None, None) == B.SA_ERR_INVALID_ARG
    lib.sa_stack_destroy(None)  # NULL-safe


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.library()


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "sketch_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f"{f} imports the oracle"
                assert "oracle/" not in text and "sa_oracle" not in text, f"{f} reaches into the oracle"


def test_grad_entry_points_validate_before_device_work():
    lib = B.library()
    assert lib.sa_grad_check_config(128, 256, 0.1, B.SA_BF16) == B.SA_OK
    assert lib.sa_grad_check_config(64, 1, 0.1, B.SA_BF16) == B.SA_OK
    assert lib.sa_grad_check_config(128, 257, 0.1, B.SA_BF16) == B.SA_OK
    assert lib.sa_grad_check_config(128, 1024, 0.1, B.SA_BF16) == B.SA_OK
    assert lib.sa_grad_check_config(64, 1000, 0.1, B.SA_BF16) == B.SA_OK
    assert lib.sa_grad_check_config(128, 1025, 0.1, B.SA_BF16) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_grad_check_config(128, 64, 0.1, B.SA_F32) == B.SA_OK
    assert lib.sa_grad_check_config(64, 1024, 0.1, B.SA_F32) == B.SA_OK
    assert lib.sa_grad_check_config(128, 1025, 0.1, B.SA_F32) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_grad_check_config(96, 64, 0.1, B.SA_BF16) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_grad_check_config(128, 0, 0.1, B.SA_BF16) == B.SA_ERR_INVALID_ARG
    assert lib.sa_grad_check_config(128, 64, float("nan"), B.SA_BF16) == B.SA_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.sa_grad_create(ctypes.byref(h), 128, 64, 0.1, B.SA_BF16, None, None, None, None) == \
        B.SA_ERR_INVALID_ARG
    assert lib.sa_grad_create(None, 128, 64, 0.1, B.SA_BF16, None, None, None, None) == B.SA_ERR_INVALID_ARG
    offs = np.array([0, 4], dtype=np.int64)
    assert lib.sa_grad_compute(None, None, offs.ctypes.data, 1, None, None, None, None, None, None) == \
        B.SA_ERR_INVALID_ARG
    f, g, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    assert lib.sa_grad_read_kernel_timing(None, ctypes.byref(f), ctypes.byref(g), ctypes.byref(n)) == \
        B.SA_ERR_INVALID_ARG
    assert lib.sa_grad_set_kernel_timing(None, 1) == B.SA_ERR_INVALID_ARG
    lib.sa_grad_destroy(None)


def test_action_entry_points_validate_before_device_work():
    lib = B.library()
    ok = B.SA_OK
    assert lib.sa_action_check_config(128, 64, 256, 8, B.SA_BF16) == ok
    assert lib.sa_action_check_config(128, 0, 64, 1, B.SA_BF16) == ok
    assert lib.sa_action_check_config(64, 192, 128, 4, B.SA_BF16) == ok
    assert lib.sa_action_check_config(128, 128, 32, 4, B.SA_BF16) == ok       # d + d_a = 256: chunks of 32
    assert lib.sa_action_check_config(128, 64, 32, 4, B.SA_BF16) == B.SA_ERR_UNSUPPORTED  # needs a multiple of 64
    assert lib.sa_action_check_config(128, 136, 64, 4, B.SA_BF16) == B.SA_ERR_UNSUPPORTED  # d + d_a > 256
    assert lib.sa_action_check_config(128, 12, 64, 4, B.SA_BF16) == B.SA_ERR_UNSUPPORTED   # d_a % 8
    assert lib.sa_action_check_config(96, 32, 64, 4, B.SA_BF16) == B.SA_ERR_UNSUPPORTED
    # float32: d_ff a multiple of 32, the same d, d_a and K limits
    assert lib.sa_action_check_config(128, 32, 64, 4, B.SA_F32) == ok
    assert lib.sa_action_check_config(64, 8, 96, 4, B.SA_F32) == ok
    assert lib.sa_action_check_config(128, 32, 48, 4, B.SA_F32) == B.SA_ERR_UNSUPPORTED   # d_ff % 32
    assert lib.sa_action_check_config(128, 136, 64, 4, B.SA_F32) == B.SA_ERR_UNSUPPORTED  # d + d_a > 256
    assert lib.sa_action_check_config(96, 32, 64, 4, B.SA_F32) == B.SA_ERR_UNSUPPORTED
    assert lib.sa_action_check_config(128, 32, 64, 0, B.SA_BF16) == B.SA_ERR_INVALID_ARG
    assert lib.sa_action_check_config(128, -8, 64, 4, B.SA_BF16) == B.SA_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.sa_action_create(ctypes.byref(h), 128, 32, 64, 4, B.SA_BF16, None, None, None, None, None) == \
        B.SA_ERR_INVALID_ARG
    assert lib.sa_action_fuse(None, None, None, 10, None, None) == B.SA_ERR_INVALID_ARG
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.sa_action_read_kernel_timing(None, ctypes.byref(ms), ctypes.byref(n)) == B.SA_ERR_INVALID_ARG
    lib.sa_action_destroy(None)


def test_reserve_rejects_a_null_handle_and_bad_bounds():
    lib = B.library()
    assert lib.sa_reserve(None, 100, 2, 1, None) == B.SA_ERR_INVALID_ARG


def test_action_compress_rejects_null_handles():
    lib = B.library()
    offs = (ctypes.c_int64 * 2)(0, 0)
    assert lib.sa_action_compress_batch(None, None, None, None, offs, 1, None, None) == B.SA_ERR_INVALID_ARG
