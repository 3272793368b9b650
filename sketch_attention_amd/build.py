"""Build the HIP library libsa.so in-tree for gfx950 with hipcc.

The library is compiled on the CPU (hipcc cross-compiles for gfx950) and
placed next to the binding at sketch_attention_amd/_lib/libsa.so.  Objects go
to _build/ at the repository root.  Translation units compile in parallel.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG_DIR, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libsa.so")

ARCH = "gfx950"
SOURCES = [
    "sa_api.cpp",
    "sa_kernels.hip",
    "sa_fused_bf16_d64.hip",
    "sa_fused_bf16_d128.hip",
    "sa_fused_f32_d64.hip",
    "sa_fused_f32_d128.hip",
    "sa_stream_d64.hip",
    "sa_stream_d128.hip",
    "sa_refine.hip",
    "sa_grad.hip",
    "sa_grad_f32.hip",
    "sa_grad_api.cpp",
    "sa_action.hip",
    "sa_action_sa.hip",
    "sa_action_api.cpp",
    "sa_ceilings.hip",
]
# The bf16 plans (accumulators of at most 128 registers per lane) keep every
# matrix-core result in VGPRs, so the softmax reads the affinity tile without
# AGPR moves.
VGPR_FORM = {"sa_fused_bf16_d64.hip", "sa_fused_bf16_d128.hip", "sa_stream_d64.hip", "sa_stream_d128.hip"}
# Packed fp32 VALU instructions are disabled for all device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines() if "is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every translation unit and link libsa.so; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src in VGPR_FORM else []
        cmds.append([cc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for fut in [ex.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side sanitizer check (tests/sanitize/sa_host_check.cpp): the library's
# host translation units and the driver are built with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host side only (each -fsanitize= behind
# -Xarch_host), then linked with the library's unsanitized device objects.
HOST_SOURCES = ["sa_api.cpp", "sa_grad_api.cpp", "sa_action_api.cpp"]
HOST_CHECK = os.path.join(LIB_DIR, "sa_host_check")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def build_host_check(verbose: bool = False) -> str:
    """The sanitized host-check executable; needs the device objects of build_library."""
    cc = hipcc()
    san_dir = os.path.join(BUILD_DIR, "sanitize")
    os.makedirs(san_dir, exist_ok=True)
    objs, cmds = [], []
    driver = os.path.join(ROOT, "tests", "sanitize", "sa_host_check.cpp")
    for src in HOST_SOURCES + [driver]:
        obj = os.path.join(san_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
        objs.append(obj)
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        cmds.append([cc, *HIPCC_FLAGS, *SANITIZE, "-c", path, "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for fut in [ex.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    dev_objs = [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES if src.endswith(".hip")]
    for o in dev_objs:
        if not os.path.exists(o):
            raise RuntimeError(f"missing {o}: build the library first")
    tmp = HOST_CHECK + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", *SANITIZE, "-o", tmp, *objs, *dev_objs], verbose)
    os.replace(tmp, HOST_CHECK)
    return HOST_CHECK


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
