"""Device-assembly checks of the kernels that stage tiles by LDS DMA (CPU only:
hipcc cross-compiles for gfx950).

The DMA helper writes M0 in inline assembly and declares it clobbered.  The
compiler does not save or restore a reserved register around inline assembly,
so the helper is only sound while the compiler itself keeps no value in M0
across it.  This test compiles every translation unit that uses the helper to
gfx950 assembly with the library's own flags and checks that each reference to
M0 is one of the helpers' sequence: the move of the LDS address into M0, then
the global_load_lds_dwordx4 (or, for the per-row statistics of the two-phase
pass, global_load_lds_dword) that reads it.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from sketch_attention_amd import build as B

DMA_UNITS = ["sa_stream_d64.hip", "sa_stream_d128.hip", "sa_grad.hip", "sa_action.hip"]


def _device_asm(unit: str, out_dir: str) -> str:
    out = os.path.join(out_dir, unit + ".s")
    extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if unit in B.VGPR_FORM else []
    subprocess.run([B.hipcc(), *B.HIPCC_FLAGS, *extra, "--cuda-device-only", "-S", "-o", out,
                    os.path.join(B.CSRC, unit)], check=True, capture_output=True)
    with open(out) as fh:
        return fh.read()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_m0_is_written_only_by_the_dma_helper(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(len(DMA_UNITS)) as ex:
        asms = dict(zip(DMA_UNITS, ex.map(lambda u: _device_asm(u, str(tmp_path)), DMA_UNITS)))
    for unit, asm in asms.items():
        lines = [l.split(";")[0].strip() for l in asm.splitlines()]
        lines = [l for l in lines if l and not l.startswith(".")]
        dmas = 0
        for i, l in enumerate(lines):
            if not re.search(r"\bm0\b", l):
                continue
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), (unit, l)
            # the helpers: s_mov_b32 m0, sN ; s_nop 0 ; global_load_lds_dword[x4] v, s[..]
            assert lines[i + 1] == "s_nop 0" and re.match(r"global_load_lds_dword(x4)? ", lines[i + 2]), (
                unit, lines[i:i + 3])
            dmas += 1
        n_lds = sum(1 for l in lines if l.startswith("global_load_lds_dword"))
        assert dmas > 0 and n_lds == dmas, (unit, dmas, n_lds)
