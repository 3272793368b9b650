"""On-device ceilings (include/sa.h sa_measure_ceilings, sa_measure_hbm_read):
every figure is positive and below what any MI355X part can deliver, so a
broken timing (zero or negative elapsed time, a loop the compiler removed)
shows up as a failure rather than as a wrong roofline denominator."""
import pytest
import torch

from sketch_attention_amd import binding

pytestmark = pytest.mark.gpu


def test_hbm_read_ceiling_is_plausible():
    gbs = binding.sa_measure_hbm_read()
    # a read-only stream over 1 GiB: well above PCIe, below the 8 TB/s of the HBM3E stacks
    assert 500.0 < gbs < 8000.0, gbs


def test_ceilings_are_plausible():
    c = binding.sa_measure_ceilings()
    assert 100.0 < c["mfma_bf16_tflops"] < 2600.0
    assert 100.0 < c["mfma_bf16_32x32_tflops"] < 2600.0
    assert 10.0 < c["valu_fma_tflops"] < 160.0
    assert 1e12 < c["exp2_per_sec"] < 1e14
    assert 500.0 < c["copy_gbs"] < 8000.0
    torch.cuda.synchronize()
