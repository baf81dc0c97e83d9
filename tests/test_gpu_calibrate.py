"""The measurement aids run and report plausible machine ceilings (through the C ABI)."""
import pytest
import torch

import convolution_implicit_gemm_amd as c3d

pytestmark = pytest.mark.gpu


def test_mfma_calibration_reports_plausible_rate_and_clock():
    scratch = torch.empty(c3d.conv3d_calibrate_scratch_bytes(), dtype=torch.uint8, device="cuda:0")
    tflops, mhz = c3d.conv3d_calibrate_mfma(scratch)
    # dense fp16 peak is 2516.6 TFLOP/s at 2400 MHz; power limits both below that
    assert 300.0 < tflops < 2600.0
    assert 500.0 < mhz < 2600.0


def test_hbm_calibration_reports_plausible_bandwidth():
    nb = 512 << 20
    src = torch.ones(nb, dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros_like(src)
    rd, cp = c3d.conv3d_calibrate_hbm(src, dst, nb)
    assert 1000.0 < rd < 12000.0 and 1000.0 < cp < 12000.0
    assert torch.equal(dst[:4096], src[:4096]) and torch.equal(dst[-4096:], src[-4096:])
