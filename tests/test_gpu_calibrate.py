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


def test_clock_stamps_cover_every_xcd_and_give_a_plausible_clock():
    import numpy as np
    nb = c3d.conv3d_clock_stamp_bytes()
    before = torch.zeros(nb, dtype=torch.uint8, device="cuda:0")
    after = torch.zeros_like(before)
    scratch = torch.empty(c3d.conv3d_calibrate_scratch_bytes(), dtype=torch.uint8, device="cuda:0")
    c3d.conv3d_clock_stamp(before)
    _, cal_mhz = c3d.conv3d_calibrate_mfma(scratch)   # a few ms of MFMA load between the stamps (synchronises)
    c3d.conv3d_clock_stamp(after)
    torch.cuda.synchronize()
    b = before.cpu().numpy().view(np.uint64).reshape(-1, 3)
    a = after.cpu().numpy().view(np.uint64).reshape(-1, 3)
    assert sorted(set((b[:, 2] & 0xF).tolist())) == list(range(8)) == sorted(set((a[:, 2] & 0xF).tolist()))
    # nearly every CU (8 XCDs x 32) is stamped both times
    assert len(set(b[:, 2].tolist()) & set(a[:, 2].tolist())) >= 200
    mhz = c3d.sclk_between(b.reshape(-1), a.reshape(-1))
    assert sorted(mhz) == list(range(8))
    assert all(500.0 < v < 2600.0 for v in mhz.values()), mhz
    # The XCDs clock independently (up to about 12% apart under this load), but
    # CU-paired figures stay close together and close to the clock the
    # calibration kernel measures inside its own waves; stamps paired across
    # CUs had given figures a factor of two apart
    assert max(mhz.values()) < 1.3 * min(mhz.values()), mhz
    mean = sum(mhz.values()) / len(mhz)
    assert abs(mean - cal_mhz) < 0.15 * cal_mhz, (mhz, cal_mhz)
