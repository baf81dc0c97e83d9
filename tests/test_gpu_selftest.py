"""The library's start-up self-test (conv3d_selftest) on the GPU, in process and in a child process."""
import pytest

import convolution_implicit_gemm_amd as c3d

pytestmark = pytest.mark.gpu


def test_selftest_passes():
    rc = c3d.conv3d_selftest()
    assert rc == 0, (rc, c3d.conv3d_last_error())
    assert c3d.conv3d_last_error() == ""


def test_selftest_in_a_subprocess_passes():
    assert c3d.selftest_in_subprocess(timeout=240) == 0
