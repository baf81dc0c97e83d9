"""The binding refuses tensors the C layer cannot check: wrong dtype, too few elements."""
import pytest
import torch

import convolution_implicit_gemm_amd as c3d

pytestmark = pytest.mark.gpu


def test_conv_binding_checks_dtype_and_size_before_the_call():
    d = c3d.make_desc(1, 4, 8, 8, 16, 16, 3, 3, 3, 2, 0, 1, 1, c3d.CONV3D_TPAD_REPLICATE, c3d.CONV3D_F_BIAS)
    p = c3d.conv3d_plan(d)
    x = torch.zeros(1, 4, 8, 8, 16, dtype=torch.float16, device="cuda:0")
    w = torch.zeros(16, 3, 3, 3, 16, dtype=torch.float16, device="cuda:0")
    b = torch.zeros(16, dtype=torch.float16, device="cuda:0")
    y = torch.empty(1, 4, 8, 8, 16, dtype=torch.float16, device="cuda:0")
    with pytest.raises(c3d.Conv3dError, match="x is torch.bfloat16"):
        c3d.conv3d_forward(p, x.view(torch.bfloat16), w, b, None, y)
    with pytest.raises(c3d.Conv3dError, match="y holds 1024 elements, 4096 needed"):
        c3d.conv3d_forward(p, x, w, b, None, y[:, :1].contiguous())
    with pytest.raises(c3d.Conv3dError, match="weight holds"):
        c3d.conv3d_forward(p, x, w[:8], b, None, y)
    c3d.conv3d_forward(p, x, w, b, None, y)       # the right tensors pass
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_groupnorm_binding_checks_dtype_and_size():
    x = torch.zeros(1, 64, 16, dtype=torch.float16, device="cuda:0")
    g = torch.ones(16, dtype=torch.float16, device="cuda:0")
    ws = torch.zeros(c3d.groupnorm_silu_workspace(1, 64, 16, 2), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(c3d.Conv3dError, match="beta holds 8 elements"):
        c3d.groupnorm_silu(x, g, g[:8], x, 1, 64, 16, 2, 1e-6, True, ws)
    with pytest.raises(c3d.Conv3dError, match="is torch.float16, the plan expects torch.bfloat16"):
        c3d.groupnorm_silu_bf16(x, g, g, x, 1, 64, 16, 2, 1e-6, True, ws)
