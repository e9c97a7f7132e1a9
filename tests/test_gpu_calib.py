"""The calibration copy kernel reproduces its source byte for byte (it sets
the counter scale factor of the roofline measurement, so it must move exactly
the bytes it claims)."""
import pytest
import torch

import pooled_selective_state_amd as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_floats", [4, 1020, 4096, 4096 * 257 + 12])
def test_calib_copy_exact(n_floats):
    g = torch.Generator(device="cuda").manual_seed(n_floats)
    src = torch.randn(n_floats, device="cuda", generator=g)
    dst = torch.full_like(src, float("nan"))
    P.calib_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_calib_copy_leaves_neighbours():
    """Only the requested bytes are written."""
    buf = torch.zeros(8192 + 64, device="cuda")
    src = torch.ones(4096 + 8, device="cuda")
    P.calib_copy(buf[16:16 + src.numel()], src)
    torch.cuda.synchronize()
    h = buf.cpu()
    assert torch.all(h[:16] == 0) and torch.all(h[16:16 + src.numel()] == 1) and torch.all(h[16 + src.numel():] == 0)
