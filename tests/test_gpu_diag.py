"""The diagnostic entry points on the GPU: the streaming copy (ragged tail included) and the
L2-resident read, whose single store happens only when its sum is -1."""
import pytest
import torch

from multiresolution_hash_grid_multires_amd import api

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("n", [1, 3, 4, 1000, (1 << 20) + 7])
def test_copy_is_exact(n):
    src = torch.randn(n, device=DEV)
    dst = torch.full((n,), float("nan"), device=DEV)
    api.hashenc_diag_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_cache_read_reads_every_pass():
    n = 32 * 4096
    out = torch.full((1,), 7.0, device=DEV)
    ones = torch.ones(n, device=DEV)
    api.hashenc_diag_cache_read(ones, 3, out)
    torch.cuda.synchronize()
    assert out.item() == 7.0  # a buffer of ones never sums to -1
    buf = torch.zeros(n, device=DEV)
    buf[0] = -1.0  # read by one lane: its sum is -1 per pass
    api.hashenc_diag_cache_read(buf, 1, out)
    torch.cuda.synchronize()
    assert out.item() == -1.0
    out.fill_(7.0)
    api.hashenc_diag_cache_read(buf, 2, out)  # two passes: -2, no store
    torch.cuda.synchronize()
    assert out.item() == 7.0
