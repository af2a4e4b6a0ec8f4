"""GPU: the NVFP4 (W4A16) path through the C ABI. The quantiser must match the oracle's
codes, block scales and matrix scale bit for bit (its scale choice is an integer taken
by float32 comparisons in a fixed order on both sides)."""
import numpy as np
import pytest
import torch

from looped_ngpt_transformer_amd import dory as D
from oracle import nvfp4 as NV

pytestmark = pytest.mark.gpu


def quantize_gpu(w):
    rows, cols = w.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty((1,), dtype=torch.float32, device="cuda")
    D.dory_quantize_nvfp4(w, codes, scales, g)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), float(g.cpu()[0])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,std", [((64, 256), 0.02), ((33, 160), 1.0), ((8, 4096), 3e-4)])
def test_quantiser_bit_exact(dtype, shape, std):
    g = torch.Generator().manual_seed(shape[0] * 7 + shape[1])
    w = torch.randn(shape, generator=g) * std
    w[0, :16] = 0.0                       # all-zero block
    w[1, 16:32] = w[1, 16]                # constant block
    w[2, 5] = 40 * std                    # an outlier in its block
    w = w.to(dtype)
    c, s, gs = quantize_gpu(w.cuda())
    wc, ws, wg = NV.quantize(w.float().numpy())
    assert gs == float(wg)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(c, wc)


def test_quantiser_all_zero_matrix():
    c, s, gs = quantize_gpu(torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda"))
    assert gs == 1.0 and np.all(c == 0) and np.all(s == 1)
