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


# forward parity with NVFP4 weights: the oracle runs on the dequantised codes its own
# quantiser produces from the same bf16 weights (bit-identical codes, checked above). The
# oracle's exhaustive float32 scale search is slow in NumPy, so the forward tests use a
# narrow bf16 layer shape that routes to the same kernels: hidden 512, 4/1 heads of 128,
# SwiGLU 1024, [q|k|v|gate] 1280 rows, one layer per block, window 64.
from tests.test_gpu_parity import _run_case, xin  # noqa: E402
import synth  # noqa: E402

NSMALL = dict(synth.config("P", n_in=1, n_rec=1, n_out=1, window=64), hidden=512, n_q_heads=4, n_kv_heads=1,
              head_dim=128, intermediate=1024, attn_scale=128 ** 0.5, weight_format="nvfp4")


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_nvfp4_small_forward(mode):
    """A 300-row prefill (the large-M GEMMs on matrices expanded to bf16), a 100-row chunk
    and two decode steps (the 4-bit split-K tiles), with undamped rates."""
    S = NSMALL
    sched = [("prefill", [(0, xin(S, 300, 41))]),
             ("prefill", [(0, xin(S, 100, 44))]),
             ("decode", [(0, xin(S, 1, 42))]),
             ("decode", [(0, xin(S, 1, 43))])]
    _run_case(S, 2, mode, sched, max_rows=320, max_seq_len=512, max_seqs=1, sharp=True)


@pytest.mark.parametrize("batch", [1, 40, 128])
def test_nvfp4_decode_batches(batch):
    """NVFP4 weights at decode batch sizes (split-K tiles of 32 and 64 rows): prefill
    `batch` short sequences in one call, then one decode step for all of them."""
    S = NSMALL
    sched = [("prefill", [(i, xin(S, 2 + i % 3, 700 + i)) for i in range(batch)]),
             ("decode", [(i, xin(S, 1, 900 + i)) for i in range(batch)])]
    _run_case(S, 2, "last_loop", sched, max_rows=512, max_seq_len=16, max_seqs=batch, sharp=True)
