"""The sustained-MFMA probe behind the GEMM roofline context (dory_test_mfma_rate) does
the work it reports: every work-group runs, and each thread's result equals the exact
value of its 8 accumulator chains (small dyadic operands, so fp32 sums are exact). The
operand layout of v_mfma_f32_32x32x16_bf16 used here: lane l holds row l % 32 of A and
column l % 32 of B at K elements 8 (l / 32) .. + 7; register r of the result is
C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]."""
import numpy as np
import pytest
import torch

from looped_ngpt_transformer_amd import dory as D

pytestmark = pytest.mark.gpu


def expected_sink(iters):
    t = np.arange(512)
    i = np.arange(8)
    a = ((t[:, None] * 7 + i[None, :] * 13) % 17 - 8) * 0.0625
    b = ((t[:, None] * 5 + i[None, :] * 11) % 19 - 9) * 0.03125
    out = np.zeros(512)
    for w in range(8):
        la, lb = a[64 * w: 64 * w + 64], b[64 * w: 64 * w + 64]
        A = np.zeros((32, 16))
        B = np.zeros((16, 32))
        for l in range(64):
            A[l % 32, 8 * (l // 32): 8 * (l // 32) + 8] = la[l]
            B[8 * (l // 32): 8 * (l // 32) + 8, l % 32] = lb[l]
        Cm = A @ B
        for l in range(64):
            rows = [8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)]
            out[64 * w + l] = 8 * iters * Cm[rows, l % 32].sum()
    return out


def test_mfma_rate_probe_does_its_work():
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    cyc = torch.zeros(n_cu, dtype=torch.int64, device="cuda")
    sink = torch.full((n_cu * 512,), float("nan"), dtype=torch.float32, device="cuda")
    n = D.dory_test_mfma_rate(10, cyc, sink)
    torch.cuda.synchronize()
    assert n == n_cu
    assert (cyc > 0).all()
    got = sink.cpu().double().numpy().reshape(n_cu, 512)
    exp = expected_sink(10)
    assert np.array_equal(got, np.broadcast_to(exp, got.shape))
    with pytest.raises(D.DoryError):
        D.dory_test_mfma_rate(0, cyc, sink)
