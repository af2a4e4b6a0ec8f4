"""GPU: the projection GEMM kernels through the C ABI (dory_test_gemm), each shape routed
to the kernel a layer call would use, against a plain float32 matmul of the same bf16
(or dequantised MXFP8) operands. Shapes cover the 256x256 ping-pong tiles (every
epilogue, ragged M, row stride > K), the 256x160 tiles, launches that split the columns
between the two, and the split-K decode kernels.

Tolerances: float outputs |d| <= 2e-3 * (|ref| + 1) (bf16 products, float32 sums in
another order over K <= 4096 terms of size ~0.02); bf16 outputs additionally one
rounding of the output (2^-8 relative)."""
import pytest
import torch

from looped_ngpt_transformer_amd import dory as D

pytestmark = pytest.mark.gpu

SENTINEL = 8192.0  # exact in bf16 and float32


def operands(M, N, K, seed, lda=None):
    g = torch.Generator(device="cpu").manual_seed(seed)
    lda = lda or K
    Abig = torch.randn(M, lda, generator=g).to(torch.bfloat16).cuda()
    B = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).cuda()
    return Abig[:, :K], B


def reference(A, B):
    return A.float() @ B.float().t()


def check(out, ref, bf16_out):
    tol = 2e-3 * (ref.abs() + 1.0)
    if bf16_out:
        tol = tol + ref.abs() * 2.0 ** -8
    d = (out.float() - ref).abs()
    bad = d > tol
    assert not bad.any(), f"{int(bad.sum())} outside tolerance, max |d| {float(d.max()):.3e}"


@pytest.mark.parametrize("M,N,K,lda,ldc", [
    (2600, 6400, 2560, None, None),   # [q|k|v|gate] shape: 15 wide + 16 narrow column tiles, ragged M
    (4096, 6400, 2560, 2624, None),   # the same split on full row tiles, A row stride > K
    (8192, 6400, 2560, None, None),   # 8192-row chunk: two rounds of each tile width
    (150, 6400, 2560, None, None),    # too few tiles for 256x256: 256x160 tiles
    (150, 6400, 2560, None, 6408),    # output row stride > N (16-byte stores)
    (300, 6400, 2560, None, 6404),    # output rows not 16-byte aligned: register-staged tiles
    (600, 6400, 2624, None, None),    # odd number of 64-wide K slices: not the ping-pong tiles
])
def test_store_bf16(M, N, K, lda, ldc):
    A, B = operands(M, N, K, 1, lda)
    ldc = ldc or N
    out = torch.full((M + 4, ldc), SENTINEL, dtype=torch.bfloat16, device="cuda")
    assert D.dory_test_gemm(A, B, D.EPI_STORE_BF16, out, M=M, N=N, lda=A.stride(0), ldc=ldc) == 1
    torch.cuda.synchronize()
    check(out[:M, :N], reference(A, B), True)
    assert (out[M:].float() == SENTINEL).all(), "rows beyond M written"
    assert (out[:, N:].float() == SENTINEL).all(), "columns beyond N written"


@pytest.mark.parametrize("M,N,K", [
    (4000, 4096, 512),    # 256 ping-pong tiles with the float epilogue, ragged M
    (4096, 6400, 512),    # float epilogue on a column split (wide then narrow tiles)
    (1000, 2560, 4096),   # output / down projection shape: 256x160 tiles
    (4096, 2560, 2560),
])
def test_f32(M, N, K):
    A, B = operands(M, N, K, 2)
    out = torch.full((M + 4, N), SENTINEL, dtype=torch.float32, device="cuda")
    assert D.dory_test_gemm(A, B, D.EPI_F32, out, M=M) == 1
    torch.cuda.synchronize()
    check(out[:M], reference(A, B), False)
    assert (out[M:] == SENTINEL).all()


@pytest.mark.parametrize("M", [300, 4096, 37])
def test_swiglu(M):
    N, K = 8192, 2560  # gate rows then up rows, as W_gu
    A, B = operands(M, N, K, 3)
    out = torch.full((M + 4, N // 2), SENTINEL, dtype=torch.bfloat16, device="cuda")
    assert D.dory_test_gemm(A, B, D.EPI_SWIGLU, out, M=M) == 1
    torch.cuda.synchronize()
    gu = reference(A, B)
    gate, up = gu[:, : N // 2], gu[:, N // 2:]
    ref = torch.nn.functional.silu(gate) * up
    check(out[:M], ref, True)
    assert (out[M:].float() == SENTINEL).all()


@pytest.mark.parametrize("M,N,K", [(1, 6400, 2560), (32, 2560, 4096), (100, 8192, 2560), (128, 2560, 2560),
                                   (160, 6400, 2560), (256, 2560, 4096)])
def test_split_k_bf16(M, N, K):
    A, B = operands(M, N, K, 4)
    S = D.dory_test_gemm(A, B, D.EPI_PARTIAL, None, M=M)
    assert 1 <= S <= 32
    out = torch.zeros((S, M, N), dtype=torch.float32, device="cuda")
    assert D.dory_test_gemm(A, B, D.EPI_PARTIAL, out, M=M) == S
    torch.cuda.synchronize()
    check(out.sum(0), reference(A, B), False)


def dequant_mxfp8(codes, scales):
    w = codes.view(torch.float8_e4m3fn).float()
    e = scales.to(torch.int32).float() - 127.0
    return w * torch.exp2(e).repeat_interleave(32, dim=1)


# 33-128 rows take k_gemv_mx: K ranges of 10 chunks of 128 (128 x 8192 x 2560, 33 x 6400),
# 5 (97 x 6144 x 1280), 4 (70 x 2560 x 2560, 128 x 2560 x 4096), 8 (40 x 12288 x 1024)
# and 2 (33 x 1280 x 2560)
@pytest.mark.parametrize("M,N,K", [(1, 6400, 2560), (32, 2560, 4096), (128, 8192, 2560), (70, 2560, 2560),
                                   (200, 2560, 2560), (33, 6400, 2560), (97, 6144, 1280), (128, 2560, 4096),
                                   (40, 12288, 1024), (33, 1280, 2560)])
def test_split_k_mxfp8(M, N, K):
    A, B = operands(M, N, K, 5)
    codes = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    D.dory_quantize_mxfp8(B, codes, scales)
    S = D.dory_test_gemm(A, codes, D.EPI_PARTIAL, None, B_scales=scales, M=M)
    out = torch.zeros((S, M, N), dtype=torch.float32, device="cuda")
    assert D.dory_test_gemm(A, codes, D.EPI_PARTIAL, out, B_scales=scales, M=M) == S
    torch.cuda.synchronize()
    check(out.sum(0), A.float() @ dequant_mxfp8(codes, scales).t(), False)


def test_rejects_bad_sizes():
    A, B = operands(64, 128, 96, 6)
    with pytest.raises(D.DoryError):
        D.dory_test_gemm(A, B, D.EPI_F32, None)  # K % 64 != 0


def nvfp4_operands(N, K, seed):
    """Synthetic NVFP4 weights drawn directly as codes (not from the quantiser): random
    E2M1 codes, E4M3 block scales in [2^-3, 2^3), a power-of-two matrix scale; and their
    value by the format's definition (e2m1 * e4m3 * g)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    codes = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(0x20, 0x50, (N, K // 16), generator=g, dtype=torch.int32).to(torch.uint8)
    gs = torch.tensor([2.0 ** -9])
    e2m1 = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    c = codes.to(torch.int64)
    q = torch.stack([e2m1[c & 15], e2m1[c >> 4]], dim=2).reshape(N, K)
    s = scales.to(torch.int64)
    e, m = (s >> 3) & 15, (s & 7).to(torch.float32)
    sv = torch.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * torch.exp2(e.to(torch.float32) - 7))
    W = q * sv.repeat_interleave(16, dim=1) * gs
    return codes.cuda(), scales.cuda(), gs.cuda(), W


@pytest.mark.parametrize("M,N,K", [(1, 6400, 2560), (32, 2560, 4096), (100, 8192, 2560), (128, 2560, 2560),
                                   (160, 6400, 2560), (256, 2560, 4096)])
def test_split_k_nvfp4(M, N, K):
    A, _ = operands(M, 64, K, 7)
    codes, scales, gs, W = nvfp4_operands(N, K, 8)
    S = D.dory_test_gemm(A, codes, D.EPI_PARTIAL, None, B_scales=scales, B_gscale=gs, M=M, N=N)
    out = torch.zeros((S, M, N), dtype=torch.float32, device="cuda")
    assert D.dory_test_gemm(A, codes, D.EPI_PARTIAL, out, B_scales=scales, B_gscale=gs, M=M, N=N) == S
    torch.cuda.synchronize()
    ref = A.float().cpu() @ W.t()
    # weights of size up to 6 * 2^3 * 2^-9 ~ 0.1: scale the absolute term of the tolerance
    d = (out.sum(0).cpu() - ref).abs()
    assert not (d > 2e-3 * (ref.abs() + 5.0)).any(), f"max |d| {float(d.max()):.3e}"


def test_fragment_order_copy_is_the_documented_permutation():
    """dory_arrange_weights against the layout dory.h states, built by reshaping:
    element (n, k) of block (n/16)(K/32) + k/32 at 8 (16 ((k % 32) / 8) + n % 16) + k % 8."""
    N, K = 2560, 4096
    g = torch.Generator(device="cuda").manual_seed(11)
    W = torch.randn((N, K), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty(N * K, dtype=torch.bfloat16, device="cuda")
    D.dory_arrange_weights(W, out)
    ref = W.view(N // 16, 16, K // 32, 4, 8).permute(0, 2, 3, 1, 4).contiguous().view(-1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M", [1, 32])
@pytest.mark.parametrize("N,K", [(6400, 2560), (2560, 2560), (8192, 2560), (2560, 4096)])
def test_decode_gemv_on_fragment_copy_is_bitwise_the_same(M, N, K):
    """The decode GEMV reading the fragment-order copy gives bitwise the partials it gives
    reading the row-major matrix (same values, same arithmetic order), and both match a
    float32 matmul."""
    A, B = operands(M, N, K, 12)
    Bf = torch.empty(N * K, dtype=torch.bfloat16, device="cuda")
    D.dory_arrange_weights(B, Bf)
    S = D.dory_test_gemm(A, B, D.EPI_PARTIAL, None)
    outs = []
    for frag in (None, Bf):
        C = torch.full((S, M, N), SENTINEL, dtype=torch.float32, device="cuda")
        assert D.dory_test_gemm(A, B, D.EPI_PARTIAL, C, B_frag=frag) == S
        outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    check(outs[1].sum(0), reference(A, B), False)
