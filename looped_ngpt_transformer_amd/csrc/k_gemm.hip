// Projections C = A B^T of the looped nGPT layer: [q|k|v|gate], attention output,
// SwiGLU gate/up and down ("Dory1.0-4B" paper summary / arXiv §2; shapes from the
// MXFP8 article's config fields).
//
// bf16 / MXFP8 weights: one MFMA kernel (v_mfma_f32_16x16x32_bf16, wave64) with A and B
// tiles staged in LDS (16-byte chunks, XOR-swizzled per row against bank conflicts) and
// the next K-tile prefetched into registers while the current one is multiplied.
// MXFP8 weights (E4M3 + one E8M0 scale per 32 along K, W8A16: arXiv §5, MXFP8 article)
// are dequantised to bf16 exactly while staged into LDS, so the MFMAs are bf16 x bf16
// with fp32 accumulation.
// Epilogues fuse what follows each projection: bf16 store; fp32 store scaled by the
// pre-projection row norm; SwiGLU with the sum of squares the down projection's norm
// needs; or fp32 split-K partials for small-M (decode) shapes.
#include "common.h"
#include "kernels.h"

namespace dory {

constexpr int GT = 256;  // threads per GEMM work-group (4 waves)
constexpr int BK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// 4 E4M3 bytes of `word` times the group scale -> 4 bf16 packed in 2 words (byte i
// of the word is element i). Exact whenever the product is a bf16 value.
__device__ __forceinline__ void dq4(uint32_t word, float sc, uint32_t* out) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
  out[0] = (uint32_t)f2bf(lo.x * sc) | ((uint32_t)f2bf(lo.y * sc) << 16);
  out[1] = (uint32_t)f2bf(hi.x * sc) | ((uint32_t)f2bf(hi.y * sc) << 16);
}

template <int BM, int BN, int WMW, int WNW, int EPI, int WF>
__global__ __launch_bounds__(GT) void k_gemm_mfma(GemmArgs g) {
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_CH = BM * 8 / GT;                         // 16B chunks of A per thread
  constexpr int B_CH = WF == W_MXFP8 ? BN * 4 / GT : BN * 8 / GT;  // MXFP8: 16 codes each
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs gate/up pairs per wave");

  __shared__ __align__(16) uint4 As[BM * 8];
  __shared__ __align__(16) uint4 Bs[BN * 8];
  __shared__ float rowscale[EPI == EPI_F32_ROWSCALE ? BM : 1];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int n_tile = blockIdx.x, m0 = blockIdx.y * BM;
  const int split = blockIdx.z;
  const int Ks = g.K / g.splits;
  const int kbeg = split * Ks, kend = kbeg + Ks;

  const bf16_t* A = (const bf16_t*)g.A;
  // B tile row r -> weight row
  auto brow = [&](int r) -> int {
    if (EPI == EPI_SWIGLU) {
      const int c0 = n_tile * (BN / 2);
      return r < BN / 2 ? c0 + r : g.n_half + c0 + (r - BN / 2);
    }
    return n_tile * BN + r;
  };

  uint4 ra[A_CH];
  uint4 rb[B_CH];
  uint32_t rsc[WF == W_MXFP8 ? B_CH : 1];

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = t & 7, r = (t >> 3) + i * (GT / 8);
      const int m = m0 + r;
      ra[i] = m < g.M ? *(const uint4*)(A + (size_t)m * g.lda + k0 + c * 8) : make_uint4(0, 0, 0, 0);
    }
    if (WF == W_MXFP8) {
      const uint8_t* B8 = (const uint8_t*)g.B;
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = t & 3, r = (t >> 2) + i * (GT / 4);
        const int n = brow(r);
        rb[i] = *(const uint4*)(B8 + (size_t)n * g.K + k0 + c * 16);
        rsc[i] = g.Bs[(size_t)n * (g.K / 32) + (k0 + c * 16) / 32];
      }
    } else {
      const bf16_t* B = (const bf16_t*)g.B;
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = t & 7, r = (t >> 3) + i * (GT / 8);
        rb[i] = *(const uint4*)(B + (size_t)brow(r) * g.K + k0 + c * 8);
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = t & 7, r = (t >> 3) + i * (GT / 8);
      As[swz(r, c)] = ra[i];
    }
    if (WF == W_MXFP8) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = t & 3, r = (t >> 2) + i * (GT / 4);
        const float sc = e8m0_to_f32(rsc[i]);
        uint32_t v[8];
        dq4(rb[i].x, sc, v);
        dq4(rb[i].y, sc, v + 2);
        dq4(rb[i].z, sc, v + 4);
        dq4(rb[i].w, sc, v + 6);
        Bs[swz(r, 2 * c)] = make_uint4(v[0], v[1], v[2], v[3]);
        Bs[swz(r, 2 * c + 1)] = make_uint4(v[4], v[5], v[6], v[7]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = t & 7, r = (t >> 3) + i * (GT / 8);
        Bs[swz(r, c)] = rb[i];
      }
    }
  };

  if (EPI == EPI_F32_ROWSCALE) {
    for (int r = t; r < BM; r += GT) {
      const int m = m0 + r;
      float s = 0.f;
      if (m < g.M)
        for (int j = 0; j < g.rs_n; ++j) s += g.rs_ss[(size_t)m * g.rs_n + j];
      rowscale[r] = inv_norm(s);
    }
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wave's B-tile row for its j-th 16-column block
  auto bblock = [&](int j) -> int {
    if (EPI == EPI_SWIGLU) {
      constexpr int TNh = TN / 2;
      return j < FN / 2 ? wn * TNh + j * 16 : BN / 2 + wn * TNh + (j - FN / 2) * 16;
    }
    return wn * TN + j * 16;
  };

  gload(kbeg);
  sstore();
  __syncthreads();
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[swz(wm * TM + i * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, Bs[swz(bblock(j) + (lane & 15), ch)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      sstore();
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds C[m = i*16 + 4*(lane>>4) + r][n = j*16 + (lane&15)]
  const int mrow0 = m0 + wm * TM + 4 * (lane >> 4);
  if (EPI == EPI_SWIGLU) {
    constexpr int TNh = TN / 2;
    bf16_t* H = (bf16_t*)g.C;
    const int c0 = n_tile * (BN / 2) + wn * TNh + (lane & 15);
    const int part = n_tile * WNW + wn;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mrow0 + i * 16 + r;
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const float gt = acc[i][j][r], up = acc[i][j + FN / 2][r];
          const float hv = gt / (1.f + __expf(-gt)) * up;
          if (m < g.M) H[(size_t)m * g.ldc + c0 + j * 16] = f2bf(hv);
          sq += hv * hv;
        }
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) sq += __shfl_xor(sq, msk, 64);
        if ((lane & 15) == 0 && m < g.M) g.ss_out[(size_t)m * g.ss_n + part] = sq;
      }
    }
    return;
  }
  const int ncol0 = n_tile * BN + wn * TN + (lane & 15);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mrow0 + i * 16 + r;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = ncol0 + j * 16;
        const float v = acc[i][j][r];
        if (EPI == EPI_STORE_ACT) {
          ((bf16_t*)g.C)[(size_t)m * g.ldc + n] = f2bf(v);
        } else if (EPI == EPI_F32_ROWSCALE) {
          ((float*)g.C)[(size_t)m * g.ldc + n] = v * rowscale[m - m0];
        } else {  // EPI_PARTIAL / EPI_F32
          ((float*)g.C)[(size_t)split * g.M * g.ldc + (size_t)m * g.ldc + n] = v;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 GEMM (T)
// Plain LDS-tiled FMA kernel for the fp32 configuration: 64x64 tile, 4x4 per thread.
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const float* A = (const float*)g.A;
  const float* B = (const float*)g.B;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
      const int r = e / 16, k = e % 16;
      const int m = m0 + r, n = n0 + r;
      As[k][r] = (m < g.M && k0 + k < g.K) ? A[(size_t)m * g.lda + k0 + k] : 0.f;
      Bs[k][r] = (n < g.N && k0 + k < g.K) ? B[(size_t)n * g.K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  float* C = (float*)g.C;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < g.M && n < g.N) C[(size_t)m * g.ldc + n] = acc[i][j];
    }
}

// ------------------------------------------------------------------------ dispatch
int gemm_pick_splits(int M, int N, int K, int wfmt) {
  // small-M (decode) tiles are BN = 64 wide; aim for >= 512 work-groups
  const int tiles = (N / 64) * ((M + 127) / 128);
  int s = 1;
  while (s < 16 && tiles * s < 512 && (K / BK) % (2 * s) == 0 && K / (2 * s) >= 2 * BK) s *= 2;
  return s;
}

int gemm_swiglu_ss_parts(const GemmArgs& g) {
  // prefill SwiGLU tile: BN = 128 (64 gate + 64 up columns), 2 waves along N
  return (g.n_half / 64) * 2;
}

template <int BM, int BN, int WMW, int WNW, int EPI>
static hipError_t go(const GemmArgs& g, hipStream_t st, int ntiles_n) {
  dim3 grid(ntiles_n, (g.M + BM - 1) / BM, g.splits);
  if (g.wfmt == W_MXFP8)
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WMW, WNW, EPI, W_MXFP8>), grid, dim3(GT), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WMW, WNW, EPI, W_BF16>), grid, dim3(GT), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& gin, hipStream_t st) {
  GemmArgs g = gin;
  if (g.M == 0) return hipSuccess;
  if (g.wfmt == W_F32) {
    if (g.epi != EPI_F32 || g.act != ACT_F32) return hipErrorInvalidValue;
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  if (g.act != ACT_BF16 || g.K % BK != 0 || g.K % (g.splits * BK) != 0) return hipErrorInvalidValue;
  switch (g.epi) {
    case EPI_PARTIAL:
      if (g.N % 64) return hipErrorInvalidValue;
      if (g.M <= 32) return go<32, 64, 1, 4, EPI_PARTIAL>(g, st, g.N / 64);
      if (g.M <= 64) return go<64, 64, 1, 4, EPI_PARTIAL>(g, st, g.N / 64);
      return go<128, 64, 1, 4, EPI_PARTIAL>(g, st, g.N / 64);
    case EPI_STORE_ACT:
      if (g.N % 128 || g.splits != 1) return hipErrorInvalidValue;
      return go<128, 128, 2, 2, EPI_STORE_ACT>(g, st, g.N / 128);
    case EPI_F32_ROWSCALE:
      if (g.N % 128 || g.splits != 1) return hipErrorInvalidValue;
      return go<128, 128, 2, 2, EPI_F32_ROWSCALE>(g, st, g.N / 128);
    case EPI_SWIGLU:
      if (g.n_half % 64 || g.splits != 1) return hipErrorInvalidValue;
      g.ss_n = gemm_swiglu_ss_parts(g);
      return go<128, 128, 2, 2, EPI_SWIGLU>(g, st, g.n_half / 64);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dory
