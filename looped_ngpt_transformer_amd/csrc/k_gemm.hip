// Projections C = A B^T of the looped nGPT layer: [q|k|v|gate], attention output,
// SwiGLU gate/up and down ("Dory1.0-4B" paper summary / arXiv §2; shapes from the
// MXFP8 article's config fields), all on gfx950 bf16 MFMA with fp32 accumulation.
//
// Large M (prefill, > 256 rows): k_gemm_pp, 256 x 256 or 256 x 160 tiles on 8 waves in
// two groups one phase apart (one group feeds the matrix cores while the other reads
// LDS), 64-wide K slices streamed straight into two LDS stages. Quantised weights
// (MXFP8: E4M3 + one E8M0 scale per 32 along K, W8A16, arXiv §5; NVFP4) are first
// expanded to bf16 exactly (k_mxfp8_expand here, k_nvfp4_expand), so these tiles serve
// every format.
// Small M (decode, <= 256 rows): split-K streaming kernels that read each weight once
// and leave fp32 partials for the consumer: k_gemv (bf16, <= 32 rows: weights straight
// into registers, every load of a wave in flight at once), k_gemm_pipe (bf16, more
// rows), k_gemv_mx (MXFP8, 33-128 rows: codes in registers, the activations through
// LDS, each weight read once), k_gemm_mx32 / k_gemm_nv32 (MXFP8 / NVFP4 codes converted
// to bf16 in registers just before the MFMA).
// k_gemm_mfma (register-staged tiles) covers the shapes the others cannot take.
// Epilogues fuse what follows each projection: bf16 store; fp32 store; SwiGLU; or the
// split-K partials. The L2 norms before the output and down projections only scale a
// row, and the nGPT update normalises the projection's output, so they need no work.
#include <type_traits>

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
// of the word is element i), with gfx950's scaled conversion (two codes per
// instruction). Exact whenever the product is a bf16 value, which holds for every
// code times a power-of-two group scale outside the extreme E8M0 range.
__device__ __forceinline__ void dq4(uint32_t word, float sc, uint32_t* out) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)word, sc, false));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)word, sc, true));
}

// W = E4M3 code * 2^(scale - 127) as bf16 (MXFP8 weights for the large-M GEMMs, which
// then run on the bf16 tiles), one thread per group of 32 along K: 32 code bytes and a
// scale byte in, 64 bytes out, with the same exact scaled conversion as the split-K
// tiles.
__global__ __launch_bounds__(256) void k_mxfp8_expand(const uint8_t* codes, const uint8_t* scales, int64_t ngroups,
                                                      bf16_t* out) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= ngroups) return;
  const float sc = e8m0_to_f32(scales[gi]);
  const uint4* src = (const uint4*)(codes + (size_t)gi * 32);
  uint4* dst = (uint4*)(out + (size_t)gi * 32);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 c = src[h];
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) dq4(w[i], sc, o + 2 * i);
    dst[2 * h] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[2 * h + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

hipError_t launch_expand_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, void* out,
                               hipStream_t st) {
  const int64_t ng = rows * (cols / 32);
  if (ng == 0) return hipSuccess;
  hipLaunchKernelGGL(k_mxfp8_expand, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, st, codes, scales, ng,
                     (bf16_t*)out);
  return hipGetLastError();
}

// Epilogue: lane holds C[m = i*16 + 4*(lane>>4) + r][n = j*16 + (lane&15)] of its wave tile.
template <int BM, int BN, int WMW, int WNW, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x4 (&acc)[BM / WMW / 16][BN / WNW / 16],
                                              int n_tile, int m0, int split, int wm, int wn, int lane) {
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 16, FN = TN / 16;
  const int mrow0 = m0 + wm * TM + 4 * (lane >> 4);
  if (EPI == EPI_SWIGLU) {
    constexpr int TNh = TN / 2;
    bf16_t* H = (bf16_t*)g.C;
    const int c0 = n_tile * (BN / 2) + wn * TNh + (lane & 15);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mrow0 + i * 16 + r;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const float gt = acc[i][j][r], up = acc[i][j + FN / 2][r];
          H[(size_t)m * g.ldc + c0 + j * 16] = f2bf(silu(gt) * up);
        }
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
        } else {  // EPI_PARTIAL / EPI_F32
          ((float*)g.C)[(size_t)split * g.M * g.ldc + (size_t)m * g.ldc + n] = v;
        }
      }
    }
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Epilogue of the 32x32 MFMA tiles: register r of lane l holds
// C[m = i*32 + 8*(r/4) + 4*(l/32) + r%4][n = j*32 + l%32] of the wave tile.
template <int BM, int BN, int WMW, int WNW, int EPI>
__device__ __forceinline__ void gemm_epilogue32(const GemmArgs& g, f32x16 (&acc)[BM / WMW / 32][BN / WNW / 32],
                                                int n_tile, int m0, int wm, int wn, int lane) {
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 32, FN = TN / 32;
  const int mrow0 = m0 + wm * TM + 4 * (lane >> 5);
  if (EPI == EPI_SWIGLU) {
    bf16_t* H = (bf16_t*)g.C;
    const int c0 = n_tile * (BN / 2) + wn * (TN / 2) + (lane & 31);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mrow0 + i * 32 + 8 * (r >> 2) + (r & 3);
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const float gt = acc[i][j][r], up = acc[i][j + FN / 2][r];
          H[(size_t)m * g.ldc + c0 + j * 32] = f2bf(silu(gt) * up);
        }
      }
    return;
  }
  const int ncol0 = n_tile * BN + wn * TN + (lane & 31);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mrow0 + i * 32 + 8 * (r >> 2) + (r & 3);
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = ncol0 + j * 32;
        if (EPI == EPI_STORE_ACT) ((bf16_t*)g.C)[(size_t)m * g.ldc + n] = f2bf(acc[i][j][r]);
        else ((float*)g.C)[(size_t)m * g.ldc + n] = acc[i][j][r];  // EPI_F32, one split
      }
    }
}

// XCD-aware tile order. Work-groups are dispatched round-robin over the 8 XCDs (each
// with its own L2); give each XCD a contiguous share of the tiles, ordered in groups of
// GM m-tiles (m fastest) so the tiles resident on one XCD share A rows and B columns.
template <int GM>
__device__ __forceinline__ void tile_coords(int* n_tile, int* m_tile) {
  const int nx = gridDim.x, ny = gridDim.y, total = nx * ny;
  const int bid = blockIdx.x + blockIdx.y * nx;
  const int L = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  const int per_group = GM * nx;
  const int first_m = (L / per_group) * GM;
  const int gm = min(ny - first_m, GM);
  const int r = L % per_group;
  *m_tile = first_m + r % gm;
  *n_tile = r / gm;
}

template <int BM, int BN, int WMW, int WNW, int EPI, int WF>
__global__ __launch_bounds__(GT) void k_gemm_mfma(GemmArgs g) {
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_CH = BM * 8 / GT;                         // 16B chunks of A per thread
  constexpr int B_CH = WF == W_MXFP8 ? BN * 4 / GT : BN * 8 / GT;  // MXFP8: 16 codes each
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs gate/up pairs per wave");

  __shared__ __align__(16) uint4 As[2][BM * 8];  // double-buffered K-tiles
  __shared__ __align__(16) uint4 Bs[2][BN * 8];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  int n_tile, m_tile;
  tile_coords<8>(&n_tile, &m_tile);
  const int m0 = m_tile * BM;
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
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = t & 7, r = (t >> 3) + i * (GT / 8);
      As[buf][swz(r, c)] = ra[i];
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
        Bs[buf][swz(r, 2 * c)] = make_uint4(v[0], v[1], v[2], v[3]);
        Bs[buf][swz(r, 2 * c + 1)] = make_uint4(v[4], v[5], v[6], v[7]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = t & 7, r = (t >> 3) + i * (GT / 8);
        Bs[buf][swz(r, c)] = rb[i];
      }
    }
  };


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

  // one barrier per K-tile: tile i+1 is loaded into registers during tile i's MFMAs
  // and stored to the other LDS buffer, whose readers all passed the previous barrier
  gload(kbeg);
  sstore(0);
  __syncthreads();
  const int nk = (kend - kbeg) / BK;
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) gload(kbeg + (it + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[cur][swz(wm * TM + i * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, Bs[cur][swz(bblock(j) + (lane & 15), ch)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }

  gemm_epilogue<BM, BN, WMW, WNW, EPI>(g, acc, n_tile, m0, split, wm, wn, lane);
}

// ------------------------------------------------------- bf16 GEMM, direct-to-LDS pipeline
// The same product for bf16 weights with a deeper pipeline: K-tiles of 32 staged in a
// ring of STAGES LDS buffers by global_load_lds_dwordx4 (each lane's 16 bytes land at
// the wave's LDS base + 16 * lane, so the XOR swizzle is applied on the source side).
// Loads for tile i + STAGES - 1 are issued while tile i is multiplied; one barrier per
// tile. Rows of A beyond M are loaded from row M - 1 (valid memory) and never stored.
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;

// LDS position of 16-byte chunk `chunk` of tile row `row` (CPR chunks per row): XOR
// swizzle so that the 16 consecutive rows one LDS cycle serves for a fragment read
// (same logical chunk) land in 16 distinct 16-byte bank groups: with 128-byte rows, row
// parity picks the half of the 64 banks and (row / 2) % 8 the group within it.
template <int CPR>
__device__ __forceinline__ int swzc(int row, int chunk) {
  return row * CPR + (chunk ^ (CPR == 8 ? ((row >> 1) & 7) : ((row >> 1) & 3)));
}

// One 16-byte-per-lane load from global memory straight into LDS (64 lanes fill 1 KiB
// at lds) through a buffer resource over [base, base + nbytes): lanes whose offset voff
// lies beyond nbytes read zeros; soff is a wave-uniform byte offset.
__device__ __forceinline__ void buffer_load_lds16(const void* base, int nbytes, lds_void_t lds, int voff,
                                                  int soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) for a run-time n <= 31 (other counters untouched)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define DORY_WVM(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    DORY_WVM(0) DORY_WVM(1) DORY_WVM(2) DORY_WVM(3) DORY_WVM(4) DORY_WVM(5) DORY_WVM(6)
    DORY_WVM(7) DORY_WVM(8) DORY_WVM(9) DORY_WVM(10) DORY_WVM(11) DORY_WVM(12) DORY_WVM(13)
    DORY_WVM(14) DORY_WVM(15) DORY_WVM(16) DORY_WVM(17) DORY_WVM(18) DORY_WVM(19) DORY_WVM(20)
    DORY_WVM(21) DORY_WVM(22) DORY_WVM(23) DORY_WVM(24) DORY_WVM(25) DORY_WVM(26) DORY_WVM(27)
    DORY_WVM(28) DORY_WVM(29) DORY_WVM(30) DORY_WVM(31)
#undef DORY_WVM
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

template <int BM, int BN, int WMW, int WNW, int EPI, int STAGES, int PBK = 32>
__global__ __launch_bounds__(GT) void k_gemm_pipe(GemmArgs g) {
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int CPR = PBK / 8;                     // 16-byte chunks per tile row
  constexpr int ACH = BM * CPR, BCH = BN * CPR;    // chunks per K-tile
  constexpr int NINST = (ACH + BCH) / 64;         // wave load instructions per K-tile
  constexpr int MAXI = (NINST + 3) / 4;
  static_assert(ACH % 64 == 0 && BCH % 64 == 0, "tile rows must be multiples of 16");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs gate/up pairs per wave");
  static_assert((STAGES - 2) * MAXI <= 31, "vmcnt range");
  static_assert(PBK == 32 || PBK == 64, "K-tile of 32 or 64");
  static_assert(STAGES >= 2, "at least double buffering");

  __shared__ __align__(16) uint4 sm[STAGES][ACH + BCH];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  int n_tile, m_tile;
  tile_coords<8>(&n_tile, &m_tile);
  const int m0 = m_tile * BM;
  const int split = blockIdx.z;
  const int Ks = g.K / g.splits;
  const int kbeg = split * Ks;
  const int nk = Ks / PBK;
  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;
  const int my_inst = (NINST - wave + 3) / 4;  // instructions this wave issues per K-tile

  auto brow = [&](int r) -> int {
    if (EPI == EPI_SWIGLU) {
      const int c0 = n_tile * (BN / 2);
      return r < BN / 2 ? c0 + r : g.n_half + c0 + (r - BN / 2);
    }
    return n_tile * BN + r;
  };
  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int q = 0; q < MAXI; ++q) {
      const int inst = wave + 4 * q;
      if (inst < NINST) {
        const int sidx = inst * 64 + lane;
        const bf16_t* src;
        if (sidx < ACH) {
          const int r = sidx / CPR, c = swzc<CPR>(r, sidx % CPR) - r * CPR;
          const int m = min(m0 + r, g.M - 1);
          src = A + (size_t)m * g.lda + k0 + 8 * c;
        } else {
          const int s2 = sidx - ACH;
          const int r = s2 / CPR, c = swzc<CPR>(r, s2 % CPR) - r * CPR;
          src = B + (size_t)brow(r) * g.K + k0 + 8 * c;
        }
        __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(&sm[slot][inst * 64]), 16, 0, 0);
      }
    }
  };


  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto bblock = [&](int j) -> int {
    if (EPI == EPI_SWIGLU) {
      constexpr int TNh = TN / 2;
      return j < FN / 2 ? wn * TNh + j * 16 : BN / 2 + wn * TNh + (j - FN / 2) * 16;
    }
    return wn * TN + j * 16;
  };

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, kbeg + PBK * st);

  for (int it = 0; it < nk; ++it) {
    const int ahead = min(STAGES - 2, nk - 1 - it);  // later tiles already in flight
    wait_vmcnt(ahead * my_inst);
    __syncthreads();
    if (it + STAGES - 1 < nk) issue((it + STAGES - 1) % STAGES, kbeg + PBK * (it + STAGES - 1));
    const uint4* As = sm[it % STAGES];
    const uint4* Bs = As + ACH;
#pragma unroll
    for (int kk = 0; kk < PBK / 32; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[swzc<CPR>(wm * TM + i * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, Bs[swzc<CPR>(bblock(j) + (lane & 15), ch)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  gemm_epilogue<BM, BN, WMW, WNW, EPI>(g, acc, n_tile, m0, split, wm, wn, lane);
}

// Weights in fragment order for the decode GEMV: thread c copies output chunk c (16
// bytes): block c / 64, lane l = c % 64 of that block's MFMA B operand.
__global__ __launch_bounds__(256) void k_arrange_frag(const bf16_t* w, int64_t N, int64_t K, bf16_t* out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= N * K / 8) return;
  const int64_t blk = c >> 6, kb = K / 32;
  const int l = (int)(c & 63);
  const int64_t row = (blk / kb) * 16 + (l & 15), k0 = (blk % kb) * 32 + 8 * (l >> 4);
  *(uint4*)(out + 8 * c) = *(const uint4*)(w + row * K + k0);
}

hipError_t launch_arrange_frag(const void* w, int64_t N, int64_t K, void* out, hipStream_t st) {
  if (!w || !out || N < 16 || K < 32 || N % 16 || K % 32) return hipErrorInvalidValue;
  const int64_t chunks = N * K / 8;
  hipLaunchKernelGGL(k_arrange_frag, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, (const bf16_t*)w, N, K,
                     (bf16_t*)out);
  return hipGetLastError();
}

// Decode GEMV for bf16 weights and at most 32 activation rows, bound by the weight
// stream. A work-group of 4 waves owns 64 weight rows over a K range of 32 KW; each wave
// streams its 16 rows straight into registers, all KW loads in flight before the first
// MFMA (16 KW bytes per lane), so a launch keeps the whole weight matrix in flight.
// The activation slice (32 rows x 32 KW, rows beyond M repeat the last row) goes to LDS
// once per work-group with direct-to-LDS loads, 16-byte chunks XOR-swizzled by row.
// v_mfma_f32_16x16x32_bf16 with the activations as the A operand: lane l holds weight
// row l % 16, K elements 8 (l / 16) .. + 7 of each 32-wide step. From the row-major
// matrix a load instruction reads 64 contiguous bytes of each of 16 rows; from the
// fragment-order copy (FRAG) one contiguous KiB, and a wave's KW loads one contiguous
// 16 KW KiB. Same values, same arithmetic. Output: fp32 split-K partials, split = K range.
template <int KW, bool FRAG>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs g) {
  constexpr int KS = 32 * KW;       // K range of one work-group (one split)
  constexpr int CH = KS / 8;        // 16-byte chunks per activation row
  constexpr int AI = 32 * CH / 256; // activation load instructions per thread
  static_assert(KW == 8 || KW == 16, "K range of 256 or 512");
  __shared__ __align__(16) uint4 sa[32 * CH];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * 64 + wave * 16;
  const int split = blockIdx.y;
  const int kbeg = split * KS;
  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;

  // LDS slot p = 256 q + t holds chunk (p % CH) ^ (row % 8) of activation row p / CH
#pragma unroll
  for (int q = 0; q < AI; ++q) {
    const int p = q * 256 + t, row = p / CH, sl = p % CH;
    const int m = min(row, g.M - 1);
    const bf16_t* src = A + (size_t)m * g.lda + kbeg + 8 * (sl ^ (row & 7));
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(sa + q * 256 + (t & ~63)), 16, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 bw[KW];
  const bf16_t* bsrc = FRAG ? (const bf16_t*)g.Bf + ((size_t)(n0 / 16) * (g.K / 32) + kbeg / 32) * 512 + 8 * lane
                            : B + (size_t)(n0 + (lane & 15)) * g.K + kbeg + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < KW; ++ks) bw[ks] = *(const uint4*)(bsrc + (FRAG ? 512 : 32) * ks);
  __builtin_amdgcn_sched_barrier(0);
  // the activation slice (issued first) has landed once at most KW loads are pending;
  // a bare barrier (no fence) leaves the weight loads in flight
  wait_vmcnt(KW);
  asm volatile("s_barrier" ::: "memory");

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int r0 = lane & 15, cq = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < KW; ++ks) {
    const int c = 4 * ks + cq;
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, sa[r0 * CH + (c ^ (r0 & 7))]);
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, sa[(16 + r0) * CH + (c ^ (r0 & 7))]);
    const bf16x8 b = __builtin_bit_cast(bf16x8, bw[ks]);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc1, 0, 0, 0);
  }
  // lane l: column n0 + l % 16, rows 4 (l / 16) + i of each 16-row block
  float* C = (float*)g.C + (size_t)split * g.M * g.ldc + n0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * cq + i;
    if (m < g.M) C[(size_t)m * g.ldc] = acc0[i];
    if (m + 16 < g.M) C[(size_t)(m + 16) * g.ldc] = acc1[i];
  }
}

// MXFP8 decode GEMM for 33-128 activation rows (W8A16), bound by the codes, the
// activations and the split partials together: at 128 rows an activation slice is as
// large as the codes of a 64-row weight block, and every split adds 128 x N x 4 bytes of
// partials. A work-group of 4 waves owns 64 weight rows over a long K range (NCH chunks
// of 128, few splits); each wave holds its 16 rows' codes for the whole range in
// registers (issued before anything else), while the activations (128 rows, rows beyond
// M repeat the last) stream through two LDS stages of one 128-wide chunk each. Per
// 32-wide step a wave converts its B fragment (8 codes, the group's E8M0 scale, exact)
// once and runs it against the 8 row blocks of 16 (v_mfma_f32_16x16x32_bf16).
// K order inside a 64-wide block: lane l loads the 16 codes at 16 (l / 16) .. + 15 and
// uses the first 8 in the block's first step, the other 8 in its second; the activation
// fragments take the same order (a permutation of the contraction index, so the sums
// are the same products). Output: fp32 split-K partials, split = K range.
template <int NCH>
__global__ __launch_bounds__(256) void k_gemv_mx(GemmArgs g) {
  constexpr int KS = 128 * NCH;   // K range of the work-group
  __shared__ __align__(16) uint4 sa0[128 * 16];  // chunk stages: 128 rows x 16 chunks of 8 bf16
  __shared__ __align__(16) uint4 sa1[128 * 16];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * 64 + wave * 16;
  const int split = blockIdx.y;
  const int kbeg = split * KS;
  const int r16 = lane & 15, q = lane >> 4;
  const bf16_t* A = (const bf16_t*)g.A;

  // codes: 16 bytes per 64-wide block (row n0 + r16, K kbeg + 64 b + 16 q ..), and the
  // row's four E8M0 scales of each chunk (groups kbeg / 32 + 4 c ..)
  uint4 cw[2 * NCH];
  uint32_t sc4[NCH];
  {
    const uint8_t* crow = (const uint8_t*)g.B + (size_t)(n0 + r16) * g.K + kbeg + 16 * q;
    const uint8_t* srow = g.Bs + (size_t)(n0 + r16) * (g.K / 32) + kbeg / 32;
#pragma unroll
    for (int b = 0; b < 2 * NCH; ++b) cw[b] = *(const uint4*)(crow + 64 * b);
#pragma unroll
    for (int c = 0; c < NCH; ++c) sc4[c] = *(const uint32_t*)(srow + 4 * c);
  }
  // activation chunk c into a stage: slot p (row p / 16, slot p % 16) holds chunk
  // (p % 16) ^ (row % 16) of that row's 128-wide chunk; 8 loads per thread
  auto issue = [&](int c, auto S) {
    uint4* st0 = decltype(S)::value == 0 ? sa0 : sa1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = i * 256 + t, row = p >> 4, sl = p & 15;
      const bf16_t* src = A + (size_t)min(row, g.M - 1) * g.lda + kbeg + 128 * c + 8 * (sl ^ (row & 15));
      __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(st0 + i * 256 + (t & ~63)), 16, 0, 0);
    }
  };
  f32x4 acc[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int c, auto S) {
    const uint4* st0 = decltype(S)::value == 0 ? sa0 : sa1;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint4 w = cw[2 * c + h2];
      const float scf = e8m0_to_f32((sc4[c] >> (8 * (2 * h2 + (q >> 1)))) & 0xFFu);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t v[4];
        dq4(h ? w.z : w.x, scf, v);
        dq4(h ? w.w : w.y, scf, v + 2);
        const bf16x8 bfrag = __builtin_bit_cast(bf16x8, make_uint4(v[0], v[1], v[2], v[3]));
        const int ch = 8 * h2 + 2 * q + h;  // 16-byte chunk of the stage row
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          const int row = 16 * mb + r16;
          const bf16x8 afrag = __builtin_bit_cast(bf16x8, st0[row * 16 + (ch ^ r16)]);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag, acc[mb], 0, 0, 0);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  issue(0, S0{});
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // codes, scales, chunk 0
  // the codes and scales are used here once, so that the compiler's own wait for them
  // falls before the next chunk's loads go out (after them it would wait for those too)
#pragma unroll
  for (int b = 0; b < 2 * NCH; ++b) asm volatile("" ::"v"(cw[b].x), "v"(cw[b].y), "v"(cw[b].z), "v"(cw[b].w));
#pragma unroll
  for (int c = 0; c < NCH; ++c) asm volatile("" ::"v"(sc4[c]));
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    // stage (c + 1) % 2 last held chunk c - 1, which every wave finished before the
    // barrier that ended the previous step
    if (c + 1 < NCH) {
      if (c % 2 == 0) issue(c + 1, S1{});
      else issue(c + 1, S0{});
    }
    // the next chunk's loads all leave before this chunk's work (left to itself the
    // scheduler spreads them through it, and the last ones then meet the wait below)
    __builtin_amdgcn_sched_barrier(0);
    if (c % 2 == 0) compute(c, S0{});
    else compute(c, S1{});
    if (c + 1 < NCH) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // lane l: column n0 + l % 16, rows 16 mb + 4 (l / 16) + i
  float* C = (float*)g.C + (size_t)split * g.M * g.ldc + n0 + r16;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * mb + 4 * q + i;
      if (m < g.M) C[(size_t)m * g.ldc] = acc[mb][i];
    }
}

// Sustained rate of v_mfma_f32_32x32x16_bf16 on this device (the practical ceiling the
// projection GEMMs are measured against): 8 waves per work-group (two per SIMD), each
// running 8 independent accumulator chains of `iters` instructions on register operands
// holding non-zero data; thread 0 records the shader-clock cycles of the loop.
__global__ __launch_bounds__(512) void k_mfma_rate(int iters, long long* cycles, float* sink) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((float)((t * 7 + i * 13) % 17 - 8) * 0.0625f);
    b[i] = (__bf16)((float)((t * 5 + i * 11) % 19 - 9) * 0.03125f);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  __syncthreads();
  const long long c0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  __syncthreads();
  const long long c1 = clock64();
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[j][r];
  sink[(size_t)blockIdx.x * 512 + t] = sum;
  if (t == 0) cycles[blockIdx.x] = c1 - c0;
}

hipError_t launch_mfma_rate(int iters, int n_wg, long long* cycles, float* sink, hipStream_t st) {
  if (iters < 1 || n_wg < 1 || !cycles || !sink) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_rate, dim3(n_wg), dim3(512), 0, st, iters, cycles, sink);
  return hipGetLastError();
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
constexpr int SPLITK_WG = 400;    // work-groups a decode GEMM aims for
constexpr int SPLITK_MINK = 128;  // shortest K range of one split
// k_gemv takes bf16 weights, M <= 32 and splits of 256 or 512 along K (at most 32); a
// matrix with enough 64-column tiles to fill the device unsplit (the LM head) streams
// through k_gemm_pipe without partials instead
static int gemv_splits(int M, int N, int K, int wfmt) {
  if (wfmt != W_BF16 || M > 32 || N % 64 || N / 64 >= SPLITK_WG) return 0;
  if (K % 512 == 0 && (N / 64) * (K / 512) >= 300 && K / 512 <= 32) return K / 512;
  if (K % 256 == 0 && K / 256 <= 32) return K / 256;
  return 0;
}

// k_gemv_mx takes MXFP8 weights, 33-128 rows and K ranges of NCH chunks of 128 with NCH
// in {2, 4, 5, 8, 10}: the fewest splits that give at least 192 work-groups
static bool gemv_mx_nch_ok(int nch) { return nch == 2 || nch == 4 || nch == 5 || nch == 8 || nch == 10; }
static int gemv_mx_splits(int M, int N, int K, int wfmt) {
  if (wfmt != W_MXFP8 || M <= 32 || M > 128 || N % 64 || K % 128) return 0;
  for (int s = 1; s <= 32; ++s)
    if (K % (128 * s) == 0 && gemv_mx_nch_ok(K / (128 * s)) && (N / 64) * s >= 192) return s;
  return 0;
}

int gemm_pick_splits(int M, int N, int K, int wfmt) {
  if (const int s = gemv_splits(M, N, K, wfmt)) return s;
  if (const int s = gemv_mx_splits(M, N, K, wfmt)) return s;
  // small-M (decode) tiles are BN = 64 wide (128 for MXFP8); split K until there are
  // enough work-groups to keep the weight stream in flight (each split a multiple of 64,
  // not too short)
  int tiles = (N / 64) * ((M + 127) / 128), cap = 32;
  if ((wfmt == W_MXFP8 || wfmt == W_NVFP4) && N % 128 == 0) {  // 32 or 64 activation rows per tile, <= 8 splits
    tiles = (N / 128) * ((M + (M <= 32 ? 31 : 63)) / (M <= 32 ? 32 : 64));
    cap = 8;
  }
  int s = 1;
  while (s < cap && tiles * s < SPLITK_WG && (K / BK) % (2 * s) == 0 && K / (2 * s) >= SPLITK_MINK) s *= 2;
  return s;
}


// Large-M tiles on v_mfma_f32_32x32x16_bf16 (on gfx950 it sustains about 1.5x the
// rate of the 16x16x32 form). Same direct-to-LDS K-slice ring of 64-wide slices as
// k_gemm_pipe; each wave owns (BM/WMW) x (BN/WNW) outputs as 32x32 blocks. A fragment
// (lane l): row l % 32 of the block, K elements 8 (l / 32) .. + 7 of the 16-wide step,
// one swizzled 16-byte LDS chunk.
template <int BM, int BN, int WMW, int WNW, int EPI, int STAGES>
__global__ __launch_bounds__(WMW * WNW * 64) void k_gemm_pipe32(GemmArgs g) {
  constexpr int PBK = 64;
  constexpr int NW = WMW * WNW;  // 4 waves (one per SIMD) or 8 (two per SIMD)
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CPR = PBK / 8;
  constexpr int ACH = BM * CPR, BCH = BN * CPR;
  constexpr int NINST = (ACH + BCH) / 64;
  constexpr int MAXI = (NINST + NW - 1) / NW;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 blocks per wave");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(ACH % 64 == 0 && BCH % 64 == 0, "tile rows must be multiples of 8");
  static_assert(EPI != EPI_SWIGLU || FN % 2 == 0, "SwiGLU needs gate/up pairs per wave");
  static_assert((STAGES - 2) * MAXI <= 31, "vmcnt range");
  static_assert(STAGES >= 2, "at least double buffering");

  __shared__ __align__(16) uint4 sm[STAGES][ACH + BCH];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6) & (NW - 1);  // uniform, < NW
  const int wm = wave / WNW, wn = wave % WNW;
  int n_tile, m_tile;
  tile_coords<8>(&n_tile, &m_tile);
  const int m0 = m_tile * BM;
  const int nk = g.K / PBK;
  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;
  const int my_inst = (NINST - wave + NW - 1) / NW;

  auto brow = [&](int r) -> int {
    if (EPI == EPI_SWIGLU) {
      const int c0 = n_tile * (BN / 2);
      return r < BN / 2 ? c0 + r : g.n_half + c0 + (r - BN / 2);
    }
    return n_tile * BN + r;
  };
  // Instruction i fills LDS chunks 64 i .. 64 i + 63 (8 rows of 8 chunks), A rows for
  // i < ACH / 64, then B. The swizzle of row 8 i + lane / 8 depends only on i % 2 = wave
  // % 2 and the lane, so one per-lane offset serves every instruction of the wave; A goes
  // through a buffer resource from the tile's first row whose range check returns zeros
  // for rows at or beyond M.
  const int lr = lane >> 3;
  const int lc = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const int voA = (lr * g.lda + 8 * lc) * 2;
  const int voB = (lr * g.K + 8 * lc) * 2;
  const long a_rest = (long)(g.M - m0) * g.lda * 2;
  const int a_bytes = a_rest < 0x7fffffffL ? (int)a_rest : 0x7fffffff;
  const bf16_t* Am = A + (size_t)m0 * g.lda;
  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int q = 0; q < MAXI; ++q) {
      const int inst = wave + NW * q;
      if (inst < NINST) {
        if (inst < ACH / 64)
          buffer_load_lds16(Am, a_bytes, (lds_void_t)(&sm[slot][inst * 64]), voA + 16 * g.lda * inst, 2 * k0);
        else
          buffer_load_lds16(B, 0x7fffffff, (lds_void_t)(&sm[slot][inst * 64]), voB,
                            2 * (brow(8 * (inst - ACH / 64)) * g.K + k0));
      }
    }
  };
  auto bblock = [&](int j) -> int {
    if (EPI == EPI_SWIGLU) {
      constexpr int TNh = TN / 2;
      return j < FN / 2 ? wn * TNh + j * 32 : BN / 2 + wn * TNh + (j - FN / 2) * 32;
    }
    return wn * TN + j * 32;
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, PBK * st);

  for (int it = 0; it < nk; ++it) {
    const int ahead = min(STAGES - 2, nk - 1 - it);  // later tiles already in flight
    wait_vmcnt(ahead * my_inst);
    __syncthreads();
    if (it + STAGES - 1 < nk) issue((it + STAGES - 1) % STAGES, PBK * (it + STAGES - 1));
    const uint4* As = sm[it % STAGES];
    const uint4* Bs = As + ACH;
    // 16-wide K steps with two fragment sets: the reads of step ks+1 are interleaved with
    // the MFMAs of step ks (one read after each MFMA), so LDS latency stays hidden
    bf16x8 af[2][FM], bfr[2][FN];
    auto ldfrag = [&](int ks, bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
      const int ch = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = __builtin_bit_cast(bf16x8, As[swzc<CPR>(wm * TM + i * 32 + (lane & 31), ch)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[j] = __builtin_bit_cast(bf16x8, Bs[swzc<CPR>(bblock(j) + (lane & 31), ch)]);
    };
    ldfrag(0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < PBK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < PBK / 16) ldfrag(ks + 1, af[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      if (ks + 1 < PBK / 16) {
#pragma unroll
        for (int q = 0; q < FM + FN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
      }
    }
  }
  gemm_epilogue32<BM, BN, WMW, WNW, EPI>(g, acc, n_tile, m0, wm, wn, lane);
}

// 256 x BN bf16 tiles (BN 256 or 160) with two wave groups one phase apart
// ("ping-pong"). Waves 0-3 (group 0) and 4-7 (group 1) put one wave of each group on
// every SIMD; group g owns rows 128 g .. +127 of the tile, split among its four waves as
// 128 x 64 column blocks (BN 256) or 32 x 160 row blocks (BN 160). Each wave alternates
// two phases per 64-wide K slice, separated by work-group barriers:
//   read phase:    all 24 A/B fragments of the slice, LDS -> registers
//   compute phase: the slice's 32 or 20 MFMAs (v_mfma_f32_32x32x16_bf16)
// and group 1 runs one phase behind group 0, so on every SIMD one wave feeds the matrix
// core while the other reads LDS. Slice s lives in LDS stage s % 2. Group 1 streams it
// in with direct-to-LDS loads placed between the MFMAs of its compute phase of slice
// s - 2 (both groups have read slice s - 2 from that stage by then), where the wave's
// issue slots are otherwise idle, and waits for them at the end of its next read phase,
// one slot before group 0 reads slice s.
template <int BN, int EPI>
__global__ __launch_bounds__(512) void k_gemm_pp(GemmArgs g) {
  constexpr int BM = 256, PBK = 64, CPR = PBK / 8;
  constexpr int WMW = BN == 256 ? 2 : 8, WNW = BN == 256 ? 4 : 1;  // wave grid of the tile
  constexpr int TM = BM / WMW, TN = BN / WNW, FM = TM / 32, FN = TN / 32, KST = PBK / 16;
  constexpr int ACH = BM * CPR, BCH = BN * CPR, NA = ACH / 64;
  constexpr int NI = (ACH + BCH) / 64 / 4;  // load instructions per group-0 wave per slice
  static_assert(BN == 256 || BN == 160, "tile widths");
  static_assert((ACH + BCH) % 256 == 0 && NA % 4 == 0, "load instructions split evenly");
  static_assert(EPI != EPI_SWIGLU || (BN == 256 && FN % 2 == 0), "SwiGLU needs gate/up pairs per wave");

  // one array per stage, so that the reads of one stage are known not to alias the
  // direct-to-LDS loads in flight into the other
  __shared__ __align__(16) uint4 sm0[ACH + BCH];
  __shared__ __align__(16) uint4 sm1[ACH + BCH];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const int wm = BN == 256 ? grp : 4 * grp + w4, wn = BN == 256 ? w4 : 0;
  int n_tile, m_tile;
  tile_coords<8>(&n_tile, &m_tile);
  const int m0 = m_tile * BM;
  const int nk = g.K / PBK;
  const bf16_t* A = (const bf16_t*)g.A;
  const bf16_t* B = (const bf16_t*)g.B;

  auto stage = [&](auto S) -> uint4* {
    if constexpr (decltype(S)::value == 0) return sm0;
    else return sm1;
  };
  auto brow = [&](int r) -> int {
    if (EPI == EPI_SWIGLU) {
      const int c0 = n_tile * (BN / 2);
      return r < BN / 2 ? c0 + r : g.n_half + c0 + (r - BN / 2);
    }
    return n_tile * BN + r;
  };
  // Group-1 wave w4 issues load instructions w4, w4 + 4, ... of a slice; instruction i
  // fills LDS chunks 64 i .. 64 i + 63 (8 rows of 8 chunks), A rows for i < 32, then B.
  // The swizzle of row 8 i + lane / 8 only depends on w4 % 2 and the lane, so one per-lane
  // offset serves every instruction. The loads go through buffer resources: A from the
  // tile's first row, with a range check that returns zeros for rows at or beyond M (the
  // row offset is in the per-lane offset); B with its row and K offset in the scalar
  // offset.
  const int lr = lane >> 3;
  const int lc = (lane & 7) ^ ((4 * (w4 & 1) + (lane >> 4)) & 7);
  const long a_rest = (long)(g.M - m0) * g.lda * 2;
  const int a_bytes = a_rest < 0x7fffffffL ? (int)a_rest : 0x7fffffff;
  const int voA = (lr * g.lda + 8 * lc) * 2;
  const int voB = (lr * g.K + 8 * lc) * 2;
  const bf16_t* Am = A + (size_t)m0 * g.lda;
  auto issue_one = [&](auto S, int k0, int va, int vb, int q) {
    uint4* dst0 = stage(S);
    const int inst = w4 + 4 * q;  // inst < NA exactly for q < NA / 4
    if (q < NA / 4)
      buffer_load_lds16(Am, a_bytes, (lds_void_t)(dst0 + inst * 64), va + 16 * g.lda * inst, 2 * k0);
    else
      buffer_load_lds16(B, 0x7fffffff, (lds_void_t)(dst0 + inst * 64), vb,
                        2 * (brow(8 * (inst - NA)) * g.K + k0));
  };
  auto bblock = [&](int j) -> int {
    if (EPI == EPI_SWIGLU)
      return j < FN / 2 ? wn * (TN / 2) + j * 32 : BN / 2 + wn * (TN / 2) + (j - FN / 2) * 32;
    return wn * TN + j * 32;
  };

  // Everything from here on is instantiated once per wave group, so that the group's
  // role (who streams the slices, which waits it owns) is known at compile time and
  // its loop is one straight run of MFMAs and loads.
  auto body = [&](auto G) {
    constexpr bool G1 = decltype(G)::value;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    bf16x8 af[KST][FM], bfr[KST][FN];

    auto read_phase = [&](auto S) {
      // lane made opaque here, so that the fragment addresses derived from it are
      // recomputed in each phase instead of being held in registers across the loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint4* As = stage(S);
      const uint4* Bs = As + ACH;
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) {
        const int ch = ks * 2 + (ln >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[ks][i] = __builtin_bit_cast(bf16x8, As[swzc<CPR>(wm * TM + i * 32 + (ln & 31), ch)]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[ks][j] = __builtin_bit_cast(bf16x8, Bs[swzc<CPR>(bblock(j) + (ln & 31), ch)]);
      }
      // group 1 also waits for the slice it streamed in during its last compute phase
      if constexpr (G1) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int NMF = KST * FM * FN;  // MFMAs per slice
    // compute phase of slice it, in stage S. With LD (group 1, while slice it + 2 exists)
    // the wave streams slice it + 2 into that stage, load q right after MFMA q * NMF / NI
    // so that the NI loads spread over the phase; LD is a compile-time flag, so the
    // phase's MFMAs and loads form one straight run of instructions.
    auto compute_phase = [&](auto S, int it, auto LD) {
      int va = voA, vb = voB;
      asm volatile("" : "+v"(va), "+v"(vb));
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
            if constexpr (decltype(LD)::value) {
              const int idx = (ks * FM + i) * FN + j;
#pragma unroll
              for (int q = 0; q < NI; ++q)
                if (q * NMF / NI == idx) issue_one(S, PBK * (it + 2), va, vb, q);
            }
          }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if constexpr (G1) {  // slices 0 and 1 (nk >= 2)
#pragma unroll
      for (int q = 0; q < NI; ++q) issue_one(S0{}, 0, voA, voB, q);
#pragma unroll
      for (int q = 0; q < NI; ++q) issue_one(S1{}, PBK, voA, voB, q);
      // slice 0 only: slice 1 is waited for at the end of this group's first read phase,
      // before group 0 reads it
      wait_vmcnt(NI);
      asm volatile("s_barrier\n\ts_barrier" ::: "memory");  // + one phase behind
    } else {
      asm volatile("s_barrier" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    using LD = std::integral_constant<bool, G1>;  // group 1 streams the slices in
    using LDN = std::false_type;
    // nk is even (the launcher checks): slices it + 2 and it + 3 exist for every pair
    // but the last
    int it = 0;
    for (; it + 2 < nk; it += 2) {
      read_phase(S0{});
      compute_phase(S0{}, it, LD{});
      read_phase(S1{});
      compute_phase(S1{}, it + 1, LD{});
    }
    read_phase(S0{});
    compute_phase(S0{}, it, LDN{});
    read_phase(S1{});
    compute_phase(S1{}, it + 1, LDN{});
    if constexpr (EPI == EPI_STORE_ACT || EPI == EPI_SWIGLU) {
      // bf16 outputs through LDS: every LDS read of the main loop is done (group 0's last
      // barrier follows group 1's last read phase; no loads are in flight), so each wave
      // writes its output block into its own LDS region and stores it back as 16-byte
      // chunks of 8 consecutive columns. The two lane halves of a write hold rows r and
      // r + 4: rows are padded by 32 bytes where the region allows, else (128-byte rows)
      // the 64-byte halves of a row swap when bit 2 of the row is set, so that the halves
      // land on different banks.
      constexpr int TNO = EPI == EPI_SWIGLU ? TN / 2 : TN;  // output columns per wave
      constexpr bool PAD = 4 * TM * (TNO * 2 + 32) <= (ACH + BCH) * 16;
      constexpr int RS = PAD ? TNO * 2 + 32 : TNO * 2;      // LDS row stride (bytes)
      static_assert(4 * TM * RS <= (ACH + BCH) * 16, "output staging fits one stage array");
      static_assert(PAD || RS == 128, "swizzled staging assumes 128-byte rows");
      auto soff = [&](int row, int byte) { return row * RS + (PAD ? byte : byte ^ (((row >> 2) & 1) << 6)); };
      unsigned char* reg = (unsigned char*)(G1 ? sm1 : sm0) + w4 * TM * RS;
      const int l32 = lane & 31, lh = lane >> 5;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
#pragma unroll
          for (int j = 0; j < (EPI == EPI_SWIGLU ? FN / 2 : FN); ++j) {
            float v = acc[i][j][r];
            if constexpr (EPI == EPI_SWIGLU) {
              const float up = acc[i][j + FN / 2][r];
              v = silu(v) * up;
            }
            *(bf16_t*)(reg + soff(row, (j * 32 + l32) * 2)) = f2bf(v);
          }
        }
      constexpr int CPRO = TNO / 8;  // 16-byte chunks per output row
      static_assert((TM * CPRO) % 64 == 0, "whole store instructions per wave");
      const int ocol0 = EPI == EPI_SWIGLU ? n_tile * (BN / 2) + wn * TNO : n_tile * BN + wn * TNO;
      const int orow0 = m0 + wm * TM;
#pragma unroll
      for (int q = 0; q < TM * CPRO / 64; ++q) {
        const int idx = q * 64 + lane, row = idx / CPRO, ch = idx % CPRO;
        const uint4 v = *(const uint4*)(reg + soff(row, ch * 16));
        if (orow0 + row < g.M) *(uint4*)((bf16_t*)g.C + (size_t)(orow0 + row) * g.ldc + ocol0 + 8 * ch) = v;
      }
    } else {
      gemm_epilogue32<BM, BN, WMW, WNW, EPI>(g, acc, n_tile, m0, wm, wn, lane);
    }
    if constexpr (!G1) asm volatile("s_barrier" ::: "memory");  // matches group 1's extra first barrier
  };
  if (grp == 1) body(std::true_type{});
  else body(std::false_type{});
}

// MXFP8 (W8A16) split-K tiles for decode-sized M, on v_mfma_f32_32x32x16_bf16. The
// bf16 activations and the E4M3 weight codes stream straight into an LDS ring of
// 64-wide K slices; each lane turns its 8 codes of a B fragment into bf16 just before
// the MFMA (scaled fp8 -> bf16 conversion by the group's 2^e, exact), so the weights cross HBM
// once at one byte each. The E8M0 scales of the next slice are loaded into registers a
// slice ahead. Output: fp32 split-K partials (EPI_PARTIAL).
template <int BM, int BN, int WMW, int WNW, int STAGES>
__global__ __launch_bounds__(GT) void k_gemm_mx32(GemmArgs g) {
  constexpr int PBK = 64;
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * 8, BCH = BN * 4;   // 16-byte chunks of A (bf16) / B (codes)
  constexpr int NINST = (ACH + BCH) / 64;
  constexpr int MAXI = (NINST + 3) / 4;
  static_assert(WMW * WNW == 4 && TM % 32 == 0 && TN % 32 == 0, "tile");
  static_assert(ACH % 64 == 0 && BCH % 64 == 0, "tile rows");
  static_assert((STAGES - 2) * MAXI <= 31 && STAGES >= 2, "pipeline");
  __shared__ __align__(16) uint4 sm[STAGES][ACH + BCH];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int n_tile = blockIdx.x, m0 = blockIdx.y * BM, split = blockIdx.z;
  const int Ks = g.K / g.splits, kbeg = split * Ks, nk = Ks / PBK;
  const bf16_t* A = (const bf16_t*)g.A;
  const uint8_t* B = (const uint8_t*)g.B;
  const int my_inst = (NINST - wave + 3) / 4;
  const int l32 = lane & 31, lh = lane >> 5;

  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int q = 0; q < MAXI; ++q) {
      const int inst = wave + 4 * q;
      if (inst < NINST) {
        const int sidx = inst * 64 + lane;
        const void* src;
        if (sidx < ACH) {  // A row r, chunk c (8 bf16)
          const int r = sidx >> 3, c = swzc<8>(r, sidx & 7) - r * 8;
          src = A + (size_t)min(m0 + r, g.M - 1) * g.lda + k0 + 8 * c;
        } else {           // B row r, chunk c (16 codes); chunk slot c ^ ((r >> 2) & 3)
          const int s2 = sidx - ACH, r = s2 >> 2, c = (s2 & 3) ^ ((r >> 2) & 3);
          src = B + (size_t)(n_tile * BN + r) * g.K + k0 + 16 * c;
        }
        __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(&sm[slot][inst * 64]), 16, 0, 0);
      }
    }
  };
  // E8M0 scales of B fragment j for the two 32-groups of slice k0
  auto ldscale = [&](int k0, uint32_t (&sc)[FN][2]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n_tile * BN + wn * TN + j * 32 + l32;
      const uint8_t* p = g.Bs + (size_t)n * (g.K / 32) + k0 / 32;
      sc[j][0] = p[0];
      sc[j][1] = p[1];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The scale loads of slice it+1 are issued after the tile loads of this step, so the
  // wait below (which counts only tile loads as newer than tile it) is conservative.
  uint32_t scn[FN][2];
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, kbeg + PBK * st);
  ldscale(kbeg, scn);
  for (int it = 0; it < nk; ++it) {
    wait_vmcnt(min(STAGES - 2, nk - 1 - it) * my_inst);
    __syncthreads();
    if (it + STAGES - 1 < nk) issue((it + STAGES - 1) % STAGES, kbeg + PBK * (it + STAGES - 1));
    uint32_t sc[FN][2];
#pragma unroll
    for (int j = 0; j < FN; ++j) sc[j][0] = scn[j][0], sc[j][1] = scn[j][1];
    if (it + 1 < nk) ldscale(kbeg + PBK * (it + 1), scn);
    const uint4* As = sm[it % STAGES];
    const unsigned char* Bb = (const unsigned char*)(As + ACH);
#pragma unroll
    for (int ks = 0; ks < PBK / 16; ++ks) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[swzc<8>(wm * TM + i * 32 + l32, 2 * ks + lh)]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 32 + l32;
        const uint2 cw = *(const uint2*)(Bb + (r * 4 + (ks ^ ((r >> 2) & 3))) * 16 + 8 * lh);
        const float scf = e8m0_to_f32(sc[j][ks >> 1]);
        uint32_t v[4];
        dq4(cw.x, scf, v);
        dq4(cw.y, scf, v + 2);
        bfr[j] = __builtin_bit_cast(bf16x8, make_uint4(v[0], v[1], v[2], v[3]));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // split-K partials: register r of lane l = C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
  float* C = (float*)g.C + (size_t)split * g.M * g.ldc;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) C[(size_t)m * g.ldc + n_tile * BN + wn * TN + j * 32 + l32] = acc[i][j][r];
    }
}

template <int BM, int BN, int WMW, int WNW, int STAGES>
static hipError_t go_mx(const GemmArgs& g, hipStream_t st) {
  dim3 grid(g.N / BN, (g.M + BM - 1) / BM, g.splits);
  hipLaunchKernelGGL((k_gemm_mx32<BM, BN, WMW, WNW, STAGES>), grid, dim3(GT), 0, st, g);
  return hipGetLastError();
}

// NVFP4 (W4A16) split-K tiles for decode-sized M, on v_mfma_f32_32x32x16_bf16: the
// MXFP8 tiles' design with 4-bit codes. The bf16 activations and the packed E2M1 codes
// (32 bytes per weight row per 64-wide slice) stream into an LDS ring; the E4M3 block
// scales of the next slice (one per 16 along K, i.e. one per k-step: four bytes per
// weight row) are loaded into registers a slice ahead. Each lane expands its 8 codes of
// a B fragment with the hardware fp4 -> float conversion, multiplies by the block scale
// times the power-of-two matrix scale (exact), and truncates to bf16 (exact: every such
// product is a bf16 value). Output: fp32 split-K partials (EPI_PARTIAL).
__device__ __forceinline__ float e4m3_scale_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

template <int BM, int BN, int WMW, int WNW, int STAGES>
__global__ __launch_bounds__(GT) void k_gemm_nv32(GemmArgs g) {
  constexpr int PBK = 64;
  constexpr int TM = BM / WMW, TN = BN / WNW;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * 8, BCH = BN * 2;   // 16-byte chunks of A (bf16) / B (packed codes)
  constexpr int NINST = (ACH + BCH) / 64;
  constexpr int MAXI = (NINST + 3) / 4;
  static_assert(WMW * WNW == 4 && TM % 32 == 0 && TN % 32 == 0, "tile");
  static_assert(ACH % 64 == 0 && BCH % 64 == 0, "tile rows");
  static_assert((STAGES - 2) * MAXI <= 31 && STAGES >= 2, "pipeline");
  __shared__ __align__(16) uint4 sm[STAGES][ACH + BCH];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int n_tile = blockIdx.x, m0 = blockIdx.y * BM, split = blockIdx.z;
  const int Ks = g.K / g.splits, kbeg = split * Ks, nk = Ks / PBK;
  const bf16_t* A = (const bf16_t*)g.A;
  const uint8_t* B = (const uint8_t*)g.B;
  const int my_inst = (NINST - wave + 3) / 4;
  const int l32 = lane & 31, lh = lane >> 5;
  const float gsc = g.Bg[0];

  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int q = 0; q < MAXI; ++q) {
      const int inst = wave + 4 * q;
      if (inst < NINST) {
        const int sidx = inst * 64 + lane;
        const void* src;
        if (sidx < ACH) {  // A row r, chunk c (8 bf16)
          const int r = sidx >> 3, c = swzc<8>(r, sidx & 7) - r * 8;
          src = A + (size_t)min(m0 + r, g.M - 1) * g.lda + k0 + 8 * c;
        } else {           // B row r, chunk c (32 codes); chunk slot c ^ ((r >> 3) & 1)
          const int s2 = sidx - ACH, r = s2 >> 1, c = (s2 & 1) ^ ((r >> 3) & 1);
          src = B + (size_t)(n_tile * BN + r) * (g.K / 2) + k0 / 2 + 16 * c;
        }
        __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)(&sm[slot][inst * 64]), 16, 0, 0);
      }
    }
  };
  // E4M3 scales of B fragment j for the four k-steps of slice k0, one byte each
  auto ldscale = [&](int k0, uint32_t (&sc)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n_tile * BN + wn * TN + j * 32 + l32;
      sc[j] = *(const uint32_t*)(g.Bs + (size_t)n * (g.K / 16) + k0 / 16);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The scale loads of slice it+1 are issued after the tile loads of this step, so the
  // wait below (which counts only tile loads as newer than tile it) is conservative.
  uint32_t scn[FN];
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, kbeg + PBK * st);
  ldscale(kbeg, scn);
  for (int it = 0; it < nk; ++it) {
    wait_vmcnt(min(STAGES - 2, nk - 1 - it) * my_inst);
    __syncthreads();
    if (it + STAGES - 1 < nk) issue((it + STAGES - 1) % STAGES, kbeg + PBK * (it + STAGES - 1));
    uint32_t sc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) sc[j] = scn[j];
    if (it + 1 < nk) ldscale(kbeg + PBK * (it + 1), scn);
    const uint4* As = sm[it % STAGES];
    const unsigned char* Bb = (const unsigned char*)(As + ACH);
#pragma unroll
    for (int ks = 0; ks < PBK / 16; ++ks) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[swzc<8>(wm * TM + i * 32 + l32, 2 * ks + lh)]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 32 + l32;
        // codes of K elements 16 ks + 8 lh .. + 7: bytes 8 ks + 4 lh .. + 3 of the row
        const uint32_t cw = *(const uint32_t*)(Bb + (r * 2 + ((ks >> 1) ^ ((r >> 3) & 1))) * 16 + 8 * (ks & 1) + 4 * lh);
        const float S = e4m3_scale_f32((sc[j] >> (8 * ks)) & 0xFF) * gsc;
        uint32_t v[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          f32x2 f;
          if (b == 0) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
          else if (b == 1) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
          else if (b == 2) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
          else f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
          const float x0 = f[0] * S, x1 = f[1] * S;
          v[b] = (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xFFFF0000u);
        }
        bfr[j] = __builtin_bit_cast(bf16x8, make_uint4(v[0], v[1], v[2], v[3]));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // split-K partials: register r of lane l = C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
  float* C = (float*)g.C + (size_t)split * g.M * g.ldc;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) C[(size_t)m * g.ldc + n_tile * BN + wn * TN + j * 32 + l32] = acc[i][j][r];
    }
}

template <int BM, int BN, int WMW, int WNW, int STAGES>
static hipError_t go_nv(const GemmArgs& g, hipStream_t st) {
  dim3 grid(g.N / BN, (g.M + BM - 1) / BM, g.splits);
  hipLaunchKernelGGL((k_gemm_nv32<BM, BN, WMW, WNW, STAGES>), grid, dim3(GT), 0, st, g);
  return hipGetLastError();
}

template <int BM, int BN, int WMW, int WNW, int EPI, int STAGES, int PBK = 32>
static hipError_t go_pipe(const GemmArgs& g, hipStream_t st, int ntiles_n) {
  dim3 grid(ntiles_n, (g.M + BM - 1) / BM, g.splits);
  hipLaunchKernelGGL((k_gemm_pipe<BM, BN, WMW, WNW, EPI, STAGES, PBK>), grid, dim3(GT), 0, st, g);
  return hipGetLastError();
}

template <int BM, int BN, int WMW, int WNW, int EPI, int STAGES>
static hipError_t go_pipe32(const GemmArgs& g, hipStream_t st, int ntiles_n) {
  dim3 grid(ntiles_n, (g.M + BM - 1) / BM);
  hipLaunchKernelGGL((k_gemm_pipe32<BM, BN, WMW, WNW, EPI, STAGES>), grid, dim3(WMW * WNW * 64), 0, st, g);
  return hipGetLastError();
}

// compute units of the current device (one ping-pong work-group fits a CU at a time)
static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0, n = 0;
    cus = hipGetDevice(&dev) == hipSuccess &&
                  hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
              ? n
              : 256;
  }
  return cus;
}

// Columns [0, 256 a) on 256x256 tiles and [256 a, n) on 256x160 tiles (a = 0 or
// 256 a = n: one launch). One work-group runs per CU, so a launch of t tiles takes
// ceil(t / CUs) rounds, and a 256-wide tile takes about 1.4 times as long as a 160-wide
// one (measured on the prefill shapes); a is the split with the fewest estimated tile
// times. For 4096 x 6400 (the [q|k|v|gate] projection of a 4096-token prefill) that is 15
// wide and 16 narrow column tiles, one round each, instead of two rounds of 25 wide ones.
static int pp_wide_columns(int M, int n) {
  const int mt = (M + 255) / 256, cus = device_cus();
  int best_a = -1;
  long best = 0;
  for (int a = n / 256; a >= 0; --a) {
    const int rest = n - 256 * a;
    if (rest % 160) continue;
    const long t = 14L * ((a * mt + cus - 1) / cus) + 10L * ((rest / 160 * mt + cus - 1) / cus);
    if (best_a < 0 || t < best) best = t, best_a = a;
  }
  return best_a;
}

// Large-M (prefill) tiles for bf16 weights over n output columns (for SwiGLU, gate and
// up columns together): SwiGLU on 256x256 ping-pong tiles; the other epilogues on
// 256x256 and/or 256x160 ping-pong tiles as pp_wide_columns splits the columns; the
// pipelined 256x256 tiles when K has an odd number of 64-wide slices;
// hipErrorNotSupported when no tile shape divides n or the sizes need offsets beyond 32
// bits.
template <int EPI>
static hipError_t go_big(const GemmArgs& g, hipStream_t st, int n) {
  // these kernels address A and B with 32-bit byte offsets, and store bf16 outputs as
  // 16-byte chunks
  if ((long)g.N * g.K >= (1L << 30) || g.lda >= (1 << 20)) return hipErrorNotSupported;
  if (EPI != EPI_F32 && (g.ldc % 8 != 0 || ((uintptr_t)g.C & 15) != 0)) return hipErrorNotSupported;
  const bool pp = (g.K / BK) % 2 == 0;  // the ping-pong tiles take K slices in pairs
  const int mt = (g.M + 255) / 256;
  if constexpr (EPI == EPI_SWIGLU) {
    if (pp && n % 256 == 0) {
      hipLaunchKernelGGL((k_gemm_pp<256, EPI>), dim3(n / 256, mt), dim3(512), 0, st, g);
      return hipGetLastError();
    }
  } else if (pp) {
    const int a = pp_wide_columns(g.M, n);
    if (a >= 0) {
      if (a > 0) {
        GemmArgs w = g;
        w.N = 256 * a;
        hipLaunchKernelGGL((k_gemm_pp<256, EPI>), dim3(a, mt), dim3(512), 0, st, w);
      }
      if (256 * a < n) {
        GemmArgs r = g;
        const size_t esz = EPI == EPI_F32 ? 4 : 2;
        r.B = (const bf16_t*)g.B + (size_t)256 * a * g.K;
        r.C = (char*)g.C + (size_t)256 * a * esz;
        r.N = n - 256 * a;
        hipLaunchKernelGGL((k_gemm_pp<160, EPI>), dim3(r.N / 160, mt), dim3(512), 0, st, r);
      }
      return hipGetLastError();
    }
  }
  if (n % 256 == 0) return go_pipe32<256, 256, 2, 4, EPI, 2>(g, st, n / 256);
  return hipErrorNotSupported;
}

// Register-staged tiles: MXFP8 split-K when N is not a multiple of 128, and the bf16
// shapes the ping-pong tiles cannot take.
template <int BM, int BN, int WMW, int WNW, int EPI, int WF>
static hipError_t go(const GemmArgs& g, hipStream_t st, int ntiles_n) {
  dim3 grid(ntiles_n, (g.M + BM - 1) / BM, g.splits);
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WMW, WNW, EPI, WF>), grid, dim3(GT), 0, st, g);
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
  // quantised weights at large M: the caller expands them to bf16 first
  if ((g.wfmt == W_NVFP4 || g.wfmt == W_MXFP8) && g.epi != EPI_PARTIAL) return hipErrorInvalidValue;
  const bool bf = g.wfmt == W_BF16;  // bf16 weights: direct-to-LDS pipeline
  switch (g.epi) {
    case EPI_PARTIAL:  // small M (decode): stream the weights, split K
      if (g.N % 64) return hipErrorInvalidValue;
      if (bf) {
        if (g.M <= 32 && (g.K / g.splits == 256 || g.K / g.splits == 512)) {
          dim3 grid(g.N / 64, g.splits);
          const bool frag = g.Bf != nullptr;
          if (g.K / g.splits == 512) {
            if (frag) hipLaunchKernelGGL((k_gemv<16, true>), grid, dim3(256), 0, st, g);
            else hipLaunchKernelGGL((k_gemv<16, false>), grid, dim3(256), 0, st, g);
          } else {
            if (frag) hipLaunchKernelGGL((k_gemv<8, true>), grid, dim3(256), 0, st, g);
            else hipLaunchKernelGGL((k_gemv<8, false>), grid, dim3(256), 0, st, g);
          }
          return hipGetLastError();
        }
        if (g.M <= 32) return go_pipe<32, 64, 1, 4, EPI_PARTIAL, 4, 64>(g, st, g.N / 64);
        if (g.M <= 64) return go_pipe<64, 64, 1, 4, EPI_PARTIAL, 4, 64>(g, st, g.N / 64);
        return go_pipe<128, 64, 1, 4, EPI_PARTIAL, 3, 64>(g, st, g.N / 64);
      }
      if (g.wfmt == W_NVFP4) {  // 128 weight rows per tile
        if (g.N % 128 || (g.K / g.splits) % 64 || !g.Bs || !g.Bg) return hipErrorInvalidValue;
        if (g.M <= 32) return go_nv<32, 128, 1, 4, 4>(g, st);
        return go_nv<64, 128, 1, 4, 4>(g, st);
      }
      // 16-byte code and activation loads, 4-byte scale loads
      if (g.M > 32 && g.M <= 128 && g.K % (128 * g.splits) == 0 && gemv_mx_nch_ok(g.K / (128 * g.splits)) &&
          g.Bs && ((uintptr_t)g.Bs & 3) == 0 && ((uintptr_t)g.B & 15) == 0 && ((uintptr_t)g.A & 15) == 0 &&
          g.lda % 8 == 0) {
        dim3 grid(g.N / 64, g.splits);
        switch (g.K / (128 * g.splits)) {
          case 2: hipLaunchKernelGGL((k_gemv_mx<2>), grid, dim3(256), 0, st, g); break;
          case 4: hipLaunchKernelGGL((k_gemv_mx<4>), grid, dim3(256), 0, st, g); break;
          case 5: hipLaunchKernelGGL((k_gemv_mx<5>), grid, dim3(256), 0, st, g); break;
          case 8: hipLaunchKernelGGL((k_gemv_mx<8>), grid, dim3(256), 0, st, g); break;
          default: hipLaunchKernelGGL((k_gemv_mx<10>), grid, dim3(256), 0, st, g); break;
        }
        return hipGetLastError();
      }
      if (g.N % 128 == 0) {  // MXFP8: 128 weight rows per tile
        if (g.M <= 32) return go_mx<32, 128, 1, 4, 4>(g, st);
        return go_mx<64, 128, 1, 4, 4>(g, st);
      }
      if (g.M <= 32) return go<32, 64, 1, 4, EPI_PARTIAL, W_MXFP8>(g, st, g.N / 64);
      if (g.M <= 64) return go<64, 64, 1, 4, EPI_PARTIAL, W_MXFP8>(g, st, g.N / 64);
      return go<128, 64, 1, 4, EPI_PARTIAL, W_MXFP8>(g, st, g.N / 64);
    case EPI_STORE_ACT: {
      if (g.splits != 1) return hipErrorInvalidValue;
      const hipError_t e = go_big<EPI_STORE_ACT>(g, st, g.N);
      if (e != hipErrorNotSupported) return e;
      if (g.N % 128) return hipErrorInvalidValue;
      return go<128, 128, 2, 2, EPI_STORE_ACT, W_BF16>(g, st, g.N / 128);
    }
    case EPI_F32: {  // large M: fp32 output for the nGPT update
      if (g.splits != 1) return hipErrorInvalidValue;
      const hipError_t e = go_big<EPI_F32>(g, st, g.N);
      if (e != hipErrorNotSupported) return e;
      if (g.N % 128) return hipErrorInvalidValue;
      return go<128, 128, 2, 2, EPI_F32, W_BF16>(g, st, g.N / 128);
    }
    case EPI_SWIGLU: {
      if (g.n_half % 64 || g.splits != 1) return hipErrorInvalidValue;
      const hipError_t e = go_big<EPI_SWIGLU>(g, st, 2 * g.n_half);  // tiles interleave gate and up halves
      if (e != hipErrorNotSupported) return e;
      return go<128, 128, 2, 2, EPI_SWIGLU, W_BF16>(g, st, g.n_half / 64);
    }
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dory
