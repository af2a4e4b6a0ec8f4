// SwiGLU activation from split-K partial sums, and the MXFP8 weight quantiser.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dory {

// h = SiLU(gate) * up ("Dory1.0-4B" paper summary: SwiGLU MLP), from float partials
// [splits][M][2I] (gate columns [0, I), up columns [I, 2I)). The L2 norm before the down
// projection (arXiv §2) only scales the row, which the nGPT update's N(.) removes.
// grid (M, blocks per row): block b of a row covers columns [b*1024, (b+1)*1024).
template <typename T>
__global__ __launch_bounds__(256) void k_swiglu(const float* gu, int splits, int M, int I, T* h) {
  const int m = blockIdx.x, b = blockIdx.y;
  const size_t sstride = (size_t)M * 2 * I;
  const size_t row = (size_t)m * 2 * I;
  const int i1 = min(I, (b + 1) * 1024);
  for (int i = b * 1024 + threadIdx.x; i < i1; i += blockDim.x) {
    const float g = sum_splits(gu + row + i, sstride, splits);
    const float u = sum_splits(gu + row + I + i, sstride, splits);
    st<T>(h, (size_t)m * I + i, silu(g) * u);
  }
}

// I % 4 == 0: each thread owns 4 consecutive columns of gate and of up, and requests
// their partials of up to 8 splits at once (16-byte loads; summed in split order).
template <typename T>
__global__ __launch_bounds__(256) void k_swiglu4(const float* gu, int splits, int M, int I, T* h) {
  constexpr int QS = 8;
  const int m = blockIdx.x;
  const int i = 4 * (blockIdx.y * 256 + threadIdx.x);
  if (i >= I) return;
  const size_t sstride = (size_t)M * 2 * I;
  const float* p = gu + (size_t)m * 2 * I + i;
  float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += QS) {
    float4 vg[QS], vu[QS];
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      const bool ok = s0 + q < splits;
      vg[q] = ok ? *(const float4*)(p + (s0 + q) * sstride) : make_float4(0.f, 0.f, 0.f, 0.f);
      vu[q] = ok ? *(const float4*)(p + (s0 + q) * sstride + I) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      g[0] += vg[q].x; g[1] += vg[q].y; g[2] += vg[q].z; g[3] += vg[q].w;
      u[0] += vu[q].x; u[1] += vu[q].y; u[2] += vu[q].z; u[3] += vu[q].w;
    }
  }
  const size_t o = (size_t)m * I + i;
#pragma unroll
  for (int e = 0; e < 4; ++e) st<T>(h, o + e, silu(g[e]) * u[e]);
}

hipError_t launch_swiglu(const float* gu, int splits, int M, int I, void* h, int act,
                         hipStream_t st) {
  if (M == 0) return hipSuccess;
  if (I % 4 == 0) {
    const dim3 grid(M, (I / 4 + 255) / 256);
    if (act == ACT_F32)
      hipLaunchKernelGGL(k_swiglu4<float>, grid, dim3(256), 0, st, gu, splits, M, I, (float*)h);
    else
      hipLaunchKernelGGL(k_swiglu4<bf16_t>, grid, dim3(256), 0, st, gu, splits, M, I, (bf16_t*)h);
    return hipGetLastError();
  }
  const dim3 grid(M, (I + 1023) / 1024);
  if (act == ACT_F32)
    hipLaunchKernelGGL(k_swiglu<float>, grid, dim3(256), 0, st, gu, splits, M, I, (float*)h);
  else
    hipLaunchKernelGGL(k_swiglu<bf16_t>, grid, dim3(256), 0, st, gu, splits, M, I, (bf16_t*)h);
  return hipGetLastError();
}

// ------------------------------------------------------------------ MXFP8 quantiser
// OCP MX maximum scaling with group 32 along each row (arXiv §5.1-5.2: MXFP8 uses
// standard maximum scaling; MXFP8 article: group_size 32): shared exponent
// floor(log2(amax)) - 8 stored as an E8M0 byte (+127, clamped to [0, 254]; zero group
// -> 0); elements x / 2^e rounded to nearest-even E4M3 with saturation at 448.

// E4M3 code for a finite float that is already divided by the group scale.
__device__ __forceinline__ uint8_t e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7E;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal step 2^-9 (a * 2^9 is exact)
    code = (uint32_t)rintf(a * 512.f);  // 8 -> 0x08 = smallest normal: carry is correct
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6..8
    const float frac = a * __uint_as_float((uint32_t)(127 - e) << 23);  // [1, 2), exact
    const uint32_t m = (uint32_t)rintf((frac - 1.f) * 8.f);             // 0..8
    code = ((uint32_t)(e + 7) << 3) + m;  // m == 8 carries into the exponent
    if (code > 0x7E) code = 0x7E;
  }
  return (uint8_t)(code | sign);
}

template <typename T>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const T* w, int64_t rows, int64_t cols,
                                                     uint8_t* codes, uint8_t* scales) {
  // one lane per element; 32 consecutive lanes = one group
  const int64_t gid = (int64_t)blockIdx.x * (blockDim.x / 32) + threadIdx.x / 32;
  const int64_t groups = rows * (cols / 32);
  const int lane32 = threadIdx.x & 31;
  const bool valid = gid < groups;
  const int64_t e_idx = valid ? gid * 32 + lane32 : 0;
  const float x = valid ? ld<T>(w, (size_t)e_idx) : 0.f;
  float amax = fabsf(x);
#pragma unroll
  for (int msk = 16; msk >= 1; msk >>= 1) amax = fmaxf(amax, __shfl_xor(amax, msk, 32));
  if (!valid) return;
  int se;
  if (amax == 0.f) {
    se = -127;
  } else {
    int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    if (ex == 0) {  // subnormal float amax: floor(log2) from the mantissa
      ex = -126 - (__clz(__float_as_uint(amax) & 0x7FFFFF) - 9) - 1;
    } else {
      ex -= 127;
    }
    se = ex - 8;
    se = se < -127 ? -127 : (se > 127 ? 127 : se);
  }
  // x / 2^se exactly: multiply by 2^-se, split in two steps to stay in range
  const int h1 = -se / 2, h2 = -se - h1;
  const float xs = (x * exp2f((float)h1)) * exp2f((float)h2);
  codes[e_idx] = e4m3_rne(xs);
  if (lane32 == 0) scales[gid] = (uint8_t)(se + 127);
}

hipError_t launch_quantize_mxfp8(const void* w, int w_bf16, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t groups = rows * (cols / 32);
  if (groups == 0) return hipSuccess;
  const int64_t blocks = (groups + 7) / 8;
  if (w_bf16)
    hipLaunchKernelGGL(k_quant_mxfp8<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const bf16_t*)w, rows, cols, codes, scales);
  else
    hipLaunchKernelGGL(k_quant_mxfp8<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const float*)w, rows, cols, codes, scales);
  return hipGetLastError();
}

}  // namespace dory
