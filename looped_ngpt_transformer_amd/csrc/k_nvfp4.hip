// NVFP4 weights (W4A16): E2M1 elements with an E4M3 scale per 16 along K and a power-of-
// two scale per matrix ("Dory1.0-4B" pages: NVFP4 is 4-bit block scaling with E2M1
// operands and E4M3 scale factors — paper summary, "NVFP4 quantisation and QAD"; used
// weight-only — model-card digest; quantised with dynamic MSE scale selection — arXiv
// summary §5.1-5.2). The quantiser and the expansion to bf16 for the prefill GEMMs; the
// decode GEMMs read the codes directly (k_gemm.hip).
#include "common.h"
#include "kernels.h"

namespace dory {

// value of a positive finite E4M3 code (OCP FN: bias 7, subnormals m 2^-9)
__device__ __forceinline__ float e4m3_pos_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// nearest E2M1 magnitude code of |x| (0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the even code,
// saturating at 6
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  uint32_t q = 0;
  q = a > 0.25f ? 1u : q;
  q = a >= 0.75f ? 2u : q;
  q = a > 1.25f ? 3u : q;
  q = a >= 1.75f ? 4u : q;
  q = a > 2.5f ? 5u : q;
  q = a >= 3.5f ? 6u : q;
  q = a > 5.0f ? 7u : q;
  return q;
}

__device__ __forceinline__ float e2m1_mag_value(uint32_t q) {
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6
  return q < 4 ? 0.5f * (float)q : (float)(2u << ((q - 4) >> 1)) * (1.0f + 0.5f * (float)(q & 1));
}

// amax of the matrix as the bits of a non-negative float (monotone as integers)
template <typename T>
__global__ __launch_bounds__(256) void k_nvfp4_amax(const T* w, int64_t n, uint32_t* amax_bits) {
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = fmaxf(m, fabsf(ld<T>(w, (size_t)i)));
  m = wave_max(m);
  if ((threadIdx.x & (WAVE - 1)) == 0) atomicMax(amax_bits, __float_as_uint(m));
}

// the matrix scale g = 2^ceil(log2(amax / 2688)) (1 for an all-zero matrix)
__device__ __forceinline__ float nvfp4_global(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  if (amax == 0.f) return 1.f;
  const float r = amax / 2688.f;
  int e;
  const float f = frexpf(r, &e);  // r = f 2^e, f in [0.5, 1)
  return ldexpf(1.f, f == 0.5f ? e - 1 : e);
}

// One thread per block of 16 elements: the E4M3 scale code with the smallest float32 sum
// of squared errors (equal sums keep the smaller code), then the 16 E2M1 codes. The
// error terms are rounded one by one in a fixed order (no contraction), so the choice is
// the same as any float32 evaluation in that order.
template <typename T>
__global__ __launch_bounds__(256) void k_nvfp4_quant(const T* w, int64_t rows, int64_t cols,
                                                     const uint32_t* amax_bits, uint8_t* codes, uint8_t* scales) {
#pragma clang fp contract(off)
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nb = rows * (cols / 16);
  if (b >= nb) return;
  const float g = nvfp4_global(*amax_bits);
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = ld<T>(w, (size_t)b * 16 + i);
  float best = INFINITY;
  uint32_t best_c = 1;
  for (uint32_t c = 1; c < 0x7F; ++c) {
    const float S = e4m3_pos_to_f32(c) * g;  // exact: g is a power of two
    float err = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float q = e2m1_mag_value(e2m1_mag(fabsf(x[i] / S)));
      const float d = copysignf(q, x[i]) * S - x[i];
      err = err + d * d;
    }
    if (err < best) {
      best = err;
      best_c = c;
    }
  }
  const float S = e4m3_pos_to_f32(best_c) * g;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = x[i] / S;
    const uint32_t code = e2m1_mag(fabsf(v)) | (signbit(v) ? 8u : 0u);
    if (i < 8) lo |= code << (4 * i);
    else hi |= code << (4 * (i - 8));
  }
  *(uint2*)(codes + (size_t)b * 8) = make_uint2(lo, hi);
  scales[b] = (uint8_t)best_c;
}

__global__ void k_nvfp4_finish(uint32_t* gword) {
  // the amax bits become the matrix scale
  gword[0] = __float_as_uint(nvfp4_global(gword[0]));
}

__global__ void k_zero_word(uint32_t* p) { p[0] = 0u; }

// W = e2m1 * e4m3 * g as bf16 (exact: every such product is a bf16 value), one thread
// per block of 16: 8 code bytes and a scale byte in, 32 bytes out.
__global__ __launch_bounds__(256) void k_nvfp4_expand(const uint8_t* codes, const uint8_t* scales, const float* g,
                                                      int64_t nb, bf16_t* out) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nb) return;
  const float S = e4m3_pos_to_f32(scales[b]) * g[0];
  const uint2 cw = *(const uint2*)(codes + (size_t)b * 8);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t word = i < 8 ? cw.x : cw.y;
    const uint32_t c0 = (word >> (4 * (i & 7))) & 15, c1 = (word >> (4 * ((i + 1) & 7))) & 15;
    const float v0 = copysignf(e2m1_mag_value(c0 & 7), (c0 & 8) ? -1.f : 1.f) * S;
    const float v1 = copysignf(e2m1_mag_value(c1 & 7), (c1 & 8) ? -1.f : 1.f) * S;
    o[i / 2] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
  }
  uint4* dst = (uint4*)(out + (size_t)b * 16);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_quantize_nvfp4(const void* w, int w_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, float* g, hipStream_t st) {
  const int64_t n = rows * cols, nb = n / 16;
  uint32_t* gw = (uint32_t*)g;
  hipLaunchKernelGGL(k_zero_word, dim3(1), dim3(1), 0, st, gw);
  if (n > 0) {
    const unsigned grid = (unsigned)std::min<int64_t>(2048, (n + 255) / 256);
    if (w_bf16) hipLaunchKernelGGL(k_nvfp4_amax<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)w, n, gw);
    else hipLaunchKernelGGL(k_nvfp4_amax<float>, dim3(grid), dim3(256), 0, st, (const float*)w, n, gw);
    const unsigned qb = (unsigned)((nb + 255) / 256);
    if (w_bf16)
      hipLaunchKernelGGL(k_nvfp4_quant<bf16_t>, dim3(qb), dim3(256), 0, st, (const bf16_t*)w, rows, cols, gw, codes,
                         scales);
    else
      hipLaunchKernelGGL(k_nvfp4_quant<float>, dim3(qb), dim3(256), 0, st, (const float*)w, rows, cols, gw, codes,
                         scales);
  }
  hipLaunchKernelGGL(k_nvfp4_finish, dim3(1), dim3(1), 0, st, gw);
  return hipGetLastError();
}

hipError_t launch_expand_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rows,
                               int64_t cols, void* out, hipStream_t st) {
  const int64_t nb = rows * (cols / 16);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_nvfp4_expand, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, codes, scales, g, nb,
                     (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace dory
