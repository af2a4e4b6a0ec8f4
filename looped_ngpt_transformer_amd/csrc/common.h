// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dory {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an IEEE float)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr int PAGE = 64;  // tokens per KV page
constexpr float NORM_EPS = 1e-12f;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32, one instruction)
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two floats -> packed bf16 pair (a in the low half), round to nearest even, with the
// hardware conversion (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> __device__ __forceinline__ float ld(const T* p, size_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, size_t i) { return bf2f(p[i]); }

template <typename T> __device__ __forceinline__ void st(T* p, size_t i, float v);
template <> __device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, size_t i, float v) { p[i] = f2bf(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
  return v;
}

// Sum over all threads of a block of NW waves; `red` is LDS scratch of >= NW floats.
// Every thread gets the total. Contains barriers: call from uniform control flow.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += red[i];
  return t;
}

// ---------------------------------------------------------------- KV page layout
// A page holds 64 tokens of one (sequence, layer, slot) stream: for each KV head a K
// block of 64 x d elements, then for each KV head a V block of d x 64 elements. Both
// blocks are stored as 8-element chunks in the order the attention MFMAs consume them,
// so that every 16 x 32 operand fragment is 64 consecutive chunks (1 KiB in bf16):
//  * K chunk (token t, channels 8 cc .. + 7): half hf = t / 32, u = t % 32, fragment
//    (kb = (u / 4) % 2, c = cc / 4), lane (lk = cc % 4, lq = 4 (u / 8) + u % 4).
//    The rows of a 16-key fragment are tokens 8 (lq / 4) + 4 kb + lq % 4, so the S^T
//    accumulators of lane (lq, lk) cover the 8 consecutive tokens 8 lk .. + 7.
//  * V chunk (channel ch, tokens 32 hf + 8 lk .. + 7): fragment (hf, cb = ch / 16),
//    lane (lk, lq = ch % 16), the 8 tokens in order.
// d must be a multiple of 32. Offsets are in elements within the head's block.
__device__ __forceinline__ int kv_k_off(int t, int ch, int d) {
  const int hf = t >> 5, u = t & 31;
  const int lq = ((u >> 3) << 2) | (u & 3), kb = (u >> 2) & 1;
  const int cc = ch >> 3;
  const int chunk = (((hf * 2 + kb) * (d >> 5) + (cc >> 2)) * 4 + (cc & 3)) * 16 + lq;
  return chunk * 8 + (ch & 7);
}
__device__ __forceinline__ int kv_v_off(int t, int ch, int d) {
  const int hf = t >> 5, u = t & 31;
  const int chunk = ((hf * (d >> 4) + (ch >> 4)) * 4 + (u >> 3)) * 16 + (ch & 15);
  return chunk * 8 + (u & 7);
}
// Inverses for whole chunks q: K chunk -> (token, first channel); V chunk -> (channel,
// first token).
__device__ __forceinline__ void kv_k_chunk(int q, int d, int& t, int& ch) {
  const int DC = d >> 5;
  const int lq = q & 15, lk = (q >> 4) & 3, c = (q >> 6) % DC, kb = (q / (64 * DC)) & 1,
            hf = q / (128 * DC);
  t = 32 * hf + 8 * (lq >> 2) + 4 * kb + (lq & 3);
  ch = 8 * (4 * c + lk);
}
__device__ __forceinline__ void kv_v_chunk(int q, int d, int& ch, int& t) {
  const int CB = d >> 4;
  const int lq = q & 15, lk = (q >> 4) & 3, cb = (q >> 6) % CB, hf = q / (64 * CB);
  ch = 16 * cb + lq;
  t = 32 * hf + 8 * lk;
}

__device__ __forceinline__ float inv_norm(float sumsq) { return 1.0f / fmaxf(sqrtf(sumsq), NORM_EPS); }

// Sum of the n split-K partials p[0], p[stride], ..., p[(n - 1) stride]: the loads are
// issued eight at a time, so a lane waits for memory about n / 8 times instead of n.
__device__ __forceinline__ float sum_splits(const float* p, size_t stride, int n) {
  float t = 0.f;
  for (int s0 = 0; s0 < n; s0 += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = s0 + q < n ? p[(size_t)(s0 + q) * stride] : 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) t += v[q];
  }
  return t;
}

// 1 / (1 + e^-x) and x / (1 + e^-x) with the hardware reciprocal (about 1 ulp; every
// use ends in a bf16 value or a product with one), in place of an IEEE division
__device__ __forceinline__ float sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
__device__ __forceinline__ float silu(float x) { return x * sigmoid(x); }

// sigmoid gate value for (row m, channel c) from the projection output (bf16 [M, ld]
// or float split partials [splits][M][ld])
__device__ __forceinline__ float gate_at(const void* g, int f32, int ld, int splits, size_t sstride,
                                         int m, int c) {
  float x;
  if (f32) {
    x = sum_splits((const float*)g + (size_t)m * ld + c, sstride, splits);
  } else {
    x = bf2f(((const bf16_t*)g)[(size_t)m * ld + c]);
  }
  return sigmoid(x);
}

}  // namespace dory
