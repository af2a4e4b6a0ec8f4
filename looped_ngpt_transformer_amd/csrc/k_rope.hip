// RoPE + per-head QK normalisation + KV-cache write, and small page-table kernels.
//
// For each row (token at position p) of the fused [q | k | v | gate] projection:
//  * q (Hq heads) and k (Hkv heads) are rotated: pairs (i, i + d/2) by the angle
//    p * theta^(-2i/d), theta = 1e7 on full-attention layers and 1e4 on sliding ones
//    (MXFP8 article, rope_parameters; arXiv §3.4);
//  * with QK normalisation each rotated head is L2-normalised and scaled by s_qk
//    (arXiv §2: query-key scale of the nGPT backbone);
//  * k and v go to the row's page slot of the (layer, KV slot) stream; q goes to the
//    attention's input (the gate pre-activation is read in place by the attention).
// The frequencies theta^(-2i/d) come from a table computed on the host in double; the
// angle is formed and reduced modulo 2*pi in double precision (positions reach 262144),
// then sin/cos are taken in float.
#include "common.h"
#include "kernels.h"

namespace dory {

// The page slot of token pos in a (sequence, stream), and its K / V blocks of one head.
template <typename KV>
__device__ __forceinline__ KV* kv_page(const KVLayout& kv, int seq, int stream, int pos) {
  const int lp = pos / PAGE;
  const int32_t page =
      kv.table[((size_t)seq * kv.n_streams + stream) * kv.tab_len + (lp % kv.ring)];
  return (KV*)kv.pool + (size_t)page * kv.page_elems;
}
template <typename KV>
__device__ __forceinline__ KV* kv_kblock(KV* page, const KVLayout& kv, int head) {
  return page + (size_t)head * PAGE * kv.d;
}
template <typename KV>
__device__ __forceinline__ KV* kv_vblock(KV* page, const KVLayout& kv, int head) {
  return page + (size_t)(kv.Hkv + head) * PAGE * kv.d;
}

// grid (M rows, head groups + 1): block y < n_hb rotates heads 4y .. 4y+3 (one per wave,
// queries then keys); the last block copies v to the cache.
template <typename OUT>
__global__ __launch_bounds__(256) void k_rope_kv(RopeArgs a) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int d = a.d, half = d / 2;
  const int p = a.pos[m];
  const int seq = a.row_seq[m];
  const size_t rowoff = (size_t)m * a.Nqkvg;
  const size_t split_stride = (size_t)a.M * a.Nqkvg;
  auto in = [&](int col) -> float {
    if (a.in_f32) {
      const float* f = (const float*)a.qkvg;
      float t = 0.f;
      for (int s = 0; s < a.splits; ++s) t += f[s * split_stride + rowoff + col];
      return t;
    }
    return bf2f(((const bf16_t*)a.qkvg)[rowoff + col]);
  };
  const int n_heads = a.Hq + a.Hkv;
  const int n_hb = (n_heads + 3) / 4;
  if ((int)blockIdx.y < n_hb) {
    const int h = blockIdx.y * 4 + wave;
    if (h >= n_heads) return;
    const bool is_q = h < a.Hq;
    const int col0 = is_q ? h * d : a.Hq * d + (h - a.Hq) * d;
    float r[4];
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = lane + j * WAVE;
      if (i < half) {
        // angle p * theta^(-2i/d) in double, reduced modulo 2*pi before the float sin/cos
        double ang = (double)p * a.freq[i];
        ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        const float x1 = in(col0 + i), x2 = in(col0 + i + half);
        r[2 * j] = x1 * cs - x2 * sn;
        r[2 * j + 1] = x1 * sn + x2 * cs;
        sq += r[2 * j] * r[2 * j] + r[2 * j + 1] * r[2 * j + 1];
      } else {
        r[2 * j] = r[2 * j + 1] = 0.f;
      }
    }
    float sc = 1.f;
    if (a.qk_norm) sc = inv_norm(wave_sum(sq));
    OUT* qo = (OUT*)a.q_out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = lane + j * WAVE;
      if (i >= half) continue;
      float v1 = r[2 * j] * sc, v2 = r[2 * j + 1] * sc;
      if (a.qk_norm) {
        v1 *= a.s_qk[i];
        v2 *= a.s_qk[i + half];
      }
      if (is_q) {
        const size_t o = (size_t)m * a.Hq * d + (size_t)h * d;
        st<OUT>(qo, o + i, v1);
        st<OUT>(qo, o + i + half, v2);
      } else {
        OUT* kb = kv_kblock(kv_page<OUT>(a.kv, seq, a.stream_idx, p), a.kv, h - a.Hq);
        st<OUT>(kb, kv_k_off(p % PAGE, i, d), v1);
        st<OUT>(kb, kv_k_off(p % PAGE, i + half, d), v2);
      }
    }
    return;
  }
  // v -> V page (unrotated); the gate stays in the projection output
  const int vcol0 = a.Hq * d + a.Hkv * d;
  OUT* pgp = kv_page<OUT>(a.kv, seq, a.stream_idx, p);
  for (int c = threadIdx.x; c < a.Hkv * d; c += blockDim.x) {
    const int hk = c / d, j = c % d;
    st<OUT>(kv_vblock(pgp, a.kv, hk), kv_v_off(p % PAGE, j, d), in(vcol0 + c));
  }
}

hipError_t launch_rope_kv(const RopeArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (a.d > 256 || !a.freq) return hipErrorInvalidValue;
  dim3 grid(a.M, (a.Hq + a.Hkv + 3) / 4 + 1);
  if (a.kv.act == ACT_F32) {
    if (!a.in_f32) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_rope_kv<float>, grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_rope_kv<bf16_t>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------- page tables
__global__ void k_apply_deltas(int32_t* table, const int32_t* deltas, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) table[deltas[2 * i]] = deltas[2 * i + 1];
}

hipError_t launch_apply_deltas(int32_t* table, const int32_t* deltas, int n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_apply_deltas, dim3((n + 255) / 256), dim3(256), 0, st, table, deltas, n);
  return hipGetLastError();
}

// Copy seeded K/V rows [n, Hkv, d] into the pages of one (sequence, stream).
template <typename T>
__global__ __launch_bounds__(256) void k_fill_kv(KVLayout kv, int seq, int stream, int pos0,
                                                 int n, const T* k, const T* v) {
  const int r = blockIdx.x;  // row
  if (r >= n) return;
  const int p = pos0 + r;
  const int hd = kv.Hkv * kv.d;
  T* pgp = kv_page<T>(kv, seq, stream, p);
  for (int c = threadIdx.x; c < hd; c += blockDim.x) {
    const int hk = c / kv.d, j = c % kv.d;
    kv_kblock(pgp, kv, hk)[kv_k_off(p % PAGE, j, kv.d)] = k[(size_t)r * hd + c];
    kv_vblock(pgp, kv, hk)[kv_v_off(p % PAGE, j, kv.d)] = v[(size_t)r * hd + c];
  }
}

hipError_t launch_fill_kv(const KVLayout& kv, int seq_slot, int stream_idx, int pos0, int n,
                          const void* k, const void* v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (kv.act == ACT_F32)
    hipLaunchKernelGGL(k_fill_kv<float>, dim3(n), dim3(256), 0, st, kv, seq_slot, stream_idx,
                       pos0, n, (const float*)k, (const float*)v);
  else
    hipLaunchKernelGGL(k_fill_kv<bf16_t>, dim3(n), dim3(256), 0, st, kv, seq_slot, stream_idx,
                       pos0, n, (const bf16_t*)k, (const bf16_t*)v);
  return hipGetLastError();
}

}  // namespace dory
