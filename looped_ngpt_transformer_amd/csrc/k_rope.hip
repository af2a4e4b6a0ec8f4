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
// queries then keys); the last block copies v to the cache. A lane takes up to 4 input
// columns (channels lane and lane + 64 of both halves, or up to 4 v columns) and requests
// every split partial of all of them before summing any (each column's sum in split
// order), so the partial sums cost one round trip to memory instead of one per column.
template <typename OUT>
__global__ __launch_bounds__(256) void k_rope_kv(RopeArgs a) {
  constexpr int NC = 4;  // input columns per lane
  const int m = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int d = a.d, half = d / 2;
  const int p = a.pos[m];
  const int seq = a.row_seq[m];
  const size_t rowoff = (size_t)m * a.Nqkvg;
  const size_t split_stride = (size_t)a.M * a.Nqkvg;
  // x[c] = input column col[c] (summed over the splits) where ok[c]
  auto gather = [&](const int (&col)[NC], const bool (&ok)[NC], float (&x)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) x[c] = 0.f;
    if (!a.in_f32) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (ok[c]) x[c] = bf2f(((const bf16_t*)a.qkvg)[rowoff + col[c]]);
      return;
    }
    const float* base = (const float*)a.qkvg + rowoff;
    // the split offsets in vector registers: eight scalar 64-bit bases would not fit
    size_t sstr = split_stride;
    asm volatile("" : "+v"(sstr));
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      float v[8][NC];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          v[q][c] = (s0 + q < a.splits && ok[c]) ? base[(size_t)(s0 + q) * sstr + col[c]] : 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c) x[c] += v[q][c];
    }
  };
  const int n_heads = a.Hq + a.Hkv;
  const int n_hb = (n_heads + 3) / 4;
  if ((int)blockIdx.y < n_hb) {
    const int h = blockIdx.y * 4 + wave;
    if (h >= n_heads) return;
    const bool is_q = h < a.Hq;
    const int col0 = is_q ? h * d : a.Hq * d + (h - a.Hq) * d;
    // columns: (i, i + half) for i = lane and lane + 64
    const int col[NC] = {col0 + lane, col0 + lane + half, col0 + lane + WAVE, col0 + lane + WAVE + half};
    const bool ok[NC] = {lane < half, lane < half, lane + WAVE < half, lane + WAVE < half};
    float x[NC];
    gather(col, ok, x);
    OUT* kb = is_q ? nullptr : kv_kblock(kv_page<OUT>(a.kv, seq, a.stream_idx, p), a.kv, h - a.Hq);
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
        const float x1 = x[2 * j], x2 = x[2 * j + 1];
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
        st<OUT>(kb, kv_k_off(p % PAGE, i, d), v1);
        st<OUT>(kb, kv_k_off(p % PAGE, i + half, d), v2);
      }
    }
    return;
  }
  // v -> V page (unrotated); the gate stays in the projection output
  const int vcol0 = a.Hq * d + a.Hkv * d;
  OUT* pgp = kv_page<OUT>(a.kv, seq, a.stream_idx, p);
  const int nv = a.Hkv * d;
  for (int c0 = threadIdx.x; c0 < nv; c0 += NC * blockDim.x) {
    int col[NC];
    bool ok[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ok[c] = c0 + c * (int)blockDim.x < nv;
      col[c] = vcol0 + c0 + c * blockDim.x;
    }
    float x[NC];
    gather(col, ok, x);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!ok[c]) continue;
      const int cc = c0 + c * blockDim.x;
      const int hk = cc / d, jj = cc % d;
      st<OUT>(kv_vblock(pgp, a.kv, hk), kv_v_off(p % PAGE, jj, d), x[c]);
    }
  }
}

// Prefill form: one work-group per (16-row quarter of a tile of <= 64 consecutive rows
// of one sequence, KV head), bf16 projection output. The (cos, sin) pairs of the rows
// come from the call's table (k_rope_table, once per forward call for both bases) into
// LDS; a 16-lane group then rotates one (row, head) with each lane holding 8
// consecutive channels of both halves of the RoPE pairs, so q and K are read and
// written as 16-byte chunks (a K chunk of the page is 8 channels of one token). With
// q_out null only K and V are handled: the MFMA attention rotates q as it loads it. V
// is transposed through LDS so that its page chunks (8 tokens of one channel) are
// written whole; chunks the quarter covers only in part are written element by element.
constexpr int RT_ROWS = 16;
constexpr int IPG = 5;  // (row, head) items a 16-lane group loads at once

template <int D>
__global__ __launch_bounds__(256) void k_rope_tile(RopeArgs a) {
  constexpr int HALF = D / 2, HC = HALF / 8;  // 16-byte chunks per half head
  constexpr int VR = D + 8;                   // padded bf16 row of the V tile
  static_assert(D % 16 == 0 && HC <= 16, "head dim");
  __shared__ __align__(16) bf16_t Vs[RT_ROWS * VR];
  __shared__ __align__(16) float2 CS[RT_ROWS * HALF];  // (cos, sin) per row and pair
  const int hk = blockIdx.y;
  const int32_t* tl = a.tiles + 4 * blockIdx.x;
  const int seq = tl[3];
  const int r0 = RT_ROWS * blockIdx.z;
  if (r0 >= tl[1]) return;
  const int nrows = min(RT_ROWS, tl[1] - r0);
  const int row0 = tl[0] + r0, pos0 = tl[2] + r0;
  const int G = a.Hq / a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, j = lane & 15;  // 16-lane group, chunk within the half
  const bf16_t* X = (const bf16_t*)a.qkvg;
  bf16_t* Q = (bf16_t*)a.q_out;

  // V rows -> LDS (16-byte chunks)
  const int vcol0 = a.Hq * D + a.Hkv * D + hk * D;
  for (int c = threadIdx.x; c < nrows * (D / 8); c += 256) {
    const int i = c / (D / 8), k8 = c % (D / 8);
    *(uint4*)(Vs + i * VR + 8 * k8) = *(const uint4*)(X + (size_t)(row0 + i) * a.Nqkvg + vcol0 + 8 * k8);
  }
  // (row, head) items of q heads hk*G .. hk*G+G-1 (unless q is left to the attention)
  // and K head hk: group gi = 4 wave + grp takes items gi, gi + 16, ...; the IPG items of
  // a batch are loaded before any is used, so that a group keeps IPG x 32 bytes per lane
  // in flight
  const int NQ = Q ? G : 0;  // q heads per row here
  const int items = nrows * (NQ + 1);
  const int gi = wave * 4 + grp;
  uint4 u1[IPG], u2[IPG];
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
      const int item = b0 + gi + 16 * u;
      if (item < items && j < HC) {
        const int i = item / (NQ + 1), hi = item % (NQ + 1);
        const int col0 = hi == NQ ? a.Hq * D + hk * D : (hk * G + hi) * D;
        const bf16_t* x = X + (size_t)(row0 + i) * a.Nqkvg + col0 + 8 * j;
        u1[u] = *(const uint4*)x;
        u2[u] = *(const uint4*)(x + HALF);
      }
    }
  };
  load_batch(0);
  // the lane's query-key scales (its 8 channels of each half), and the K pages of the
  // quarter's rows (at most two), looked up once
  float sq1[8], sq2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sq1[e] = sq2[e] = 1.f;
  if (a.qk_norm && j < HC) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq1[e] = a.s_qk[8 * j + e];
      sq2[e] = a.s_qk[HALF + 8 * j + e];
    }
  }
  bf16_t* const pg_lo = kv_page<bf16_t>(a.kv, seq, a.stream_idx, pos0);
  bf16_t* const pg_hi = kv_page<bf16_t>(a.kv, seq, a.stream_idx, pos0 + nrows - 1);
  const int lp_lo = pos0 / PAGE;
  auto page_of = [&](int p) { return p / PAGE == lp_lo ? pg_lo : pg_hi; };

  // (cos, sin) of the quarter's rows from the tile's block of the call's table, two pairs
  // per 16-byte load (while the first batch is in flight)
  const float* cst = a.cs + (size_t)blockIdx.x * 64 * D;
  for (int c = threadIdx.x; c < nrows * HALF / 2; c += 256) {
    const int i = c % nrows, k2 = c / nrows;
    *(float4*)(CS + i * HALF + 2 * k2) = *(const float4*)(cst + 4 * (64 * k2 + r0 + i));
  }
  __syncthreads();

  // rotation + norm, one item per 16-lane group (lanes j < HC hold chunk j of both halves)
  for (int b0 = 0; b0 < items; b0 += 16 * IPG) {
    if (b0 > 0) load_batch(b0);
#pragma unroll
    for (int u = 0; u < IPG; ++u) {
      const int item = b0 + gi + 16 * u;
      if (item >= items) break;  // uniform over the 16-lane group
      const bool act = j < HC;
      const int i = item / (NQ + 1), hi = item % (NQ + 1);
      const bool is_k = hi == NQ;
      const int p = pos0 + i;
      float r1[8], r2[8];
      float sq = 0.f;
      if (act) {
        const uint32_t w1[4] = {u1[u].x, u1[u].y, u1[u].z, u1[u].w}, w2[4] = {u2[u].x, u2[u].y, u2[u].z, u2[u].w};
        const float2* cs = CS + i * HALF + 8 * j;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x1 = __uint_as_float((e & 1) ? (w1[e / 2] & 0xFFFF0000u) : (w1[e / 2] << 16));
          const float x2 = __uint_as_float((e & 1) ? (w2[e / 2] & 0xFFFF0000u) : (w2[e / 2] << 16));
          const float2 t = cs[e];
          r1[e] = x1 * t.x - x2 * t.y;
          r2[e] = x1 * t.y + x2 * t.x;
          sq += r1[e] * r1[e] + r2[e] * r2[e];
        }
      }
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) sq += __shfl_xor(sq, m, 64);  // within the 16-lane group
      if (!act) continue;
      float sc = 1.f;
      if (a.qk_norm) sc = inv_norm(sq);
      uint32_t o1[4], o2[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float a0 = r1[e] * sc * sq1[e], a1 = r1[e + 1] * sc * sq1[e + 1];
        const float b0v = r2[e] * sc * sq2[e], b1 = r2[e + 1] * sc * sq2[e + 1];
        o1[e / 2] = pack_bf16x2(a0, a1);
        o2[e / 2] = pack_bf16x2(b0v, b1);
      }
      if (!is_k) {
        bf16_t* q = Q + (size_t)(row0 + i) * a.Hq * D + (hk * G + hi) * D;
        *(uint4*)(q + 8 * j) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
        *(uint4*)(q + HALF + 8 * j) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
      } else {
        bf16_t* kb = kv_kblock(page_of(p), a.kv, hk);
        *(uint4*)(kb + kv_k_off(p % PAGE, 8 * j, D)) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
        *(uint4*)(kb + kv_k_off(p % PAGE, HALF + 8 * j, D)) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
      }
    }
  }

  // V chunks: (group of 8 positions, channel); whole chunks when the quarter holds all 8
  const int g_lo = pos0 / 8, g_hi = (pos0 + nrows - 1) / 8;
  for (int c = threadIdx.x; c < (g_hi - g_lo + 1) * D; c += 256) {
    const int g8 = g_lo + c / D, ch = c % D;
    const int p0 = 8 * g8;
    bf16_t* vb = kv_vblock(page_of(p0), a.kv, hk);
    bf16_t* dst = vb + kv_v_off(p0 % PAGE, ch, D);
    if (p0 >= pos0 && p0 + 7 <= pos0 + nrows - 1) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        u[e / 2] = (uint32_t)Vs[(p0 + e - pos0) * VR + ch] | ((uint32_t)Vs[(p0 + e + 1 - pos0) * VR + ch] << 16);
      *(uint4*)dst = make_uint4(u[0], u[1], u[2], u[3]);
    } else {
      for (int e = 0; e < 8; ++e) {
        const int pp = p0 + e;
        if (pp >= pos0 && pp < pos0 + nrows) dst[e] = Vs[(pp - pos0) * VR + ch];
      }
    }
  }
}

hipError_t launch_rope_kv_tiles(const RopeArgs& a, hipStream_t st) {
  if (a.n_tiles == 0) return hipSuccess;
  if (a.in_f32 || a.kv.act != ACT_BF16 || !a.cs || !a.tiles || a.Hq % a.Hkv) return hipErrorInvalidValue;
  dim3 grid(a.n_tiles, a.Hkv, 64 / RT_ROWS);
  switch (a.d) {
    case 64: hipLaunchKernelGGL(k_rope_tile<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(k_rope_tile<128>, grid, dim3(256), 0, st, a); break;
    case 160: hipLaunchKernelGGL(k_rope_tile<160>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One thread per (base, tile, chunk of two pairs, row).
__global__ __launch_bounds__(256) void k_rope_table(const int32_t* tiles, int n_tiles, const double* freq, int half,
                                                    size_t ld, float* cs) {
  const int nk = half / 2;
  const size_t n = (size_t)n_tiles * nk * 64;
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < 2 * n; t += (size_t)gridDim.x * blockDim.x) {
    const int b = t >= n;
    const size_t q = t - b * n;
    const int r = (int)(q % 64), k = (int)((q / 64) % nk), tile = (int)(q / (64 * (size_t)nk));
    const int32_t* tl = tiles + 4 * tile;
    if (r >= tl[1]) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      double ang = (double)(tl[2] + r) * freq[128 * b + 2 * k + e];
      ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
      sincosf((float)ang, &v[2 * e + 1], &v[2 * e]);
    }
    *(float4*)(cs + b * ld + (size_t)tile * 256 * nk + 4 * (64 * (size_t)k + r)) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_rope_table(const int32_t* tiles, int n_tiles, const double* freq, int half, size_t ld, float* cs,
                             hipStream_t st) {
  if (n_tiles <= 0) return hipSuccess;
  if (half > 128 || half % 2 || (size_t)n_tiles * 128 * half > ld) return hipErrorInvalidValue;
  const size_t n = 2 * (size_t)n_tiles * (half / 2) * 64;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_rope_table, dim3(blocks), dim3(256), 0, st, tiles, n_tiles, freq, half, ld, cs);
  return hipGetLastError();
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
// One work-group per (table index, page) pair: install the entry and clear the newly
// allocated page, so that cache entries no token has written yet hold zeros (kernels
// may read them as MFMA operands with a zero weight; they must not be NaN or Inf).
__global__ __launch_bounds__(256) void k_apply_deltas(int32_t* table, const int32_t* deltas, int n,
                                                      uint4* pool, size_t page_chunks) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const int32_t page = deltas[2 * i + 1];
  if (threadIdx.x == 0) table[deltas[2 * i]] = page;
  uint4* p = pool + (size_t)page * page_chunks;
  for (size_t c = threadIdx.x; c < page_chunks; c += 256) p[c] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_apply_deltas(int32_t* table, const int32_t* deltas, int n, void* pool,
                               size_t page_bytes, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (page_bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_apply_deltas, dim3(n), dim3(256), 0, st, table, deltas, n, (uint4*)pool,
                     page_bytes / 16);
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
