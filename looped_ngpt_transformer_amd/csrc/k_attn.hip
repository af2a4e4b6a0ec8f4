// Paged GQA attention over the KV cache, split over keys, plus the combine step.
//
// For a query row at position p and query head h (KV head h / (Hq/Hkv)): the visible
// keys are the cached entries j <= p, and p - j < W on sliding-window layers; the
// output is softmax_j(scale * q.k_j) weighted sum of v_j ("Dory1.0-4B": GQA with 16
// query / 4 KV heads, 3:1 sliding (W = 1024) / full attention — paper summary
// "technical novelty", MXFP8 article "hybrid attention").
// The combine step merges the per-split softmax partials, applies the sigmoid output
// gate elementwise and writes the per-head sum of squares of the gated output, from
// which the consumer forms the L2 norm before the output projection (arXiv §2).
//
// Work-group = (row, KV head, split); its 4 waves are the group's query heads, so
// each K/V page is read once for all of them. A page tile (64 keys of one KV head:
// K row-major and V channel-major, each contiguous in the page) is staged in LDS with
// coalesced 16-byte loads.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dory {

constexpr int ATT_THREADS = 256;
constexpr int ATT_MAXG = 4;     // query heads per KV head handled by one work-group
constexpr int ATT_MAXD = 256;
constexpr int ATT_MAX_SPLITS = 64;

template <typename T>
__global__ __launch_bounds__(ATT_THREADS) void k_attn_rows(AttnArgs a, int splits, int pps) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int d = a.d;
  const int G = a.Hq / a.Hkv;
  T* Ks = (T*)smem;                              // [64][d]
  T* Vs = Ks + PAGE * d;                         // [d][64] (channel-major, as in the page)
  float* qs = (float*)(Vs + PAGE * d);           // [G][d]
  float* part = qs + ATT_MAXG * d;               // [4][G][64] partial dots
  float* P = part + 4 * ATT_MAXG * PAGE;         // [G][64] probabilities

  const int m = blockIdx.x, hk = blockIdx.y, sp = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int p = a.pos[m];
  const int seq = a.row_seq[m];
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int pg_lo = lo / PAGE, pg_hi = p / PAGE;
  const int pa = pg_lo + sp * pps;
  const int pb = min(pg_hi, pa + pps - 1);

  const T* q = (const T*)a.q;
  for (int i = t; i < G * d; i += ATT_THREADS)
    qs[i] = ld<T>(q, (size_t)m * a.Hq * d + (size_t)(hk * G) * d + i);

  float m_run = -INFINITY, l_run = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};  // dims lane + 64 c, c < 4 (d <= 256)
  const int dq = d / 4;               // dims per QK quarter
  const int chunks = PAGE * d * (int)sizeof(T) / 16;  // 16-byte chunks per K (or V) page
  const int32_t* trow = a.kv.table + ((size_t)seq * a.kv.n_streams + a.stream_idx) * a.kv.tab_len;

  for (int pg = pa; pg <= pb; ++pg) {
    const int32_t page = trow[pg % a.kv.ring];
    const T* kp = (const T*)a.kv.pool + (size_t)page * a.kv.page_elems + (size_t)hk * PAGE * d;
    const T* vp = kp + (size_t)a.Hkv * PAGE * d;
    __syncthreads();  // previous tile fully consumed
    for (int c = t; c < chunks; c += ATT_THREADS) {
      ((uint4*)Ks)[c] = ((const uint4*)kp)[c];
      ((uint4*)Vs)[c] = ((const uint4*)vp)[c];
    }
    __syncthreads();
    {  // partial dots: key j = lane, dims [w*dq, (w+1)*dq) for every query head
      const int j = lane;
      float acc[ATT_MAXG] = {0.f, 0.f, 0.f, 0.f};
      for (int i = w * dq; i < (w + 1) * dq; ++i) {
        const float kv = ld<T>(Ks, (size_t)j * d + i);
#pragma unroll
        for (int g = 0; g < ATT_MAXG; ++g)
          if (g < G) acc[g] += qs[g * d + i] * kv;
      }
#pragma unroll
      for (int g = 0; g < ATT_MAXG; ++g)
        if (g < G) part[(w * ATT_MAXG + g) * PAGE + j] = acc[g];
    }
    __syncthreads();
    float corr = 1.f;
    if (w < G) {  // wave w = query head w of the group: online softmax over this tile
      const int j = lane;
      const int key = pg * PAGE + j;
      float s = -INFINITY;
      if (key >= lo && key <= p) {
        s = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) s += part[(c * ATT_MAXG + w) * PAGE + j];
        s *= a.scale;
      }
      const float tmax = wave_max(s);
      const float m_new = fmaxf(m_run, tmax);
      const float pe = (s == -INFINITY) ? 0.f : __expf(s - m_new);
      corr = (m_run == -INFINITY) ? 0.f : __expf(m_run - m_new);
      l_run = l_run * corr + wave_sum(pe);
      m_run = m_new;
      P[w * PAGE + j] = pe;
    }
    __syncthreads();
    if (w < G) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] *= corr;
      // only visible keys: entries outside [lo, p] may be unwritten (never multiplied,
      // so stale or uninitialised page contents cannot reach the sum)
      const int jlo = max(0, lo - pg * PAGE), jhi = min(PAGE - 1, p - pg * PAGE);
      for (int j = jlo; j <= jhi; ++j) {
        const float pj = P[w * PAGE + j];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = lane + c * 64;
          if (i < d) o[c] += pj * ld<T>(Vs, (size_t)i * PAGE + j);
        }
      }
    }
  }
  if (w < G) {
    const int h = hk * G + w;
    float* dst = a.part + (((size_t)m * a.Hq + h) * splits + sp) * (d + 2);
    if (lane == 0) {
      dst[0] = m_run;
      dst[1] = l_run;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = lane + c * 64;
      if (i < d) dst[2 + i] = o[c];
    }
  }
}

// Merge splits, apply the sigmoid gate, write o (act) and per-head sum of squares.
// One wave per (row, head): lane s < splits holds split s's weight exp(m_s - max) and
// l_s; the weights reach the other lanes by shuffles while each lane merges its channels.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int splits) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.M * a.Hq) return;
  const int m = wid / a.Hq, h = wid % a.Hq;
  const int d = a.d;
  const float* src = a.part + ((size_t)m * a.Hq + h) * splits * (d + 2);
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < splits; s0 += 64) {  // running max over all splits first
    const int s = s0 + lane;
    mx = fmaxf(mx, s < splits ? src[(size_t)s * (d + 2)] : -INFINITY);
  }
  mx = wave_max(mx);
  for (int s0 = 0; s0 < splits; s0 += 64) {
    const int s = s0 + lane;
    float wgt = 0.f, ls = 0.f;
    if (s < splits) {
      const float ms = src[(size_t)s * (d + 2)];
      wgt = ms == -INFINITY ? 0.f : __expf(ms - mx);
      ls = src[(size_t)s * (d + 2) + 1];
    }
    L += wave_sum(wgt * ls);
    const int n = min(64, splits - s0);
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float wj = __shfl(wgt, j, 64);
      if (wj == 0.f) continue;  // empty split (its o is zero): skip the loads
      const float* oj = src + (size_t)(s0 + j) * (d + 2) + 2;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = lane + 64 * c;
        if (i < d) o[c] += oj[i] * wj;
      }
    }
  }
  const float invL = 1.f / L;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = lane + 64 * c;
    if (i < d) {
      float ov = o[c] * invL;
      const size_t e = (size_t)m * a.Hq * d + (size_t)h * d + i;
      if (a.g) ov *= gate_at(a.g, a.g_f32, a.g_ld, a.g_splits, a.g_sstride, m, h * d + i);
      st<T>((T*)a.o, e, ov);
      sq += ov * ov;
    }
  }
  sq = wave_sum(sq);
  if (lane == 0) a.ss[(size_t)m * a.Hq + h] = sq;
}

// ------------------------------------------------------------- decode attention, MFMA
// One wave per (row, KV head, sub-split of the row's pages); no LDS and no barriers.
// The wave streams its pages straight from HBM, 32 keys at a time with the next 32
// in flight: K rows as MFMA A fragments (16 keys x 32 channels), V^T fragments from the
// channel-major V half of the page. S^T = K Q^T
// puts the 4 grouped query heads in the B operand (columns 4..15 are zero), and the
// probabilities feed O^T += V^T P^T from the S^T accumulators as in the prefill kernel.
// Keys outside [lo, p] get -inf logits and, on partial pages, zeroed V entries.
template <int D>
__global__ __launch_bounds__(256) void k_attn_decode(AttnArgs a, int nsub, int pps) {
  constexpr int G = 4, DC = D / 32, CB = D / 16;
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.M * a.Hkv * nsub) return;
  const int sub = wid % nsub, mh = wid / nsub;
  const int hk = mh % a.Hkv, m = mh / a.Hkv;
  const int lq = lane & 15, lk = lane >> 4;
  const int p = a.pos[m];
  const int seq = a.row_seq[m];
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int pg_lo = lo / PAGE, pg_hi = p / PAGE;
  const int pa = pg_lo + sub * pps;
  const int pb = min(pg_hi, pa + pps - 1);
  const int32_t* trow = a.kv.table + ((size_t)seq * a.kv.n_streams + a.stream_idx) * a.kv.tab_len;
  const bf16_t* pool = (const bf16_t*)a.kv.pool;

  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (lq < G) v = *(const uint4*)((const bf16_t*)a.q + (size_t)m * a.Hq * D + (size_t)(hk * G + lq) * D + 32 * c + 8 * lk);
    qf[c] = __builtin_bit_cast(bf16x8, v);
  }
  const float sl2 = a.scale * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Half-pages (32 keys) hp = 2 * page + hf. The fragments of half-page hp + 1 are
  // loaded into the second register set while hp is computed.
  struct Half {
    uint4 k[2][DC];   // K rows 32 hf + 16 kb + lq, channels 32 c + 8 lk .. + 7
    uint2 v[CB][2];   // V^T channel 16 cb + lq, keys 32 hf + 4 lk (+16) .. + 3
  };
  auto load = [&](int hp, Half& H) {
    const int pg = hp >> 1, hf = hp & 1;
    const int32_t page = trow[pg % a.kv.ring];
    const bf16_t* kp = pool + (size_t)page * a.kv.page_elems + (size_t)hk * PAGE * D;
    const bf16_t* vp = pool + (size_t)page * a.kv.page_elems + (size_t)a.Hkv * PAGE * D + (size_t)hk * D * PAGE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < DC; ++c)
        H.k[kb][c] = *(const uint4*)(kp + (size_t)(32 * hf + 16 * kb + lq) * D + 32 * c + 8 * lk);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const bf16_t* vr = vp + (size_t)(16 * cb + lq) * PAGE + 32 * hf + 4 * lk;
      H.v[cb][0] = *(const uint2*)vr;
      H.v[cb][1] = *(const uint2*)(vr + 16);
    }
  };
  auto compute = [&](int hp, const Half& H) {
    const int pg = hp >> 1, hf = hp & 1;
    const int kbase = pg * PAGE + 32 * hf;
    const bool whole = kbase >= lo && kbase + 31 <= p;
    f32x4 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c)
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, H.k[kb][c]), qf[c], st[kb], 0, 0, 0);
    }
    // S^T[key kbase + 16 kb + 4 lk + r][head lq]: online softmax for head lq
    float sv[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kbase + 16 * kb + 4 * lk + r;
        const bool vis = key >= lo && key <= p;
        sv[kb][r] = vis ? st[kb][r] * sl2 : -INFINITY;
        mt = fmaxf(mt, sv[kb][r]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float corr = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
    float pe[2][4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pe[kb][r] = sv[kb][r] == -INFINITY ? 0.f : exp2f(sv[kb][r] - m_new);
        ps += pe[kb][r];
      }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    m_run = m_new;
    uint32_t u[4];
    u[0] = (uint32_t)f2bf(pe[0][0]) | ((uint32_t)f2bf(pe[0][1]) << 16);
    u[1] = (uint32_t)f2bf(pe[0][2]) | ((uint32_t)f2bf(pe[0][3]) << 16);
    u[2] = (uint32_t)f2bf(pe[1][0]) | ((uint32_t)f2bf(pe[1][1]) << 16);
    u[3] = (uint32_t)f2bf(pe[1][2]) | ((uint32_t)f2bf(pe[1][3]) << 16);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(u[0], u[1], u[2], u[3]));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      uint2 v0 = H.v[cb][0], v1 = H.v[cb][1];
      if (!whole) {  // zero entries of keys outside [lo, p]
        uint32_t w4[4] = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = kbase + (e < 4 ? 4 * lk + e : 16 + 4 * lk + e - 4);
          if (key < lo || key > p) w4[e / 2] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        v0 = make_uint2(w4[0], w4[1]);
        v1 = make_uint2(w4[2], w4[3]);
      }
      o[cb] *= corr;
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y)), pf, o[cb], 0, 0, 0);
    }
  };

  const int h0 = 2 * pa, h1 = 2 * pb + 1;  // empty when pa > pb
  if (h0 <= h1) {
    Half A, B;
    load(h0, A);
    for (int hp = h0; hp <= h1; hp += 2) {
      if (hp + 1 <= h1) load(hp + 1, B);
      compute(hp, A);
      if (hp + 2 <= h1) load(hp + 2, A);
      if (hp + 1 <= h1) compute(hp + 1, B);
    }
  }
  if (lq < G) {
    const int h = hk * G + lq;
    float* dst = a.part + (((size_t)m * a.Hq + h) * nsub + sub) * (D + 2);
    if (lk == 0) {
      dst[0] = m_run;
      dst[1] = l_run;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[2 + 16 * cb + 4 * lk + r] = o[cb][r];
  }
}

static int attn_pages_max(int max_pos, int window) {
  const int lo = window > 0 ? (max_pos - window + 1 > 0 ? max_pos - window + 1 : 0) : 0;
  // worst case over rows with positions <= max_pos
  if (window > 0) return (window + PAGE - 2) / PAGE + 1;
  return max_pos / PAGE - lo / PAGE + 1;
}

static void attn_pick_splits(int M, int Hkv, int n_pages, size_t cap_floats, int Hq, int d,
                             int* splits, int* pps) {
  int s = 1;
  const int target_wg = 2048;
  while (s < ATT_MAX_SPLITS && s * 2 <= n_pages && (long)M * Hkv * s < target_wg) s *= 2;
  while (s > 1 && (size_t)M * Hq * s * (d + 2) > cap_floats) s /= 2;
  *pps = (n_pages + s - 1) / s;
  *splits = (n_pages + *pps - 1) / *pps;
}

size_t attn_rows_part_floats(int M, int Hq, int d, int max_pos, int window) {
  return (size_t)M * Hq * (d + 2);  // one split (minimum); more when the cap allows
}

hipError_t launch_attn_rows(const AttnArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  if (a.kv.act == ACT_BF16 && G == 4 && (a.d == 64 || a.d == 128 || a.d == 160)) {
    // MFMA decode kernel: ~4096 waves over (row, KV head, sub-split)
    const int n_pages = attn_pages_max(a.max_pos, a.window);
    int nsub = (4096 + a.M * a.Hkv - 1) / (a.M * a.Hkv);
    nsub = std::max(1, std::min(nsub, n_pages));
    while (nsub > 1 && (size_t)a.M * a.Hq * nsub * (a.d + 2) > (size_t)a.part_cap) nsub = (nsub + 1) / 2;
    const int pps = (n_pages + nsub - 1) / nsub;
    nsub = (n_pages + pps - 1) / pps;
    const int waves = a.M * a.Hkv * nsub;
    const dim3 grid((waves + 3) / 4);
    if (a.d == 64) hipLaunchKernelGGL(k_attn_decode<64>, grid, dim3(256), 0, st, a, nsub, pps);
    else if (a.d == 128) hipLaunchKernelGGL(k_attn_decode<128>, grid, dim3(256), 0, st, a, nsub, pps);
    else hipLaunchKernelGGL(k_attn_decode<160>, grid, dim3(256), 0, st, a, nsub, pps);
    hipLaunchKernelGGL(k_attn_combine<bf16_t>, dim3((a.M * a.Hq + 3) / 4), dim3(256), 0, st, a, nsub);
    return hipGetLastError();
  }
  if (G > ATT_MAXG || a.d > ATT_MAXD || a.d % 8 != 0) return hipErrorInvalidValue;
  const int n_pages = attn_pages_max(a.max_pos, a.window);
  int splits, pps;
  attn_pick_splits(a.M, a.Hkv, n_pages, (size_t)a.part_cap, a.Hq, a.d, &splits, &pps);
  const size_t esz = a.kv.act == ACT_F32 ? 4 : 2;
  const size_t shmem = 2 * PAGE * a.d * esz + (ATT_MAXG * a.d + 4 * ATT_MAXG * PAGE + ATT_MAXG * PAGE) * 4;
  dim3 grid(a.M, a.Hkv, splits);
  if (a.kv.act == ACT_F32) {
    hipLaunchKernelGGL(k_attn_rows<float>, grid, dim3(ATT_THREADS), shmem, st, a, splits, pps);
    hipLaunchKernelGGL(k_attn_combine<float>, dim3((a.M * a.Hq + 3) / 4), dim3(256), 0, st, a, splits);
  } else {
    hipLaunchKernelGGL(k_attn_rows<bf16_t>, grid, dim3(ATT_THREADS), shmem, st, a, splits, pps);
    hipLaunchKernelGGL(k_attn_combine<bf16_t>, dim3((a.M * a.Hq + 3) / 4), dim3(256), 0, st, a, splits);
  }
  return hipGetLastError();
}

}  // namespace dory
