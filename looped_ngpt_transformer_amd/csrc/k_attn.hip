// Paged GQA attention over the KV cache, split over keys, plus the combine step.
//
// For a query row at position p and query head h (KV head h / (Hq/Hkv)): the visible
// keys are the cached entries j <= p, and p - j < W on sliding-window layers; the
// output is softmax_j(scale * q.k_j) weighted sum of v_j ("Dory1.0-4B": GQA with 16
// query / 4 KV heads, 3:1 sliding (W = 1024) / full attention — paper summary
// "technical novelty", MXFP8 article "hybrid attention").
// The combine step merges the per-split softmax partials and applies the sigmoid
// output gate elementwise. (The L2 norm before the output projection, arXiv §2, only
// scales the row, which the nGPT update's N(.) removes.)
//
// Work-group = (row, KV head, split); its 4 waves are the group's query heads, so
// each K/V page is read once for all of them. A page's K and V blocks of one KV head
// (each contiguous in the page) are staged in LDS as a row-major K tile and a
// channel-major V tile.
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
  T* Vs = Ks + PAGE * d;                         // [d][64] (channel-major)
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
  const int chunks = PAGE * d / 8;    // 8-element chunks per K (or V) block
  const int32_t* trow = a.kv.table + ((size_t)seq * a.kv.n_streams + a.stream_idx) * a.kv.tab_len;

  for (int pg = pa; pg <= pb; ++pg) {
    const int32_t page = trow[pg % a.kv.ring];
    const T* kp = (const T*)a.kv.pool + (size_t)page * a.kv.page_elems + (size_t)hk * PAGE * d;
    const T* vp = kp + (size_t)a.Hkv * PAGE * d;
    __syncthreads();  // previous tile fully consumed
    for (int q8 = t; q8 < chunks; q8 += ATT_THREADS) {  // 8-element chunks, page order -> tiles
      int tok, ch;
      kv_k_chunk(q8, d, tok, ch);
#pragma unroll
      for (int e = 0; e < 8; ++e) Ks[tok * d + ch + e] = kp[q8 * 8 + e];
      kv_v_chunk(q8, d, ch, tok);
#pragma unroll
      for (int e = 0; e < 8; ++e) Vs[ch * PAGE + tok + e] = vp[q8 * 8 + e];
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

// Merge splits, apply the sigmoid gate, write o (act).
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
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = lane + 64 * c;
    if (i < d) {
      float ov = o[c] * invL;
      const size_t e = (size_t)m * a.Hq * d + (size_t)h * d + i;
      if (a.g) ov *= gate_at(a.g, a.g_f32, a.g_ld, a.g_splits, a.g_sstride, m, h * d + i);
      st<T>((T*)a.o, e, ov);
    }
  }
}

// ------------------------------------------------------------- decode attention, MFMA
// One wave per (row, KV head, sub-split of the row's pages); no LDS and no barriers.
// The wave streams its pages straight from HBM, 32 keys at a time with the next 32
// in flight. S^T = K Q^T puts the 4 grouped query heads in the B operand (columns
// 4..15 are zero) and O^T += V^T P^T takes P^T from the S^T accumulators. The page
// stores the rows of a 16-key K fragment in the order 8 (i / 4) + 4 kb + i % 4, so each
// lane's accumulators hold 8 consecutive keys, which is exactly the lane's part of the
// matching V^T fragment. Keys outside [lo, p] get -inf logits and, on partial pages,
// zeroed V entries.
//
// The split partials (max in log2 units, sum, unnormalised output per head) go to the
// workspace; k_decode_merge combines them.
constexpr int BUF_RSRC_WORD3 = 0x00020000;  // buffer resource flags: raw 32-bit dwords

// NBUF: register sets of K/V fragments per wave (2: the next half-page is in flight
// while the current one is computed); WPE: waves per SIMD the registers are cut for.
// QUAD: a wave takes up to four consecutive rows of one chunk (a quad of a prefill tile)
// as columns 4 r + g of the B operand, so a short chunk reads its keys once per quad
// instead of once per row; each column masks its own key range.
template <int D, int NBUF, int WPE, bool QUAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) void k_attn_decode(AttnArgs a, int nsub, int pps) {
  constexpr int G = 4, DC = D / 32, CB = D / 16;
  constexpr int PSTRIDE = 2 * G + G * D;  // floats per partial: m[G], l[G], o[G][D]
  const int lane = threadIdx.x & 63;
  // wave-uniform indices in scalar registers: page addresses become scalar bases
  const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (wid >= (QUAD ? a.n_quads : a.M) * a.Hkv * nsub) return;
  const int sub = wid % nsub, grp = wid / nsub;
  const int hk = grp % a.Hkv;
  int m = grp / a.Hkv, R = 1;  // first row, rows taken
  if constexpr (QUAD) {
    // quad index -> (tile, quad of the tile): tiles hold <= 64 rows, ceil(rows / 4) quads
    const int quad = m;
    int t = 0, q0 = 0, nr = 0;
    for (; t < a.n_tiles; ++t) {
      nr = a.tiles[4 * t + 1];
      const int nq = (nr + 3) >> 2;
      if (quad < q0 + nq) break;
      q0 += nq;
    }
    m = a.tiles[4 * t] + 4 * (quad - q0);
    R = min(4, nr - 4 * (quad - q0));
  }
  const int lq = lane & 15, lk = lane >> 4;
  const int rq = min(lq >> 2, R - 1);  // this column's row (columns 4R.. repeat the last)
  const int p_col = a.pos[m + rq];
  const int lo_col = a.window > 0 ? max(0, p_col - a.window + 1) : 0;
  // the rows' positions are consecutive: the key range of the quad and the part every
  // column sees
  const int p = a.pos[m + R - 1], p_min = a.pos[m];
  const int seq = a.row_seq[m];
  const int lo = a.window > 0 ? max(0, p_min - a.window + 1) : 0;
  const int lo_max = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int pg_lo = lo / PAGE, pg_hi = p / PAGE;
  const int pa = pg_lo + sub * pps;
  const int pb = min(pg_hi, pa + pps - 1);
  const int32_t* trow = a.kv.table + ((size_t)seq * a.kv.n_streams + a.stream_idx) * a.kv.tab_len;
  const bf16_t* pool = (const bf16_t*)a.kv.pool;

  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (lq < G * R)
      v = *(const uint4*)((const bf16_t*)a.q + (size_t)(m + (lq >> 2)) * a.Hq * D + (size_t)(hk * G + (lq & 3)) * D +
                          32 * c + 8 * lk);
    qf[c] = __builtin_bit_cast(bf16x8, v);
  }
  const float sl2 = a.scale * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Half-pages (32 keys) hp = 2 * page + hf; lane (lq, lk) owns keys 32 hf + 8 lk .. + 7.
  // Every fragment is 1 KiB contiguous in the page (fragment-order layout), read with
  // one 16-byte load per lane through a buffer resource on the page (scalar base,
  // bounds = the page): the per-lane offset is 16 * lane, the rest scalar.
  struct Half {
    uint4 k[2][DC];  // K fragment (kb, c): tokens 8 (lq / 4) + 4 kb + lq % 4, channels 32 c + 8 lk ..
    uint4 v[CB];     // V^T fragment cb: channel 16 cb + lq, tokens 8 lk .. + 7 of the half
  };
  const int voff = 16 * lane;
  const int kofs = hk * PAGE * D * 2;
  const int vofs = (a.Hkv + hk) * PAGE * D * 2;
  const int page_bytes = (int)(a.kv.page_elems * 2);
  auto load = [&](int hp, Half& H) {
    const int pg = hp >> 1, hf = hp & 1;
    const int32_t page = trow[pg % a.kv.ring];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(pool + (size_t)page * a.kv.page_elems), 0, page_bytes, BUF_RSRC_WORD3);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < DC; ++c)
        H.k[kb][c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, voff, kofs + ((hf * 2 + kb) * DC + c) * 1024, 0));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      H.v[cb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rs, voff, vofs + (hf * CB + cb) * 1024, 0));
  };
  auto compute = [&](int hp, const Half& H) {
    const int pg = hp >> 1, hf = hp & 1;
    const int kbase = pg * PAGE + 32 * hf + 8 * lk;  // this lane's first key
    const bool whole = pg * PAGE + 32 * hf >= lo_max && pg * PAGE + 32 * hf + 31 <= p_min;
    f32x4 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c)
        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, H.k[kb][c]), qf[c], st[kb], 0, 0, 0);
    }
    // st[kb][r] = S^T[key kbase + 4 kb + r][head lq]: online softmax for head lq
    float sv[8];
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kbase + e;
      const bool vis = key >= lo_col && key <= p_col;
      sv[e] = vis ? st[e >> 2][e & 3] * sl2 : -INFINITY;
      mt = fmaxf(mt, sv[e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float corr = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;  // no key seen yet: p = exp2(-inf) = 0
    float pe[8];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(sv[e] - m_ref);
      ps += pe[e];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    m_run = m_new;
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = (uint32_t)f2bf(pe[2 * i]) | ((uint32_t)f2bf(pe[2 * i + 1]) << 16);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(u[0], u[1], u[2], u[3]));
    if (whole) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        o[cb] *= corr;
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, H.v[cb]), pf, o[cb], 0, 0, 0);
      }
    } else {  // zero V entries of keys outside [lo, p] (may be unwritten)
      uint32_t vmask[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kbase + e;
        if (key < lo || key > p) vmask[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint4 v = H.v[cb];
        const uint4 vm = make_uint4(v.x & vmask[0], v.y & vmask[1], v.z & vmask[2], v.w & vmask[3]);
        o[cb] *= corr;
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vm), pf, o[cb], 0, 0, 0);
      }
    }
  };

  const int h0 = 2 * pa, h1 = 2 * pb + 1;  // empty when pa > pb
  if constexpr (NBUF == 2) {  // next half-page in flight while this one is computed
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
  } else {  // one half-page per wave in flight; latency hidden by resident waves
    for (int hp = h0; hp <= h1; ++hp) {
      Half A;
      load(hp, A);
      compute(hp, A);
    }
  }

  // ---- publish this split's partial: O^T[channel 16 cb + 4 lk + r][column lq], column
  // 4 r + g being head g of row m + r
  if (lq < G * R) {
    const int g = lq & 3;
    float* mine = a.part + ((size_t)((m + (lq >> 2)) * a.Hkv + hk) * nsub + sub) * PSTRIDE;
    if (lk == 0) {
      mine[g] = m_run;
      mine[G + g] = l_run;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) *(f32x4*)(mine + 2 * G + g * D + 16 * cb + 4 * lk) = o[cb];
  }
}

// Merge of the decode splits, sigmoid gate and output. One
// wave per (row, query head): lane s < nsub weighs split s, then the lanes take channel
// pairs and accumulate the splits 8 at a time (their loads in flight together; empty
// splits hold zeros and weigh 0).
template <int D>
__global__ __launch_bounds__(64) void k_decode_merge(AttnArgs a, int nsub) {
  constexpr int G = 4;
  constexpr int PSTRIDE = 2 * G + G * D;
  constexpr int NP = D / 2;                 // channel pairs
  constexpr int PPL = (NP + 63) / 64;       // pairs per lane
  const int lane = threadIdx.x;
  const int m = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int hk = h / G, g = h % G;
  const float* gbase = a.part + (size_t)(m * a.Hkv + hk) * nsub * PSTRIDE;
  const float ms = lane < nsub ? gbase[(size_t)lane * PSTRIDE + g] : -INFINITY;
  const float ls = lane < nsub ? gbase[(size_t)lane * PSTRIDE + G + g] : 0.f;
  const float mx = wave_max(ms);
  const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - mx);
  const float L = wave_sum(wgt * ls);
  const float* ob = gbase + 2 * G + g * D;
  f32x2 acc[PPL];
#pragma unroll
  for (int i = 0; i < PPL; ++i) acc[i] = f32x2{0.f, 0.f};
  for (int s0 = 0; s0 < nsub; s0 += 8) {
    f32x2 v[8][PPL];
    float w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, nsub - 1);
      w[u] = s0 + u < nsub ? __shfl(wgt, s, 64) : 0.f;
#pragma unroll
      for (int i = 0; i < PPL; ++i) {
        const int pr = lane + 64 * i;
        v[u][i] = pr < NP ? *(const f32x2*)(ob + (size_t)s * PSTRIDE + 2 * pr) : f32x2{0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < PPL; ++i) acc[i] += w[u] * v[u][i];
  }
  const float invL = 1.f / L;
  bf16_t* out = (bf16_t*)a.o + (size_t)m * a.Hq * D + (size_t)h * D;
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    const int pr = lane + 64 * i;
    if (pr >= NP) continue;
    const int c = 2 * pr;
    float v0 = acc[i][0] * invL, v1 = acc[i][1] * invL;
    if (a.g) {
      v0 *= gate_at(a.g, a.g_f32, a.g_ld, a.g_splits, a.g_sstride, m, h * D + c);
      v1 *= gate_at(a.g, a.g_f32, a.g_ld, a.g_splits, a.g_sstride, m, h * D + c + 1);
    }
    *(uint32_t*)(out + c) = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
  }
}

// One launch of the decode kernel: (row, KV head) groups split over keys so that the
// waves fill the device once (the resident count comes from the occupancy query); at
// most max_sub splits per group (the merge weighs one split per lane: <= 64).
template <int D, int NBUF, int WPE, bool QUAD>
static hipError_t launch_decode(const AttnArgs& a, int n_pages, int max_sub, int phase, int* splits_out,
                                hipStream_t st) {
  static int slots = 0;
  if (!slots) {
    int dev = 0, cus = 0, blocks = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_attn_decode<D, NBUF, WPE, QUAD>, 256, 0) !=
            hipSuccess ||
        cus <= 0 || blocks <= 0)
      return hipErrorInvalidValue;
    slots = cus * blocks * 4;
  }
  const int groups = (QUAD ? a.n_quads : a.M) * a.Hkv;
  int nsub = std::max(1, slots / groups);
  nsub = std::min({nsub, n_pages, max_sub, 64});
  while (nsub > 1 && (size_t)a.M * a.Hq * nsub * (a.d + 2) > (size_t)a.part_cap) nsub = (nsub + 1) / 2;
  const int pps = (n_pages + nsub - 1) / nsub;
  nsub = (n_pages + pps - 1) / pps;
  const int waves = groups * nsub;
  if (splits_out) *splits_out = nsub;
  if (phase == ATTN_SPLITS)
    hipLaunchKernelGGL((k_attn_decode<D, NBUF, WPE, QUAD>), dim3((waves + 3) / 4), dim3(256), 0, st, a, nsub, pps);
  else if (phase == ATTN_MERGE)
    hipLaunchKernelGGL(k_decode_merge<D>, dim3(a.M * a.Hq), dim3(64), 0, st, a, nsub);
  return hipGetLastError();
}

// Single rows: two register sets per wave (the next half-page in flight), one wave per
// SIMD; up to 16 splits over long key ranges, up to 64 over short ones (sliding windows,
// short contexts). On a sliding layer of the 72-layer shape this takes 17 us at batch 32
// and 64 us at batch 128, against 22 / 69 us with one register set, three waves per SIMD
// and a page per split. Quads of rows: one register set, three waves per SIMD over short
// ranges.
constexpr int DECODE_SHORT_PAGES = 32;
// Chunks of several rows (max_tile_rows > 1) go by quads of rows, whose key range is up
// to three positions longer than a row's (one more page at most).
template <int D>
static hipError_t launch_decode_d(const AttnArgs& a, int n_pages, int phase, int* splits, hipStream_t st) {
  if (a.max_tile_rows > 1 && a.n_quads > 0 && a.tiles) {
    if (a.window > 0) ++n_pages;
    if (n_pages > DECODE_SHORT_PAGES) return launch_decode<D, 2, 1, true>(a, n_pages, 16, phase, splits, st);
    return launch_decode<D, 1, 3, true>(a, n_pages, 64, phase, splits, st);
  }
  return launch_decode<D, 2, 1, false>(a, n_pages, n_pages > DECODE_SHORT_PAGES ? 16 : 64, phase, splits, st);
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

hipError_t launch_attn_rows(const AttnArgs& a, int phase, int* splits_out, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  if (a.kv.act == ACT_BF16 && G == 4 && (a.d == 64 || a.d == 128 || a.d == 160)) {
    // MFMA decode kernel + split merge
    const int n_pages = attn_pages_max(a.max_pos, a.window);
    if (a.d == 64) return launch_decode_d<64>(a, n_pages, phase, splits_out, st);
    if (a.d == 128) return launch_decode_d<128>(a, n_pages, phase, splits_out, st);
    return launch_decode_d<160>(a, n_pages, phase, splits_out, st);
  }
  if (G > ATT_MAXG || a.d > ATT_MAXD || a.d % 8 != 0) return hipErrorInvalidValue;
  const int n_pages = attn_pages_max(a.max_pos, a.window);
  int splits, pps;
  attn_pick_splits(a.M, a.Hkv, n_pages, (size_t)a.part_cap, a.Hq, a.d, &splits, &pps);
  const size_t esz = a.kv.act == ACT_F32 ? 4 : 2;
  const size_t shmem = 2 * PAGE * a.d * esz + (ATT_MAXG * a.d + 4 * ATT_MAXG * PAGE + ATT_MAXG * PAGE) * 4;
  if (splits_out) *splits_out = splits;
  dim3 grid(a.M, a.Hkv, splits);
  const dim3 cgrid((a.M * a.Hq + 3) / 4);
  if (a.kv.act == ACT_F32) {
    if (phase == ATTN_SPLITS) hipLaunchKernelGGL(k_attn_rows<float>, grid, dim3(ATT_THREADS), shmem, st, a, splits, pps);
    if (phase == ATTN_MERGE) hipLaunchKernelGGL(k_attn_combine<float>, cgrid, dim3(256), 0, st, a, splits);
  } else {
    if (phase == ATTN_SPLITS) hipLaunchKernelGGL(k_attn_rows<bf16_t>, grid, dim3(ATT_THREADS), shmem, st, a, splits, pps);
    if (phase == ATTN_MERGE) hipLaunchKernelGGL(k_attn_combine<bf16_t>, cgrid, dim3(256), 0, st, a, splits);
  }
  return hipGetLastError();
}

}  // namespace dory
