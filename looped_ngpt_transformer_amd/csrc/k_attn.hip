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
// K and V, contiguous in the page) is staged in LDS with coalesced 16-byte loads.
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
  T* Vs = Ks + PAGE * d;                         // [64][d]
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
          if (i < d) o[c] += pj * ld<T>(Vs, (size_t)j * d + i);
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
template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int splits) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = a.d;
  for (int h = w; h < a.Hq; h += 4) {
    const float* src = a.part + ((size_t)m * a.Hq + h) * splits * (d + 2);
    float mx = -INFINITY;
    for (int s = 0; s < splits; ++s) mx = fmaxf(mx, src[s * (d + 2)]);
    float L = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float ms = src[s * (d + 2)];
      if (ms != -INFINITY) L += src[s * (d + 2) + 1] * __expf(ms - mx);
    }
    const float invL = 1.f / L;
    float sq = 0.f;
    for (int i = lane; i < d; i += 64) {
      float acc = 0.f;
      for (int s = 0; s < splits; ++s) {
        const float ms = src[s * (d + 2)];
        if (ms != -INFINITY) acc += src[s * (d + 2) + 2 + i] * __expf(ms - mx);
      }
      float ov = acc * invL;
      const size_t e = (size_t)m * a.Hq * d + (size_t)h * d + i;
      if (a.g) ov *= 1.f / (1.f + __expf(-ld<T>((const T*)a.g, e)));
      st<T>((T*)a.o, e, ov);
      sq += ov * ov;
    }
    sq = wave_sum(sq);
    if (lane == 0) a.ss[(size_t)m * a.Hq + h] = sq;
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
  if (G > ATT_MAXG || a.d > ATT_MAXD || a.d % 8 != 0) return hipErrorInvalidValue;
  const int n_pages = attn_pages_max(a.max_pos, a.window);
  int splits, pps;
  attn_pick_splits(a.M, a.Hkv, n_pages, (size_t)a.part_cap, a.Hq, a.d, &splits, &pps);
  const size_t esz = a.kv.act == ACT_F32 ? 4 : 2;
  const size_t shmem = 2 * PAGE * a.d * esz + (ATT_MAXG * a.d + 4 * ATT_MAXG * PAGE + ATT_MAXG * PAGE) * 4;
  dim3 grid(a.M, a.Hkv, splits);
  if (a.kv.act == ACT_F32) {
    hipLaunchKernelGGL(k_attn_rows<float>, grid, dim3(ATT_THREADS), shmem, st, a, splits, pps);
    hipLaunchKernelGGL(k_attn_combine<float>, dim3(a.M), dim3(256), 0, st, a, splits);
  } else {
    hipLaunchKernelGGL(k_attn_rows<bf16_t>, grid, dim3(ATT_THREADS), shmem, st, a, splits, pps);
    hipLaunchKernelGGL(k_attn_combine<bf16_t>, dim3(a.M), dim3(256), 0, st, a, splits);
  }
  return hipGetLastError();
}

}  // namespace dory
