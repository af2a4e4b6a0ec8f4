// The steps on either side of the looped stack: token embedding, the LM head's logit
// scale, and top-p sampling ("Dory1.0-4B" pages: nGPT keeps embeddings on the unit
// sphere — paper summary, "prerequisites: nGPT"; logit-scale parameters — arXiv summary
// §2; generation settings temperature 1.0, top_p 0.95 — MXFP8 article, deployment section).
// The LM-head product itself is a projection GEMM (k_gemm.hip).
#include <climits>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dory {

// x[i] = N(E[ids[i]]) as float rows; an id outside [0, V) gives a zero row (the table
// is never read out of range). One block per row.
template <typename T>
__global__ __launch_bounds__(256) void k_embed(const T* E, int64_t V, int H, const int32_t* ids, float* x) {
  __shared__ float red[4];
  const int i = blockIdx.x;
  const int id = ids[i];
  const bool ok = id >= 0 && id < V;  // uniform over the block
  const T* row = E + (ok ? (size_t)id * H : 0);
  float ss = 0.f;
  if (ok)
    for (int c = threadIdx.x; c < H; c += 256) {
      const float v = ld(row, c);
      ss += v * v;
    }
  const float inv = inv_norm(block_sum<4>(ss, red));
  for (int c = threadIdx.x; c < H; c += 256) x[(size_t)i * H + c] = ok ? ld(row, c) * inv : 0.f;
}

// logits[i][v] = s_z[v] * sum_s part[s][i][v]: the per-token logit scale on the LM-head
// product (split-K partials when the GEMM split K; part == logits for one split).
__global__ __launch_bounds__(256) void k_logit_scale(const float* part, int splits, size_t sstride, float* logits,
                                                     int64_t ld, int64_t V, const float* sz) {
  const int i = blockIdx.y;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  const size_t o = (size_t)i * ld + v;
  logits[o] = sz[v] * sum_splits(part + o, sstride, splits);
}

// ------------------------------------------------------------------ top-p sampling
// One block of ST threads per row; thread t owns ids t, t + ST, t + 2 ST, ... (each load
// instruction of a wave reads consecutive ids). Weights e_v = 2^((l_v - max) / T * log2 e)
// are recomputed identically in every pass; their float bit patterns order the tokens
// like their probabilities. The sorted order is e descending, equal e by lower id. Each
// selection finds the first token of that order whose running mass meets a target:
// eight passes over 4-bit digits of the bit pattern, high to low, narrow the key down
// (per-thread digit masses in LDS, summed in a fixed order); the tokens with exactly that
// key all weigh the same e*, so the j-th of them in id order has running mass
// above + (j + 1) e*, which fixes j, and the token is the (j + 1)-th smallest id among
// them. Every sum has a fixed order, so the result is a deterministic function of the
// logits and u.
constexpr int ST = 1024;

struct SampleLds {
  float bins[16][ST];  // per-thread mass of each digit
  int cnt[16][ST];     // per-thread count of each digit
  float binsum[16];
  int bincnt[16];
  float red[16];
  int ired[16];
  uint32_t prefix;
  float above;
  int jsel;
  float tgt, cumsel;   // the selection's target; the chosen token's running mass
  int selcnt, ncand;   // tokens under the chosen digits; candidates collected
  float b0sum[16];     // the first pass's digit masses and counts, kept for the next
  int b0cnt[16];       // selection over the same row
};
// At most this many tokens left under the chosen digits: collect them, sort them in LDS
// (e descending, id ascending) and finish with one fixed-order scan.
constexpr int CAND = 2 * ST;

__device__ __forceinline__ float block_max16(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < ST / WAVE; ++i) t = fmaxf(t, red[i]);
  return t;
}

__device__ __forceinline__ int block_min_int(int v, int* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, WAVE));
  const int w = threadIdx.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  int t = red[0];
#pragma unroll
  for (int i = 1; i < ST / WAVE; ++i) t = min(t, red[i]);
  return t;
}

__device__ __forceinline__ int block_sum_int(int v, int* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  const int w = threadIdx.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < ST / WAVE; ++i) t += red[i];
  return t;
}

struct RowView {
  const float* L;
  int V;
  float c, mz;  // e = 2^(l c - mz)
  __device__ __forceinline__ float ew(float l) const { return exp2f(l * c - mz); }
  __device__ __forceinline__ float e(int i) const { return ew(L[i]); }
};

// f(i, L[i]) for the ids i < n a thread owns, in increasing order (t, t + ST, ...), with
// SU loads in flight per thread: a pass over the row is bound by how many L2 requests
// are outstanding, not by the arithmetic.
constexpr int SU = 16;
template <int U = SU, typename F>
__device__ __forceinline__ void row_for(const float* L, int n, F&& f) {
  for (int i0 = threadIdx.x; i0 < n; i0 += ST * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * ST;
      v[u] = i < n ? L[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u * ST < n) f(i0 + u * ST, v[u]);
  }
}

// Prefix sums of one float per thread in thread order (fixed order): returns the inclusive
// sum, *excl the exclusive one (the same additions minus this thread's).
__device__ __forceinline__ float block_scan_f(float v, float* red, float* excl) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  float x = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const float y = __shfl_up(x, d, WAVE);
    if (lane >= d) x += y;
  }
  const float xe = __shfl_up(x, 1, WAVE);
  __syncthreads();
  if (lane == WAVE - 1) red[w] = x;
  __syncthreads();
  float off = 0.f;
  for (int i = 0; i < w; ++i) off += red[i];
  *excl = lane ? off + xe : off;
  return off + x;
}

// First token of the sorted order whose inclusive running mass reaches (incl) or
// exceeds (!incl) target; if rounding leaves the target beyond the mass, the last token
// of the order. Returns the token and sets cum to its inclusive running mass.
// frac >= 0: the target is frac times the row's total mass (taken from the first pass's
// digit masses, summed high digit first). reuse0: the previous selection ran over the
// same row; its first pass is taken from LDS instead of being recomputed.
// U: loads in flight per thread in each pass.
template <int U = SU>
__device__ int select_token(SampleLds& S, const RowView& R, float target, bool incl, float* cum,
                            float frac = -1.f, bool reuse0 = false) {
  const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
  uint32_t prefix = 0;
  float above = 0.f;  // mass of the tokens whose key lies above the digits chosen so far
  for (int pass = 0; pass < 8; ++pass) {
    const int sh = 28 - 4 * pass;
    if (!(pass == 0 && reuse0)) {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        S.bins[d][t] = 0.f;
        S.cnt[d][t] = 0;
      }
      row_for<U>(R.L, R.V, [&](int, float l) {
        const float e = R.ew(l);
        const uint32_t key = __float_as_uint(e);
        if (pass == 0 || (key >> (sh + 4)) == prefix) {
          const int d = (key >> sh) & 15;
          S.bins[d][t] += e;
          S.cnt[d][t] += 1;
        }
      });
      __syncthreads();
      {  // wave w sums digit w over the threads, lane j taking threads j, j + 64, ...
        float v = 0.f;
        int c = 0;
#pragma unroll
        for (int j = 0; j < ST / WAVE; ++j) {
          v += S.bins[w][j * WAVE + lane];
          c += S.cnt[w][j * WAVE + lane];
        }
        v = wave_sum(v);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, WAVE);
        if (lane == 0) {
          S.binsum[w] = v;
          S.bincnt[w] = c;
          if (pass == 0) {
            S.b0sum[w] = v;
            S.b0cnt[w] = c;
          }
        }
      }
    } else if (t < 16) {
      S.binsum[t] = S.b0sum[t];
      S.bincnt[t] = S.b0cnt[t];
    }
    __syncthreads();
    if (t == 0) {
      if (pass == 0) {
        if (frac >= 0.f) {
          float total = 0.f;
          for (int d = 15; d >= 0; --d) total += S.binsum[d];
          target = frac * total;
        }
        S.tgt = target;
      }
      float acc = above, acc_last = above;
      int sel = -1, last = -1;
      for (int d = 15; d >= 0; --d) {
        if (S.bincnt[d] == 0) continue;
        last = d;
        acc_last = acc;
        const float nxt = acc + S.binsum[d];
        if (incl ? nxt >= target : nxt > target) {
          sel = d;
          break;
        }
        acc = nxt;
      }
      if (sel < 0) {
        sel = last;
        acc = acc_last;
      }
      S.prefix = (prefix << 4) | (uint32_t)sel;
      S.above = acc;
      S.selcnt = S.bincnt[sel];
    }
    __syncthreads();
    prefix = S.prefix;
    above = S.above;
    target = S.tgt;
    const int n = S.selcnt;
    __syncthreads();
    if (pass < 7 && n <= CAND) {
      // few tokens left under these digits: collect (e, id), sort, scan
      float* ce = &S.bins[0][0];        // CAND floats (bins[0], bins[1])
      int* cid = (int*)&S.bins[2][0];   // CAND ints (bins[2], bins[3])
      if (t == 0) S.ncand = 0;
      __syncthreads();
      row_for<U>(R.L, R.V, [&](int i, float l) {
        const float e = R.ew(l);
        if ((__float_as_uint(e) >> sh) == prefix) {
          const int k = atomicAdd(&S.ncand, 1);
          if (k < CAND) {
            ce[k] = e;
            cid[k] = i;
          }
        }
      });
      __syncthreads();
      int np2 = 1;
      while (np2 < n) np2 <<= 1;
      for (int k = n + t; k < np2; k += ST) {
        ce[k] = -1.f;
        cid[k] = INT_MAX;
      }
      __syncthreads();
      // bitonic sort into the sorted order: e descending, equal e by lower id
      for (int size = 2; size <= np2; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int k = t; k < np2 / 2; k += ST) {
            const int i = 2 * stride * (k / stride) + k % stride, j = i + stride;
            const float ea = ce[i], eb = ce[j];
            const int ia = cid[i], ib = cid[j];
            const bool a_first = ea > eb || (ea == eb && ia < ib);
            if (a_first != ((i & size) == 0)) {
              ce[i] = eb;
              ce[j] = ea;
              cid[i] = ib;
              cid[j] = ia;
            }
          }
          __syncthreads();
        }
      // running mass in that order, two candidates per thread
      const int i0 = 2 * t, i1 = 2 * t + 1;
      const float e0 = i0 < n ? ce[i0] : 0.f, e1 = i1 < n ? ce[i1] : 0.f;
      float excl;
      block_scan_f(e0 + e1, S.red, &excl);
      const float c0 = above + (excl + e0), c1 = above + ((excl + e0) + e1);
      int hit = INT_MAX;
      if (i0 < n && (incl ? c0 >= target : c0 > target)) hit = i0;
      else if (i1 < n && (incl ? c1 >= target : c1 > target)) hit = i1;
      int first = block_min_int(hit, S.ired);
      if (first == INT_MAX) first = n - 1;
      if (t == first / 2) {
        S.jsel = cid[first];
        S.cumsel = (first & 1) ? c1 : c0;
      }
      __syncthreads();
      const int tok = S.jsel;
      *cum = S.cumsel;
      __syncthreads();
      return tok;
    }
  }
  // the tokens whose key is exactly `prefix`: their count (the last digit's count), the
  // first j whose running mass above + (j + 1) e* meets the target (else the last one)
  const float es = __uint_as_float(prefix);
  const int n_tied = S.bincnt[prefix & 15];
  if (t == 0) {
    int j = n_tied - 1;
    for (int q = 0; q < n_tied; ++q) {
      const float c = above + (float)(q + 1) * es;
      if (incl ? c >= target : c > target) {
        j = q;
        break;
      }
    }
    S.jsel = j;
  }
  __syncthreads();
  const int jsel = S.jsel;
  *cum = above + (float)(jsel + 1) * es;
  int tok;
  if (n_tied == 1) {
    int mine = INT_MAX;
    row_for<U>(R.L, R.V, [&](int i, float l) {
      if (__float_as_uint(R.ew(l)) == prefix) mine = i;
    });
    tok = block_min_int(mine, S.ired);
  } else {
    // the (jsel + 1)-th smallest id among them: the largest x with fewer than jsel + 1
    // of them below x, by bisection on x
    int lo = 0, hi = R.V;  // count(lo) <= jsel < count(hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      int n = 0;
      row_for<U>(R.L, mid, [&](int, float l) { n += __float_as_uint(R.ew(l)) == prefix; });
      if (block_sum_int(n, S.ired) <= jsel) lo = mid;
      else hi = mid;
    }
    tok = lo;
  }
  __syncthreads();
  return tok;
}

__global__ __launch_bounds__(ST) void k_sample_top_p(const float* logits, int64_t ld, int V, float inv_t,
                                                     float top_p, const float* u, int32_t* out, int out_stride) {
  __shared__ SampleLds S;
  const int t = threadIdx.x;
  RowView R;
  R.L = logits + (size_t)blockIdx.x * ld;
  R.V = V;
  R.c = inv_t * 1.4426950408889634f;
  float m = -INFINITY;
  row_for(R.L, V, [&](int, float l) { m = fmaxf(m, l); });
  R.mz = block_max16(m, S.red) * R.c;
  // nucleus: the first token whose running mass reaches top_p of the total
  float mass;
  const int cut = select_token(S, R, 0.f, true, &mass, top_p);
  // the draw: the first token whose running mass exceeds u times the nucleus mass
  float cum;
  int tok = select_token(S, R, u[blockIdx.x] * mass, false, &cum, -1.f, true);
  // rounding may not place the draw after the cut: order (e descending, id ascending)
  if (t == 0) {
    const float ec = R.e(cut), et = R.e(tok);
    if (et < ec || (et == ec && tok > cut)) tok = cut;
    out[(size_t)blockIdx.x * out_stride] = tok;
  }
}

// ------------------------------------------------------ speculative acceptance
// A processed row: temperature, then the top-p nucleus renormalised. `init` finds the max,
// the total weight, the nucleus cut (the sampler's first selection) and the nucleus mass;
// prob(v) is the renormalised probability of token v (0 outside the nucleus).
struct Processed {
  RowView R;
  int cut;
  float ecut, mass;
  template <int U = SU>
  __device__ void init(SampleLds& S, const float* L, int V, float inv_t, float top_p) {
    const int t = threadIdx.x;
    R.L = L;
    R.V = V;
    R.c = inv_t * 1.4426950408889634f;
    float m = -INFINITY;
    row_for<U>(L, V, [&](int, float l) { m = fmaxf(m, l); });
    R.mz = block_max16(m, S.red) * R.c;
    cut = select_token<U>(S, R, 0.f, true, &mass, top_p);
    ecut = R.e(cut);
  }
  __device__ float prob_l(int v, float l) const {  // l = the row's logit of token v
    const float e = R.ew(l);
    const bool in = e > ecut || (e == ecut && v <= cut);
    return in ? e / mass : 0.f;
  }
  __device__ float prob(int v) const { return prob_l(v, R.L[v]); }
};

// The token u draws from max(0, p - q) renormalised, by inverse CDF over increasing ids
// (from p itself if the residual is empty). Thread t owns the ids [t C, t C + C).
__device__ int residual_draw(SampleLds& S, const Processed& P, const Processed& Q, int V, float u) {
  const int t = threadIdx.x, C = (V + ST - 1) / ST, beg = min(t * C, V), end = min(beg + C, V);
  // f(v, residual weight, p weight) over the thread's ids in increasing order, 8 loads
  // of each row in flight
  auto chunk = [&](auto&& f) {
    for (int v0 = beg; v0 < end; v0 += 8) {
      float lp[8], lq[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        lp[u] = v0 + u < end ? P.R.L[v0 + u] : 0.f;
        lq[u] = v0 + u < end ? Q.R.L[v0 + u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (v0 + u < end) {
          const float pv = P.prob_l(v0 + u, lp[u]);
          f(v0 + u, fmaxf(pv - Q.prob_l(v0 + u, lq[u]), 0.f), pv);
        }
    }
  };
  float mine = 0.f, acc;
  chunk([&](int, float r, float) { mine += r; });
  float incl = block_scan_f(mine, S.red, &acc);
  __syncthreads();
  if (t == ST - 1) S.above = incl;
  __syncthreads();
  const bool from_p = !(S.above > 0.f);
  __syncthreads();
  if (from_p) {  // empty residual
    mine = 0.f;
    chunk([&](int, float, float pv) { mine += pv; });
    incl = block_scan_f(mine, S.red, &acc);
    __syncthreads();
    if (t == ST - 1) S.above = incl;
    __syncthreads();
  }
  const float target = u * S.above;
  int cand = INT_MAX, last = -1;
  chunk([&](int v, float r, float pv) {
    const float w = from_p ? pv : r;
    if (w > 0.f) last = v;
    acc += w;
    if (cand == INT_MAX && acc > target && w > 0.f) cand = v;
  });
  int tok = block_min_int(cand, S.ired);
  if (tok == INT_MAX) tok = -block_min_int(-last, S.ired);
  return tok;
}

// One work-group per (sequence b, position j < gamma); draft rows, tokens and acceptance
// draws are position-major ([gamma, n]), the verifying rows sequence-major
// ([n, gamma + 1]). The draft token x_j is accepted when u_accept < p_j(x_j) / q_j(x_j),
// else the group draws the residual token with u_sample and lowers n_out[b] to j + 1 (an
// atomic minimum: the first rejection wins). Every group writes out[b, j]; n_out[b]
// starts at gamma + 1 (k_fill_n), and the token that follows a fully accepted block is
// the top-p sampler's on the verifier's last row (k_sample_top_p, launched beside). The
// groups of later positions do their work whether or not an earlier one rejects.
__global__ void k_fill_n(int32_t* n_out, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) n_out[i] = v;
}

__global__ __launch_bounds__(ST) void k_spec_accept(int gamma, int V, const float* draft, int64_t ld_d,
                                                    const float* target, int64_t ld_t, const int32_t* dtok,
                                                    float inv_t, float top_p, const float* u_acc,
                                                    const float* u_smp, int32_t* out, int32_t* n_out) {
  __shared__ SampleLds S;
  const int b = blockIdx.x, j = blockIdx.y, t = threadIdx.x;
  const size_t dj = (size_t)j * gridDim.x + b;  // draft side: position-major
  // the verifier's row, then the draft's, through one copy of the code (registers)
  Processed P, Q;
#pragma nounroll
  for (int which = 0; which < 2; ++which) {
    Processed X;
    X.init<8>(S, which ? draft + dj * ld_d : target + ((size_t)b * (gamma + 1) + j) * ld_t, V, inv_t, top_p);
    if (which) Q = X;
    else P = X;
  }
  int32_t* o = out + (size_t)b * (gamma + 1) + j;
  const int x = dtok[dj];
  const bool valid = x >= 0 && x < V;
  const float q = valid ? Q.prob(x) : 0.f;
  const float ratio = q > 0.f ? P.prob(x) / q : 0.f;
  if (u_acc[dj] < ratio) {
    if (t == 0) *o = x;
    return;
  }
  const int r = residual_draw(S, P, Q, V, u_smp[b]);
  if (t == 0) {
    *o = r;
    atomicMin(n_out + b, j + 1);
  }
}

hipError_t launch_spec_accept(int n, int gamma, int64_t V, const float* draft, int64_t ld_d, const float* target,
                              int64_t ld_t, const int32_t* dtok, float temperature, float top_p, const float* u_acc,
                              const float* u_smp, int32_t* out, int32_t* n_out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_n, dim3((n + 255) / 256), dim3(256), 0, st, n_out, n, gamma + 1);
  hipLaunchKernelGGL(k_spec_accept, dim3(n, gamma), dim3(ST), 0, st, gamma, (int)V, draft, ld_d, target, ld_t,
                     dtok, 1.0f / temperature, top_p, u_acc, u_smp, out, n_out);
  // the token after a fully accepted block: row gamma of each sequence's verifying rows
  hipLaunchKernelGGL(k_sample_top_p, dim3(n), dim3(ST), 0, st, target + (size_t)gamma * ld_t, ld_t * (gamma + 1),
                     (int)V, 1.0f / temperature, top_p, u_smp, out + gamma, gamma + 1);
  return hipGetLastError();
}

hipError_t launch_embed(const void* E, int e_bf16, int64_t V, int H, const int32_t* ids, int n, float* x,
                        hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (e_bf16)
    hipLaunchKernelGGL(k_embed<bf16_t>, dim3(n), dim3(256), 0, st, (const bf16_t*)E, V, H, ids, x);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(n), dim3(256), 0, st, (const float*)E, V, H, ids, x);
  return hipGetLastError();
}

hipError_t launch_logit_scale(const float* part, int splits, size_t sstride, float* logits, int64_t ld, int n,
                              int64_t V, const float* sz, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((V + 255) / 256), n);
  hipLaunchKernelGGL(k_logit_scale, grid, dim3(256), 0, st, part, splits, sstride, logits, ld, V, sz);
  return hipGetLastError();
}

hipError_t launch_sample_top_p(const float* logits, int64_t ld, int n, int64_t V, float temperature, float top_p,
                               const float* u, int32_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sample_top_p, dim3(n), dim3(ST), 0, st, logits, ld, (int)V, 1.0f / temperature, top_p,
                     u, out, 1);
  return hipGetLastError();
}

// Device scratch of the LM-head entry point that allocates nothing (dory_logits_noalloc):
// the staged states and split-K partials live here instead of in a bound workspace.
// Each GPU the library runs on holds its own copy for the life of the process, and
// every call on that GPU shares it.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

// The device address of this GPU's scratch (the current device). The array's name is a
// host-side stand-in, so its address is looked up once per device with the device
// current and kept; kernels get the looked-up pointer.
hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace dory
