// Prefill attention on bf16 with MFMA (flash-style online softmax over KV pages).
//
// Same maths as the row kernel: GQA (4 query heads per KV head), causal, sliding
// window W on sliding layers, softmax(scale * q.k) v, then the sigmoid output gate
// ("Dory1.0-4B": paper summary "technical novelty"; arXiv §2; MXFP8 article "hybrid
// attention").
//
// Work-group = (tile of <= 64 consecutive query rows of one sequence, KV head): 16
// waves, wave = (query head g of the group, 16-row quarter of the tile). Per KV page:
//   S^T = K Q^T   with v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q in registers),
//   online softmax per query in registers (lane's query is lane % 16),
//   O^T += V^T P^T (A = V^T from LDS, B = P straight from the S^T accumulators: the lane
//   already holds 2x4 keys of its query, which is a valid k-ordering of the MFMA when
//   V^T is read with the same key permutation).
// The page's K and V blocks (8-element chunks in MFMA fragment order) are staged as a
// row-major K tile and a V^T tile in padded LDS rows; the next page is prefetched into
// registers while the current one is consumed. Entries of the last page beyond the chunk's last position are zeroed, so
// unwritten cache memory can never reach the sums.
#include "common.h"
#include "kernels.h"

namespace dory {

constexpr int PF_THREADS = 1024;
constexpr int PF_MAX_PAGES = 4096;  // positions up to 262144

template <int D>
__global__ __launch_bounds__(PF_THREADS) void k_attn_prefill(AttnArgs a) {
  constexpr int G = 4;
  constexpr int DC = D / 32;       // 32-wide chunks of the head dim (QK contraction)
  constexpr int CB = D / 16;       // 16-channel blocks of the output
  constexpr int KCH = D / 8 + 1;   // 16-byte chunks per padded K row
  // bf16 per padded V^T row: a 136-byte stride puts the 16 rows of an 8-byte fragment
  // read in distinct banks (row r at 8r mod 128 bytes)
  constexpr int VTR = 64 + 4;
  constexpr int NCH = 2 * 64 * D / 8;  // 16-byte chunks of K and V per page and head
  constexpr int CPT = (NCH + PF_THREADS - 1) / PF_THREADS;  // chunks per thread (last partial)
  static_assert(D % 32 == 0, "head dim");

  __shared__ uint4 Ks[2][64 * KCH];                  // double-buffered page tiles
  __shared__ __align__(16) bf16_t Vt[2][D * VTR];
  __shared__ int32_t pages[PF_MAX_PAGES];            // the tile's page ids

  const int tile = a.n_tiles - 1 - blockIdx.x;  // longest (latest) tiles first
  const int hk = blockIdx.y;
  const int32_t* tl = a.tiles + 4 * tile;
  const int row0 = tl[0], nrows = tl[1], pos0 = tl[2], seq = tl[3];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = w >> 2, qq = w & 3;  // query head, 16-row quarter
  const int h = hk * G + g;
  const int HqD = a.Hq * D;
  const int lq = lane & 15, lk = lane >> 4;

  const int kmax = pos0 + nrows - 1;
  const bool full = a.window == 0;
  const int klo = full ? 0 : max(0, pos0 - a.window + 1);
  const int pg_lo = klo / PAGE, pg_hi = kmax / PAGE;
  const int32_t* trow = a.kv.table + ((size_t)seq * a.kv.n_streams + a.stream_idx) * a.kv.tab_len;
  const bf16_t* pool = (const bf16_t*)a.kv.pool;

  // Q fragments (B operand): query 16 qq + lq, dims 32 c + 8 lk + e
  bf16x8 qf[1][DC];
#pragma unroll
  for (int qb = 0; qb < 1; ++qb) {
    const int i = 16 * qq + lq;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (i < nrows)
        v = *(const uint4*)((const bf16_t*)a.q + (size_t)(row0 + i) * HqD + (size_t)h * D + 32 * c + 8 * lk);
      qf[qb][c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  for (int i = t; i <= pg_hi - pg_lo; i += PF_THREADS) pages[i] = trow[(pg_lo + i) % a.kv.ring];
  __syncthreads();

  // K/V of page pg into registers
  auto gload = [&](int pg, uint4 (&pre)[CPT]) {
    const int32_t page = pages[pg - pg_lo];
    const bf16_t* kp = pool + (size_t)page * a.kv.page_elems + (size_t)hk * 64 * D;
    const bf16_t* vp = kp + (size_t)a.kv.Hkv * 64 * D;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int s = t + PF_THREADS * i;
      if (s < NCH) pre[i] = s < NCH / 2 ? ((const uint4*)kp)[s] : ((const uint4*)vp)[s - NCH / 2];
    }
  };
  auto sstore = [&](int pg, const uint4 (&pre)[CPT], int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int s = t + PF_THREADS * i;
      if (s >= NCH) break;
      const bool isv = s >= NCH / 2;
      const int s2 = isv ? s - NCH / 2 : s;
      if (!isv) {  // K chunk: token j, channels 8 ch .. 8 ch + 7
        int j, c8;
        kv_k_chunk(s2, D, j, c8);
        const int ch = c8 >> 3;
        Ks[buf][j * KCH + ch] = (pg * PAGE + j > kmax) ? make_uint4(0, 0, 0, 0) : pre[i];
      } else {     // V^T chunk: channel c, tokens 8 kc .. 8 kc + 7
        int c, t8;
        kv_v_chunk(s2, D, c, t8);
        const int kc = t8 >> 3;
        uint4 v = pre[i];
        const int over = pg * PAGE + 8 * kc + 7 - kmax;  // tokens past the chunk's last
        if (over > 0) {
          uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (8 * kc + e > kmax - pg * PAGE) wv[e / 2] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
        uint2* dst = (uint2*)(Vt[buf] + c * VTR + 8 * kc);  // 8-byte aligned rows
        dst[0] = make_uint2(v.x, v.y);
        dst[1] = make_uint2(v.z, v.w);
      }
    }
  };

  const float sl2 = a.scale * 1.4426950408889634f;  // logits in log2 units
  float m_run[1] = {-INFINITY}, l_run[1] = {0.f};
  f32x4 o[CB][1];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb][0] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one page per step from LDS buffer (pg - pg_lo) & 1; the next page's tiles go to the
  // other buffer (its readers passed the previous barrier) while the page after that is
  // loaded into registers
  auto compute = [&](int pg, int buf) {
    // S^T[key 16 kb + 4 lk + r][query 16 qb + lq]
    f32x4 st[4][1];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      st[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, Ks[buf][(16 * kb + lq) * KCH + 4 * c + lk]);
        st[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][c], st[kb][0], 0, 0, 0);
      }
    }
    // online softmax; probabilities packed as the PV B operand
    bf16x8 pf[1][2];
#pragma unroll
    for (int qb = 0; qb < 1; ++qb) {
      const int i = 16 * qq + lq;
      const int qpos = pos0 + i;
      const bool qv = i < nrows;
      float sv[4][4];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kpos = pg * PAGE + 16 * kb + 4 * lk + r;
          const bool vis = qv && kpos <= qpos && (full || qpos - kpos < a.window);
          sv[kb][r] = vis ? st[kb][qb][r] * sl2 : -INFINITY;
          mt = fmaxf(mt, sv[kb][r]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run[qb], mt);
      const float corr = m_run[qb] == -INFINITY ? 0.f : exp2f(m_run[qb] - m_new);
      float ps = 0.f;
      float pv[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = sv[kb][r] == -INFINITY ? 0.f : exp2f(sv[kb][r] - m_new);
          pv[kb][r] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run[qb] = l_run[qb] * corr + ps;
      m_run[qb] = m_new;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) o[cb][qb] *= corr;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          u[e / 2] = (uint32_t)f2bf(pv[2 * kc][e]) | ((uint32_t)f2bf(pv[2 * kc][e + 1]) << 16);
          u[2 + e / 2] = (uint32_t)f2bf(pv[2 * kc + 1][e]) | ((uint32_t)f2bf(pv[2 * kc + 1][e + 1]) << 16);
        }
        pf[qb][kc] = __builtin_bit_cast(bf16x8, make_uint4(u[0], u[1], u[2], u[3]));
      }
    }
    // O^T[channel 16 cb + 4 lk + r][query 16 qb + lq] += V^T P^T
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const bf16_t* vr = Vt[buf] + (16 * cb + lq) * VTR + 32 * kc + 4 * lk;
        const uint2 lo = *(const uint2*)vr;
        const uint2 hi = *(const uint2*)(vr + 16);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[cb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0][kc], o[cb][0], 0, 0, 0);
      }
    }
  };

  uint4 pre[CPT];
  gload(pg_lo, pre);
  sstore(pg_lo, pre, 0);
  if (pg_lo + 1 <= pg_hi) gload(pg_lo + 1, pre);
  __syncthreads();
  for (int pg = pg_lo; pg <= pg_hi; ++pg) {
    const int buf = (pg - pg_lo) & 1;
    if (pg + 1 <= pg_hi) sstore(pg + 1, pre, buf ^ 1);
    if (pg + 2 <= pg_hi) gload(pg + 2, pre);
    compute(pg, buf);
    __syncthreads();
  }

  // epilogue: normalise, gate, store
#pragma unroll
  for (int qb = 0; qb < 1; ++qb) {
    const int i = 16 * qq + lq;
    const bool qv = i < nrows;
    const float invl = qv ? 1.f / l_run[qb] : 0.f;
    const size_t base = (size_t)(row0 + (qv ? i : 0)) * HqD + (size_t)h * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int c = 16 * cb + 4 * lk;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[cb][qb][r] * invl;
      if (qv) {
        if (a.g) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] *= gate_at(a.g, a.g_f32, a.g_ld, a.g_splits, a.g_sstride, row0 + i, h * D + c + r);
        }
        uint2 ov;
        ov.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        ov.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *(uint2*)((bf16_t*)a.o + base + c) = ov;
      }
    }
  }
}

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t st) {
  if (a.n_tiles == 0) return hipSuccess;
  if (a.kv.act != ACT_BF16 || a.Hq != 4 * a.Hkv) return hipErrorInvalidValue;
  dim3 grid(a.n_tiles, a.Hkv);
  switch (a.d) {
    case 64:
      hipLaunchKernelGGL(k_attn_prefill<64>, grid, dim3(PF_THREADS), 0, st, a);
      break;
    case 128:
      hipLaunchKernelGGL(k_attn_prefill<128>, grid, dim3(PF_THREADS), 0, st, a);
      break;
    case 160:
      hipLaunchKernelGGL(k_attn_prefill<160>, grid, dim3(PF_THREADS), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dory
