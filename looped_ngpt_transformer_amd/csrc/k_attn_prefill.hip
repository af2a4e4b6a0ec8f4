// Prefill attention on bf16 with MFMA (flash-style online softmax over KV pages).
//
// Same maths as the row kernel: GQA (4 query heads per KV head), causal, sliding
// window W on sliding layers, softmax(scale * q.k) v, then the sigmoid output gate
// ("Dory1.0-4B": paper summary "technical novelty"; arXiv §2; MXFP8 article "hybrid
// attention").
//
// Work-group = (tile of <= 64 consecutive query rows of one sequence, KV head): 8
// waves, wave = (query head g of the group, 32-row half hh of the tile); the waves of
// half 0 (group A) and half 1 (group B) put one wave of each group on every SIMD. Per
// 64-key KV page, with v_mfma_f32_32x32x16_bf16 (on gfx950 about 1.5x the rate of the
// 16x16x32 form):
//   S^T = K Q^T   (A = K rows from LDS, B = Q in registers): two 32-key blocks whose
//   rows are read in the key order 16 (r / 16) + 8 ((r / 4) % 2) + 4 ((r / 8) % 2) + r % 4,
//   so that each lane's eight accumulators of a 16-key step hold 8 consecutive keys;
//   online softmax per query in registers (lanes l and l + 32 share query l % 32),
//   O^T += V^T P^T (A = V^T from LDS, one 16-byte chunk of 8 consecutive keys per lane;
//   B = P straight from the S^T accumulators).
// Each wave alternates two phases per page, separated by work-group barriers:
//   matrix phase:  O^T += V^T P^T of the previous page, then S^T of this page (MFMA)
//   softmax phase: masks, running maximum, exponentials, sums, rescale (VALU)
// and group B runs one phase behind group A, so on every SIMD one wave's softmax
// overlaps the other wave's MFMAs instead of both waiting for the same unit.
// The page's K and V blocks are stored as 1 KiB groups of 16-byte chunks in MFMA
// fragment order; they go straight from HBM into LDS (global_load_lds) through three
// stages: group B issues page p + 2 during its softmax phase of page p and waits for it
// at the end of its next matrix phase, one phase before group A first reads it. The
// 32x32 fragment reads of the stages are free of bank conflicts. Keys beyond the chunk's last position are masked out of the softmax; their
// V entries are multiplied by zero probabilities and hold zeros or stale finite values
// (pages are cleared when first allocated).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dory {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = PF_WAVES * 64;

typedef __attribute__((address_space(3))) void* pf_lds_t;
typedef __attribute__((address_space(1))) void* pf_gbl_t;

template <int D>
__global__ __launch_bounds__(PF_THREADS) void k_attn_prefill(AttnArgs a) {
  constexpr int G = 4;
  constexpr int KS = D / 16;       // 16-wide steps of the head dim (QK contraction)
  constexpr int CB = D / 32;       // 32-channel blocks of the output
  constexpr int DC = D / 32;       // 32-channel chunks of a K fragment group
  constexpr int CB16 = D / 16;     // 16-channel blocks of V
  constexpr int NG = D / 8;        // 1 KiB groups per K (or V) block of one head
  // K and V groups at a 1 KiB stride: the fragment reads (16-byte chunks of two groups
  // DC apart for K, 256 contiguous bytes per 16 lanes for V) then take no bank
  // conflicts (counted: a 128-byte pad on the K stride made every K read conflict
  // two-way; 256 and 512 are conflict-free as well)
  constexpr int KGS = 1024;
  constexpr int VGS = 1024;
  constexpr int STAGE = NG * (KGS + VGS);  // bytes per page stage
  constexpr int NSTAGE = 3;
  constexpr int GPB = 2 * NG / 4;  // load instructions per group-B wave per page
  static_assert(D % 32 == 0 && DC >= 1 && (DC == 5 || 128 % DC == 0), "head dim");
  static_assert((2 * NG) % 4 == 0 && 2 * GPB <= 63, "page loads split over four waves, vmcnt range");

  // one array per stage: LDS reads of one stage are then known not to alias the
  // direct-to-LDS loads in flight into the others, so they need not wait for them
  __shared__ __align__(16) unsigned char sm0[STAGE];
  __shared__ __align__(16) unsigned char sm1[STAGE];
  __shared__ __align__(16) unsigned char sm2[STAGE];
  __shared__ __align__(16) float sqk_lds[D];  // query-key scales for the query prologue
  auto stage_ptr = [&](auto S) -> unsigned char* {
    if constexpr (decltype(S)::value == 0) return sm0;
    else if constexpr (decltype(S)::value == 1) return sm1;
    else return sm2;
  };

  // Work-groups go to the 8 XCDs (each with its own L2) round-robin in linear id order.
  // Each XCD takes the tiles of one KV head (8 / Hkv XCDs per head, interleaved tile by
  // tile, so that each gets long and short tiles alike), so that the K/V pages the
  // tiles of a head share are fetched into one or two L2s instead of all eight; the
  // longest (latest) tiles of each XCD go first. Other shapes keep the plain order.
  int tile, hk;
  {
    const int n = a.n_tiles, nh = gridDim.y, xph = 8 / nh;
    const int id = blockIdx.x + blockIdx.y * n;
    if (nh <= 8 && 8 % nh == 0 && n % xph == 0) {  // a bijection of the grid onto (tile, head)
      const int x = id & 7, j = id >> 3;
      hk = x / xph;
      tile = n - 1 - (xph * j + x % xph);
    } else {
      tile = n - 1 - blockIdx.x;
      hk = blockIdx.y;
    }
  }
  const int32_t* tl = a.tiles + 4 * tile;
  const int row0 = tl[0], nrows = tl[1], pos0 = tl[2], seq = tl[3];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6) & (PF_WAVES - 1);
  const int g = w & 3, hh = w >> 2;  // query head, 32-row half = group (A: 0, B: 1)
  const int h = hk * G + g;
  const int HqD = a.Hq * D;
  const int l32 = lane & 31, lh = lane >> 5;

  const int kmax = pos0 + nrows - 1;
  const bool full = a.window == 0;
  const int klo = full ? 0 : max(0, pos0 - a.window + 1);
  const int pg_lo = klo / PAGE, pg_hi = kmax / PAGE;
  const int npg = pg_hi - pg_lo;  // pages pg_lo .. pg_lo + npg
  const int32_t* trow = a.kv.table + ((size_t)seq * a.kv.n_streams + a.stream_idx) * a.kv.tab_len;
  const bf16_t* pool = (const bf16_t*)a.kv.pool;

  // Q fragments (B operand): query 32 hh + l32, channels 16 c + 8 lh .. + 7
  const int qi = 32 * hh + l32;
  const bool qv = qi < nrows;
  const int qpos = pos0 + qi;
  bf16x8 qf[KS];  // filled below, after group B has issued its first pages

  // Page ids of relative pages 64 c .. 64 c + 63 (chunk c), one per lane. A page id read
  // from the table at issue time would put a dependent global-memory round trip in front
  // of every page's loads; held in a register it costs one lane read, and the table is
  // read again once every 64 pages.
  auto load_ids = [&](int c) -> int {
    const int rr = 64 * c + lane;
    return rr <= npg ? trow[(pg_lo + rr) % a.kv.ring] : 0;
  };
  int ids = load_ids(0);

  // relative page r -> its stage S (r % 3): group-B wave g loads groups g, g + 4, ...
  // (K groups 0..NG-1, then V)
  auto issue = [&](int r, auto S) {
    if (r > 0 && (r & 63) == 0) ids = load_ids(r >> 6);
    const int32_t page = __builtin_amdgcn_readlane(ids, r & 63);
    const unsigned char* kb = (const unsigned char*)(pool + (size_t)page * a.kv.page_elems + (size_t)hk * 64 * D);
    const unsigned char* vb = (const unsigned char*)(pool + (size_t)page * a.kv.page_elems + (size_t)(a.kv.Hkv + hk) * 64 * D);
    unsigned char* st0 = stage_ptr(S);
#pragma unroll
    for (int q = 0; q < GPB; ++q) {
      const int grp = g + 4 * q;
      const bool isv = grp >= NG;
      const int gi = isv ? grp - NG : grp;
      const unsigned char* src = (isv ? vb : kb) + gi * 1024 + lane * 16;
      unsigned char* dst = st0 + (isv ? NG * KGS + gi * VGS : gi * KGS);
      __builtin_amdgcn_global_load_lds((pf_gbl_t)src, (pf_lds_t)dst, 16, 0, 0);
    }
  };

  // per-lane parts of the fragment addresses (bytes within a stage)
  //   K fragment (key block hf, 16-channel step c), A row l32 = key
  //   u = 16 (l32 / 16) + 8 ((l32 / 4) % 2) + 4 ((l32 / 8) % 2) + l32 % 4 of the block:
  //   group (2 hf + (u / 4) % 2) DC + c / 2, chunk (2 (c % 2) + lh) 16 + 4 (u / 8) + u % 4
  const int koff = ((l32 >> 3) & 1) * DC * KGS +
                   (lh * 16 + ((l32 >> 4) << 3) + (((l32 >> 2) & 1) << 2) + (l32 & 3)) * 16;
  //   V fragment (channel block cb, key step s): group (s / 2) CB16 + 2 cb + l32 / 16,
  //   chunk (2 (s % 2) + lh) 16 + l32 % 16 (keys 16 s + 8 lh .. + 7 of channel l32)
  const int voff = NG * KGS + (l32 >> 4) * VGS + (lh * 16 + (l32 & 15)) * 16;
  const float sl2 = a.scale * 1.4426950408889634f;  // logits in log2 units
  // With q and k L2-normalised and scaled by s_qk, |q.k| <= max s_qk^2, so no logit
  // exceeds B = scale * max s_qk^2 in magnitude (log2 units here, with a margin for the
  // bf16 rounding of q and k). Softmax is unchanged by a common shift of the logits, and
  // for B < 60 every 2^logit lies in [2^-60, 2^60], well inside the normal range of
  // float and bf16, with row sums far from overflow; then the probabilities are taken
  // as 2^logit directly: no running maximum, no rescaling of the accumulators. In that
  // case q carries the factor scale * log2(e) (folded into its normalisation), so that
  // the S^T accumulators already hold log2-unit logits and each probability is one
  // exponential.
  float bound = INFINITY;
  if (a.s_qk) {
    float m = 0.f;
    for (int i = lane; i < D; i += 64) m = fmaxf(m, fabsf(a.s_qk[i]));
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) m = fmaxf(m, __shfl_xor(m, o2, 64));
    bound = sl2 * m * m * 1.02f + 0.5f;
  }
  const bool fixed_ref = sl2 > 0.f && bound < 60.f;  // uniform over the work-group
  const float qscale = fixed_ref ? sl2 : 1.f;         // factor carried by q
  // m_run: running maximum (log2 units) of the query's visible logits; l_run: this
  // lane's part (its 32 keys of each page) of the softmax denominator, relative to the
  // current reference
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.f;
  // S^T[key 32 kb + 16 (r / 8) + 8 lh + r % 8][query l32] of the current page, and the
  // previous page's probabilities as P^T fragments (slot e of 16-key step s: key
  // 16 s + 8 lh + e, accumulator 8 (s % 2) + e of block s / 2)
  f32x16 st[2];
  bf16x8 pf[4];

  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // matrix phase: O^T += V^T P^T of relative page r - 1 (stage SV), then S^T of page r
  // (stage SK); group B then waits for the page it issued in its last softmax phase
  auto matrix_phase = [&](bool pv, bool sk, auto SK, auto SV) {
    // fragments double-buffered by step: the reads of step i + 1 are issued before the
    // MFMAs of step i, so LDS latency overlaps the matrix core
    if (pv) {
      const unsigned char* sv = stage_ptr(SV) + voff;
      bf16x8 vf[2][CB];
      auto ldv = [&](int s, bf16x8 (&dst)[CB]) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          dst[cb] = *(const bf16x8*)(sv + ((s >> 1) * CB16 + 2 * cb) * VGS + (s & 1) * 32 * 16);
      };
      ldv(0, vf[0]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s + 1 < 4) ldv(s + 1, vf[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)  // the CB output blocks: independent chains
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s & 1][cb], pf[s], o[cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (sk) {
      const unsigned char* sk0 = stage_ptr(SK) + koff;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
      bf16x8 kf[2][2];
      auto ldk = [&](int c, bf16x8 (&dst)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          dst[kb] = *(const bf16x8*)(sk0 + (2 * kb * DC + (c >> 1)) * KGS + (c & 1) * 32 * 16);
      };
      ldk(0, kf[0]);
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        if (c + 1 < KS) ldk(c + 1, kf[(c + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)  // the two key blocks: independent chains
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c & 1][kb], qf[c], st[kb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (hh == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier();
  };
  // softmax phase of relative page r (absolute pg_lo + r); group B also issues page
  // r + 2 into stage SI
  auto softmax_phase = [&](int r, auto SI) {
    if (hh == 1 && r + 2 <= npg) issue(r + 2, SI);
    const int pg = pg_lo + r;
    // pages every query of the tile sees in full skip the per-key masks
    const bool all_vis = pg * PAGE + PAGE - 1 <= pos0 && (full || pos0 + nrows - 1 - pg * PAGE < a.window);
    if (fixed_ref) {
      if (!all_vis) {
        const int wlim = full ? 0x7fffffff : a.window;  // keys visible at 0 <= qpos - kpos < wlim
        const int d0 = qv ? qpos - pg * PAGE - 8 * lh : -1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int dlt = d0 - (32 * kb + 16 * (e >> 3) + (e & 7));  // qpos - kpos
            st[kb][e] = (dlt >= 0) & (dlt < wlim) ? st[kb][e] : -INFINITY;
          }
      }
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(st[kb][e]);  // log2 units already; exp2(-inf) = 0
          st[kb][e] = p;
          ps[kb] += p;
        }
      l_run += ps[0] + ps[1];
    } else {
    float mt = -INFINITY;
    if (all_vis) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, st[kb][e]);
    } else {
      const int wlim = full ? 0x7fffffff : a.window;  // keys visible at 0 <= qpos - kpos < wlim
      const int d0 = qv ? qpos - pg * PAGE - 8 * lh : -1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dlt = d0 - (32 * kb + 16 * (e >> 3) + (e & 7));  // qpos - kpos
          const bool vis = (dlt >= 0) & (dlt < wlim);
          st[kb][e] = vis ? st[kb][e] : -INFINITY;
          mt = fmaxf(mt, st[kb][e]);
        }
    }
    // raw logits so far: the running maximum is kept in scaled (log2) units, the scale
    // being positive, and the scale is applied inside the exponent's FMA
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * sl2;
    const float m_new = fmaxf(m_run, mt);
    // a query that has seen no visible key yet keeps m = -inf; its (all -inf) logits
    // give p = exp2(-inf) = 0 against a finite reference instead of NaN
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[kb][e], sl2, -m_ref));  // exp2(-inf) = 0
        st[kb][e] = p;
        ps[kb] += p;
      }
    if (!__all(m_new == m_run)) {  // rescale only when some query's maximum moved
      const float corr = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) o[cb] *= corr;
    }
    l_run += ps[0] + ps[1];
    m_run = m_new;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) u[e / 2] = pack_bf16x2(st[s >> 1][8 * (s & 1) + e], st[s >> 1][8 * (s & 1) + e + 1]);
      pf[s] = __builtin_bit_cast(bf16x8, make_uint4(u[0], u[1], u[2], u[3]));
    }
    barrier();
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  auto load_q = [&]() {
    if (a.rope_cs) {
      // unrotated q from the projection output: channel x (< D/2) pairs with x + D/2,
      // which this lane holds in fragment c + KS/2; lane ^ 32 holds the rest of the row.
      // The tile's block of the (cos, sin) table (64 rows x D/2 pairs, chunk-major: the
      // size of a page stage) goes straight into stage 2, which no page uses before group
      // B's first softmax phase, and the query-key scales into LDS: each is read from HBM
      // or L2 once per work-group instead of once per wave. Chunk-major, the 16-byte reads
      // of 32 consecutive rows below are consecutive, free of bank conflicts.
      constexpr int HS = KS / 2, HALF = D / 2;
      static_assert(64 * HALF * 8 == STAGE && STAGE % (PF_WAVES * 1024) == 0, "a tile's block fills one stage");
      const unsigned char* csg = (const unsigned char*)(a.rope_cs + (size_t)tile * 64 * D);
#pragma unroll
      for (int b = w; b < STAGE / 1024; b += PF_WAVES)
        __builtin_amdgcn_global_load_lds((pf_gbl_t)(csg + (size_t)b * 1024 + lane * 16), (pf_lds_t)(sm2 + b * 1024), 16,
                                         0, 0);
      const bf16_t* qr = (const bf16_t*)a.q_raw + (size_t)(row0 + qi) * a.q_ld + (size_t)h * D + 8 * lh;
      uint4 x1[HS], x2[HS];
#pragma unroll
      for (int c = 0; c < HS; ++c) {
        x1[c] = x2[c] = make_uint4(0, 0, 0, 0);
        if (qv) {
          x1[c] = *(const uint4*)(qr + 16 * c);
          x2[c] = *(const uint4*)(qr + HALF + 16 * c);
        }
      }
      if (t < D) sqk_lds[t] = a.s_qk ? a.s_qk[t] : 1.f;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's (cos, sin) chunks are in LDS
      __syncthreads();
      const unsigned char* csl = sm2 + (size_t)(64 * 4 * lh + qi) * 16;  // chunk 4 lh of row qi
      float r1[HS][8], r2[HS][8];
      float sq = 0.f;
#pragma unroll
      for (int c = 0; c < HS; ++c) {
        float4 cs[4] = {};
        if (qv) {
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[e] = *(const float4*)(csl + (8 * c + e) * 64 * 16);  // chunk 8 c + 4 lh + e
        }
        float s1[8], s2[8];
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
          const float4 v1 = *(const float4*)(sqk_lds + 16 * c + 8 * lh + e);
          const float4 v2 = *(const float4*)(sqk_lds + HALF + 16 * c + 8 * lh + e);
          s1[e] = v1.x; s1[e + 1] = v1.y; s1[e + 2] = v1.z; s1[e + 3] = v1.w;
          s2[e] = v2.x; s2[e + 1] = v2.y; s2[e + 2] = v2.z; s2[e + 3] = v2.w;
        }
        const uint32_t w1[4] = {x1[c].x, x1[c].y, x1[c].z, x1[c].w}, w2[4] = {x2[c].x, x2[c].y, x2[c].z, x2[c].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a1 = __uint_as_float((e & 1) ? (w1[e / 2] & 0xFFFF0000u) : (w1[e / 2] << 16));
          const float a2 = __uint_as_float((e & 1) ? (w2[e / 2] & 0xFFFF0000u) : (w2[e / 2] << 16));
          const float co = (e & 1) ? cs[e / 2].z : cs[e / 2].x, sn = (e & 1) ? cs[e / 2].w : cs[e / 2].y;
          const float v1 = a1 * co - a2 * sn, v2 = a1 * sn + a2 * co;
          sq += v1 * v1 + v2 * v2;
          r1[c][e] = v1 * s1[e];
          r2[c][e] = v2 * s2[e];
        }
      }
      sq += __shfl_xor(sq, 32, 64);
      const float sc = (a.s_qk ? inv_norm(sq) : 1.f) * qscale;
#pragma unroll
      for (int c = 0; c < HS; ++c) {
        uint32_t o1[4], o2[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          o1[e / 2] = pack_bf16x2(r1[c][e] * sc, r1[c][e + 1] * sc);
          o2[e / 2] = pack_bf16x2(r2[c][e] * sc, r2[c][e + 1] * sc);
        }
        qf[c] = __builtin_bit_cast(bf16x8, make_uint4(o1[0], o1[1], o1[2], o1[3]));
        qf[c + HS] = __builtin_bit_cast(bf16x8, make_uint4(o2[0], o2[1], o2[2], o2[3]));
      }
    } else {
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qv) v = *(const uint4*)((const bf16_t*)a.q + (size_t)(row0 + qi) * HqD + (size_t)h * D + 16 * c + 8 * lh);
        if (fixed_ref) {
          uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wv[e] = pack_bf16x2(__uint_as_float(wv[e] << 16) * qscale, __uint_as_float(wv[e] & 0xFFFF0000u) * qscale);
          v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
        qf[c] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  // group B issues pages 0 and 1 before the query loads, so their latencies overlap;
  // then it runs one phase behind group A
  if (hh == 1) {
    issue(0, S0{});
    if (npg >= 1) issue(1, S1{});
  }
  load_q();
  if (hh == 1) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier\n\ts_barrier" ::: "memory");
  else asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // relative page r lives in stage r % 3; the loop is unrolled by the stage count so
  // every stage index is a compile-time constant
  for (int r = 0; r <= npg; r += 3) {
    matrix_phase(r > 0, true, S0{}, S2{});
    softmax_phase(r, S2{});
    if (r + 1 <= npg) {
      matrix_phase(true, true, S1{}, S0{});
      softmax_phase(r + 1, S0{});
    }
    if (r + 2 <= npg) {
      matrix_phase(true, true, S2{}, S1{});
      softmax_phase(r + 2, S1{});
    }
  }
  // O^T += V^T P^T of the last page
  switch (npg % 3) {
    case 0: matrix_phase(true, false, S1{}, S0{}); break;
    case 1: matrix_phase(true, false, S2{}, S1{}); break;
    default: matrix_phase(true, false, S0{}, S2{}); break;
  }

  // epilogue: normalise, gate, store; lane holds 4 consecutive channels per (cb, r / 4).
  // The bf16 gate pre-activations of those channels (8 bytes each) are all requested
  // before the first is used.
  const float lsum = l_run + __shfl_xor(l_run, 32, 64);  // both halves of the query's keys
  if (qv) {
    const float invl = 1.f / lsum;
    const size_t base = (size_t)(row0 + qi) * HqD + (size_t)h * D;
    uint2 graw[CB][4];
    const bool gbf = a.g != nullptr;  // bf16 (the launcher rejects float gates)
    if (gbf) {
      const bf16_t* gr = (const bf16_t*)a.g + (size_t)(row0 + qi) * a.g_ld + (size_t)h * D + 4 * lh;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) graw[cb][rb] = *(const uint2*)(gr + 32 * cb + 8 * rb);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int c = 32 * cb + 8 * rb + 4 * lh;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = o[cb][4 * rb + r] * invl;
        if (gbf) {
          const uint32_t gw[2] = {graw[cb][rb].x, graw[cb][rb].y};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = __uint_as_float((gw[r >> 1] >> (16 * (r & 1))) << 16);
            v[r] *= sigmoid(x);
          }
        }
        uint2 ov;
        ov.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        ov.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *(uint2*)((bf16_t*)a.o + base + c) = ov;
      }
    }
  }
  if (hh == 0) asm volatile("s_barrier" ::: "memory");  // matches group B's extra first barrier
}

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t st) {
  if (a.n_tiles == 0) return hipSuccess;
  if (a.kv.act != ACT_BF16 || a.Hq != 4 * a.Hkv || (a.g && a.g_f32)) return hipErrorInvalidValue;
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
