// Fused nGPT residual update and loop boundary (one work-group per row).
//
// s <- N((1 - a) * s + a * N(y))  — the nGPT update ("Dory1.0-4B" paper summary,
// nGPT prerequisite; arXiv summary §2: normalised sublayer output blended with the
// normalised residual by per-channel rates, then normalised). y arrives as split-K
// partial sums (decode) or as one bf16 array (prefill: the sublayer output in the
// activation type). The L2 norm the pages put before the output and down projections (arXiv
// §2) scales y's row by a positive factor, which N(y) removes, so it needs no work.
// Loop boundaries (paper summary, core-method equation): at the end of the input block
// x is saved and u_1 = N(x + x); at the end of loop t, s_t = N(.) and, unless t = k,
// u_{t+1} = N(s_t + x).
//
// All of the row's loads (partials, state, rates, x) are issued first. Every norm the
// update and the boundary need follows from sums over the row taken in one pass
// (wave shuffles plus one LDS exchange): with t = (1 - a) s + a y / ||y||,
//   ||t||^2 = sum((1-a)s)^2 + 2 sum((1-a)s a y) / ||y|| + sum(a y)^2 / ||y||^2,
// and for u = N(s_t + x), s_t . x = (sum((1-a)s x) + sum(a y x) / ||y||) / ||t||. The row
// stays in registers.
#include "common.h"
#include "kernels.h"

namespace dory {

// 8 fp16 values (one 16-byte chunk) <-> floats; the stores round to nearest even
__device__ __forceinline__ void f16x8_to_f32(const uint4& w, float* out) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 h = __builtin_bit_cast(h2, ws[i]);
    out[2 * i] = (float)h[0];
    out[2 * i + 1] = (float)h[1];
  }
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// THREADS per row: 512 for many rows, 1024 for few rows (decode) so that each row's
// loads are spread over more waves.
template <typename SB, int UPD_THREADS>
__global__ __launch_bounds__(UPD_THREADS) void k_update(UpdateArgs u) {
  constexpr int UPD_MAXPER = 4096 / UPD_THREADS;  // H <= 4096
  constexpr int NW = UPD_THREADS / WAVE;
  constexpr int NS = 7;  // sums: yy, A, B, C, (1-a)s.x, a y.x, x.x
  __shared__ float red[NW][NS];
  const int m = blockIdx.x;
  const int H = u.H;
  const size_t row = (size_t)m * H;
  const int bnd = u.bnd == BND_LOOP_CONTINUE && m >= u.final_from ? BND_LOOP_FINAL : u.bnd;
  const bool need_x = bnd == BND_LOOP_CONTINUE;
  float yv[UPD_MAXPER], sv[UPD_MAXPER], av[UPD_MAXPER], xv[UPD_MAXPER];
  float acc[NS] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) {
    const int i = threadIdx.x + k * UPD_THREADS;
    yv[k] = sv[k] = av[k] = xv[k] = 0.f;
    if (i < H) {
      if (u.y_bf16) yv[k] = bf2f(((const bf16_t*)u.y)[row + i]);
      sv[k] = u.s[row + i];
      av[k] = u.alpha[i];
      if (need_x) xv[k] = u.x[row + i];
    }
  }
  if (!u.y_bf16) {
    // split partials: QS splits of every element of the thread requested together
    constexpr int QS = UPD_MAXPER >= 16 ? 1 : 16 / UPD_MAXPER;
    const size_t sstride = (size_t)u.M * H;
    for (int s0 = 0; s0 < u.splits; s0 += QS) {
      float v[QS][UPD_MAXPER];
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int k = 0; k < UPD_MAXPER; ++k) {
          const int i = threadIdx.x + k * UPD_THREADS;
          v[q][k] = (s0 + q < u.splits && i < H) ? u.y[(s0 + q) * sstride + row + i] : 0.f;
        }
#pragma unroll
      for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int k = 0; k < UPD_MAXPER; ++k) yv[k] += v[q][k];
    }
  }
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) {
    const float y = yv[k];
    const float bs = (1.f - av[k]) * sv[k], ay = av[k] * y;
    acc[0] += y * y;
    acc[1] += bs * bs;
    acc[2] += bs * ay;
    acc[3] += ay * ay;
    acc[4] += bs * xv[k];
    acc[5] += ay * xv[k];
    acc[6] += xv[k] * xv[k];
  }
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = wave_sum(acc[q]);
  if ((threadIdx.x & (WAVE - 1)) == 0)
#pragma unroll
    for (int q = 0; q < NS; ++q) red[threadIdx.x / WAVE][q] = acc[q];
  __syncthreads();
  float tot[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    tot[q] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[q] += red[w][q];
  }
  const float ny = inv_norm(tot[0]);
  const float tt = fmaxf(tot[1] + 2.f * tot[2] * ny + tot[3] * ny * ny, 0.f);  // ||t||^2
  const float nt = inv_norm(tt);
  float scale = nt;          // s' = t * nt
  float norm_sp = sqrtf(tt) * nt;  // ||s'||
  float add_x = 0.f;         // coefficient of x in the result
  if (bnd == BND_LOOP_CONTINUE || bnd == BND_LOOP_FINAL) {  // s_t = N(F(u_t))
    const float n2 = inv_norm(norm_sp * norm_sp);
    scale *= n2;
    norm_sp *= n2;
  }
  if (bnd == BND_LOOP_CONTINUE) {  // u = N(s_t + x)
    const float dot = (tot[4] + tot[5] * ny) * scale;  // s_t . x
    const float n3 = inv_norm(norm_sp * norm_sp + 2.f * dot + tot[6]);
    scale *= n3;
    add_x = n3;
  } else if (bnd == BND_SAVE_X) {  // x = s'; u = N(s' + s')
    const float n3 = inv_norm(4.f * norm_sp * norm_sp);
    float* X = u.x;
#pragma unroll
    for (int k = 0; k < UPD_MAXPER; ++k) {
      const int i = threadIdx.x + k * UPD_THREADS;
      if (i < H) X[row + i] = ((1.f - av[k]) * sv[k] + av[k] * yv[k] * ny) * nt;
    }
    scale *= 2.f * n3;
  }
  SB* sb = (SB*)u.sb;
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) {
    const int i = threadIdx.x + k * UPD_THREADS;
    if (i < H) {
      const float t = (1.f - av[k]) * sv[k] + av[k] * yv[k] * ny;
      const float v = t * scale + add_x * xv[k];
      u.s_out[row + i] = v;
      if (sb) st<SB>(sb, row + i, v);
    }
  }
}

// Decode form (y as split partials, H % 256 == 0, H <= 4096): H / 4 threads per row, each
// owning 4 consecutive channels, so that every access is one 16-byte load or store and a
// thread requests the partials of up to 16 splits at once (summed in split order).
template <typename SB>
__global__ __launch_bounds__(1024) void k_update_split4(UpdateArgs u) {
  constexpr int NS = 7, QS = 16;
  __shared__ float red[1024 / WAVE][NS];
  const int H = u.H, NW = blockDim.x / WAVE;
  const size_t row = (size_t)blockIdx.x * H;
  const int i0 = 4 * threadIdx.x;
  const int bnd = u.bnd == BND_LOOP_CONTINUE && (int)blockIdx.x >= u.final_from ? BND_LOOP_FINAL : u.bnd;
  const bool need_x = bnd == BND_LOOP_CONTINUE;
  const size_t sstride = (size_t)u.M * H;
  const float4 s4 = *(const float4*)(u.s + row + i0), a4 = *(const float4*)(u.alpha + i0);
  const float4 x4 = need_x ? *(const float4*)(u.x + row + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
  float yv[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < u.splits; s0 += QS) {
    float4 v[QS];
#pragma unroll
    for (int q = 0; q < QS; ++q)
      v[q] = s0 + q < u.splits ? *(const float4*)(u.y + (s0 + q) * sstride + row + i0) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      yv[0] += v[q].x;
      yv[1] += v[q].y;
      yv[2] += v[q].z;
      yv[3] += v[q].w;
    }
  }
  const float sv[4] = {s4.x, s4.y, s4.z, s4.w}, av[4] = {a4.x, a4.y, a4.z, a4.w}, xv[4] = {x4.x, x4.y, x4.z, x4.w};
  float acc[NS] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float bs = (1.f - av[e]) * sv[e], ay = av[e] * yv[e];
    acc[0] += yv[e] * yv[e];
    acc[1] += bs * bs;
    acc[2] += bs * ay;
    acc[3] += ay * ay;
    acc[4] += bs * xv[e];
    acc[5] += ay * xv[e];
    acc[6] += xv[e] * xv[e];
  }
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = wave_sum(acc[q]);
  if ((threadIdx.x & (WAVE - 1)) == 0)
#pragma unroll
    for (int q = 0; q < NS; ++q) red[threadIdx.x / WAVE][q] = acc[q];
  __syncthreads();
  float tot[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    tot[q] = 0.f;
    for (int w = 0; w < NW; ++w) tot[q] += red[w][q];
  }
  const float ny = inv_norm(tot[0]);
  const float tt = fmaxf(tot[1] + 2.f * tot[2] * ny + tot[3] * ny * ny, 0.f);
  const float nt = inv_norm(tt);
  float scale = nt, norm_sp = sqrtf(tt) * nt, add_x = 0.f;
  if (bnd == BND_LOOP_CONTINUE || bnd == BND_LOOP_FINAL) {
    const float n2 = inv_norm(norm_sp * norm_sp);
    scale *= n2;
    norm_sp *= n2;
  }
  float t[4], v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) t[e] = (1.f - av[e]) * sv[e] + av[e] * yv[e] * ny;
  if (bnd == BND_LOOP_CONTINUE) {
    const float dot = (tot[4] + tot[5] * ny) * scale;
    const float n3 = inv_norm(norm_sp * norm_sp + 2.f * dot + tot[6]);
    scale *= n3;
    add_x = n3;
  } else if (bnd == BND_SAVE_X) {
    const float n3 = inv_norm(4.f * norm_sp * norm_sp);
    *(float4*)(u.x + row + i0) = make_float4(t[0] * nt, t[1] * nt, t[2] * nt, t[3] * nt);
    scale *= 2.f * n3;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = t[e] * scale + add_x * xv[e];
  *(float4*)(u.s_out + row + i0) = make_float4(v[0], v[1], v[2], v[3]);
  if (u.sb) {
    if constexpr (sizeof(SB) == 2)
      *(uint2*)((bf16_t*)u.sb + row + i0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    else
      *(float4*)((float*)u.sb + row + i0) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Prefill form (y one bf16 array, H % 8 == 0, H <= 8 T): each thread owns 8 consecutive
// channels of the row, so every access is 16 or 32 bytes wide; same sums and algebra.
// With state_act the state between sublayers is kept in fp16 (s16, rewritten in place:
// each thread rewrites only the channels it read) beside its bf16 GEMM copy, so an update
// moves y, s, the new s and its copy at 2 bytes each: 8 bytes per element instead of 14.
template <typename SB, int T>
__global__ __launch_bounds__(T) void k_update_vec(UpdateArgs u) {
  constexpr int NW = T / WAVE;
  constexpr int NS = 7;
  __shared__ float red[NW][NS];
  const int H = u.H;
  const size_t row = (size_t)blockIdx.x * H;
  const int i0 = threadIdx.x * 8;
  const bool act = i0 < H;
  const int bnd = u.bnd == BND_LOOP_CONTINUE && (int)blockIdx.x >= u.final_from ? BND_LOOP_FINAL : u.bnd;
  const bool need_x = bnd == BND_LOOP_CONTINUE;
  float yv[8], sv[8], av[8], xv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) yv[e] = sv[e] = av[e] = xv[e] = 0.f;
  if (act) {
    const uint4 yr = *(const uint4*)((const bf16_t*)u.y + row + i0);
    const float4 a0 = *(const float4*)(u.alpha + i0), a1 = *(const float4*)(u.alpha + i0 + 4);
    const uint32_t yw[4] = {yr.x, yr.y, yr.z, yr.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) yv[e] = __uint_as_float((e & 1) ? (yw[e / 2] & 0xFFFF0000u) : (yw[e / 2] << 16));
    if (u.state_act) {  // fp16 state: 8 channels in one 16-byte load
      f16x8_to_f32(*(const uint4*)((const uint16_t*)u.s16 + row + i0), sv);
    } else {
      const float4 s0 = *(const float4*)(u.s + row + i0), s1 = *(const float4*)(u.s + row + i0 + 4);
      sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w; sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
    }
    av[0] = a0.x; av[1] = a0.y; av[2] = a0.z; av[3] = a0.w; av[4] = a1.x; av[5] = a1.y; av[6] = a1.z; av[7] = a1.w;
    if (need_x) {
      const float4 x0 = *(const float4*)(u.x + row + i0), x1 = *(const float4*)(u.x + row + i0 + 4);
      xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w; xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
    }
  }
  float acc[NS] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float bs = (1.f - av[e]) * sv[e], ay = av[e] * yv[e];
    acc[0] += yv[e] * yv[e];
    acc[1] += bs * bs;
    acc[2] += bs * ay;
    acc[3] += ay * ay;
    acc[4] += bs * xv[e];
    acc[5] += ay * xv[e];
    acc[6] += xv[e] * xv[e];
  }
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = wave_sum(acc[q]);
  if ((threadIdx.x & (WAVE - 1)) == 0)
#pragma unroll
    for (int q = 0; q < NS; ++q) red[threadIdx.x / WAVE][q] = acc[q];
  __syncthreads();
  float tot[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    tot[q] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot[q] += red[w][q];
  }
  const float ny = inv_norm(tot[0]);
  const float tt = fmaxf(tot[1] + 2.f * tot[2] * ny + tot[3] * ny * ny, 0.f);
  const float nt = inv_norm(tt);
  float scale = nt, norm_sp = sqrtf(tt) * nt, add_x = 0.f;
  if (bnd == BND_LOOP_CONTINUE || bnd == BND_LOOP_FINAL) {
    const float n2 = inv_norm(norm_sp * norm_sp);
    scale *= n2;
    norm_sp *= n2;
  }
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (1.f - av[e]) * sv[e] + av[e] * yv[e] * ny;
  if (bnd == BND_LOOP_CONTINUE) {
    const float dot = (tot[4] + tot[5] * ny) * scale;
    const float n3 = inv_norm(norm_sp * norm_sp + 2.f * dot + tot[6]);
    scale *= n3;
    add_x = n3;
  } else if (bnd == BND_SAVE_X) {
    const float n3 = inv_norm(4.f * norm_sp * norm_sp);
    if (act) {
      *(float4*)(u.x + row + i0) = make_float4(t[0] * nt, t[1] * nt, t[2] * nt, t[3] * nt);
      *(float4*)(u.x + row + i0 + 4) = make_float4(t[4] * nt, t[5] * nt, t[6] * nt, t[7] * nt);
    }
    scale *= 2.f * n3;
  }
  if (!act) return;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = t[e] * scale + add_x * xv[e];
  if (u.s_out) {
    *(float4*)(u.s_out + row + i0) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(u.s_out + row + i0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  if (u.state_act)
    *(uint4*)((uint16_t*)u.s16 + row + i0) =
        make_uint4(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7]));
  if (u.sb) {
    if constexpr (sizeof(SB) == 2) {
      *(uint4*)((bf16_t*)u.sb + row + i0) =
          make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
      *(float4*)((float*)u.sb + row + i0) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)((float*)u.sb + row + i0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// Prefill form with the fp16 state (state_act, H = 512 NC): one wave per row, lane l
// holding channels 512 c + 8 l .. + 7 (c < NC) of y, s and the rates, so each load
// instruction of a wave reads one contiguous KiB. Four rows per work-group and no LDS or
// barrier: every row of the launch has its loads in flight in one round, and the 7 row
// sums are wave reductions only. y (bf16) and s (fp16) stay packed in registers and are
// widened where they are used; the new state goes out as fp16 and as the bf16 GEMM copy.
template <int NC>
__global__ __launch_bounds__(256) void k_update_wave(UpdateArgs u) {
  constexpr int NS = 7;
  const int lane = threadIdx.x & (WAVE - 1);
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= u.M) return;
  const size_t row = (size_t)m * u.H;
  const int bnd = u.bnd == BND_LOOP_CONTINUE && m >= u.final_from ? BND_LOOP_FINAL : u.bnd;
  const bool need_x = bnd == BND_LOOP_CONTINUE;
  const bf16_t* Y = (const bf16_t*)u.y + row;
  const uint16_t* S = (const uint16_t*)u.s16 + row;
  uint4 yr[NC], sr[NC];
  float av[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 512 * c + 8 * lane;
    yr[c] = *(const uint4*)(Y + i);
    sr[c] = *(const uint4*)(S + i);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = 512 * c + 8 * lane;
    const float4 a0 = *(const float4*)(u.alpha + i), a1 = *(const float4*)(u.alpha + i + 4);
    av[c][0] = a0.x; av[c][1] = a0.y; av[c][2] = a0.z; av[c][3] = a0.w;
    av[c][4] = a1.x; av[c][5] = a1.y; av[c][6] = a1.z; av[c][7] = a1.w;
  }
  auto widen = [](const uint4& w, int e) -> float {  // bf16 element e
    const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
  };
  auto widen_h = [](const uint4& w, int e) -> float {  // fp16 element e
    const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((e & 1) ? x >> 16 : x & 0xFFFFu));
  };
  float acc[NS] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = widen(yr[c], e), bs = (1.f - av[c][e]) * widen_h(sr[c], e), ay = av[c][e] * y;
      acc[0] += y * y;
      acc[1] += bs * bs;
      acc[2] += bs * ay;
      acc[3] += ay * ay;
    }
  if (need_x) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 x0 = *(const float4*)(u.x + row + 512 * c + 8 * lane);
      const float4 x1 = *(const float4*)(u.x + row + 512 * c + 8 * lane + 4);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bs = (1.f - av[c][e]) * widen_h(sr[c], e), ay = av[c][e] * widen(yr[c], e);
        acc[4] += bs * xs[e];
        acc[5] += ay * xs[e];
        acc[6] += xs[e] * xs[e];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = wave_sum(acc[q]);
  const float ny = inv_norm(acc[0]);
  const float tt = fmaxf(acc[1] + 2.f * acc[2] * ny + acc[3] * ny * ny, 0.f);
  const float nt = inv_norm(tt);
  float scale = nt, norm_sp = sqrtf(tt) * nt, add_x = 0.f;
  if (bnd == BND_LOOP_CONTINUE || bnd == BND_LOOP_FINAL) {
    const float n2 = inv_norm(norm_sp * norm_sp);
    scale *= n2;
    norm_sp *= n2;
  }
  if (bnd == BND_LOOP_CONTINUE) {
    const float dot = (acc[4] + acc[5] * ny) * scale;
    const float n3 = inv_norm(norm_sp * norm_sp + 2.f * dot + acc[6]);
    scale *= n3;
    add_x = n3;
  } else if (bnd == BND_SAVE_X) {
    scale *= 2.f * inv_norm(4.f * norm_sp * norm_sp);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const size_t i = row + 512 * c + 8 * lane;
    float xs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (need_x) {  // x again (from L2): it is read only at a loop's end
      const float4 x0 = *(const float4*)(u.x + i), x1 = *(const float4*)(u.x + i + 4);
      xs[0] = x0.x; xs[1] = x0.y; xs[2] = x0.z; xs[3] = x0.w; xs[4] = x1.x; xs[5] = x1.y; xs[6] = x1.z; xs[7] = x1.w;
    }
    float t[8], v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      t[e] = (1.f - av[c][e]) * widen_h(sr[c], e) + av[c][e] * widen(yr[c], e) * ny;
      v[e] = t[e] * scale + add_x * xs[e];
    }
    if (bnd == BND_SAVE_X) {
      *(float4*)(u.x + i) = make_float4(t[0] * nt, t[1] * nt, t[2] * nt, t[3] * nt);
      *(float4*)(u.x + i + 4) = make_float4(t[4] * nt, t[5] * nt, t[6] * nt, t[7] * nt);
    }
    *(uint4*)((bf16_t*)u.sb + i) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    *(uint4*)((uint16_t*)u.s16 + i) =
        make_uint4(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7]));
    if (u.s_out) {
      *(float4*)(u.s_out + i) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(u.s_out + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

template <typename SB>
__global__ __launch_bounds__(256) void k_stage_input(const float* x, float* s, SB* sb, size_t n, const int32_t* rows,
                                                     int H, _Float16* s16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t src = rows ? (size_t)rows[i / H] * H + i % H : i;
    const float v = x[src];
    if (s) s[i] = v;
    if (s16) s16[i] = (_Float16)v;
    st<SB>(sb, i, v);
  }
}

__global__ __launch_bounds__(256) void k_scatter_rows(const float* s, const int32_t* rows, int H, size_t n, float* y) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    y[(size_t)rows[i / H] * H + i % H] = s[i];
}

// Verification that reuses a draft's activations (self-speculative decoding, arXiv
// summary §6.2): x and the first loop's state s_1 of each row come from the draft pass;
// the state entering loop 2 is u_2 = N(s_1 + x). One block per row; rows[r] names the
// caller's row of internal row r (null: the same).
template <typename SB>
__global__ __launch_bounds__(256) void k_resume_state(const float* x_in, const float* s1_in, const int32_t* rows,
                                                      int H, float* x, float* s, SB* sb) {
  __shared__ float red[4];
  const size_t r = blockIdx.x;
  const size_t src = (rows ? (size_t)rows[r] : r) * H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H; c += 256) {
    const float v = s1_in[src + c] + x_in[src + c];
    ss += v * v;
  }
  const float inv = inv_norm(block_sum<4>(ss, red));
  for (int c = threadIdx.x; c < H; c += 256) {
    const float xv = x_in[src + c];
    const float v = (s1_in[src + c] + xv) * inv;
    x[r * H + c] = xv;
    s[r * H + c] = v;
    st<SB>(sb, r * H + c, v);
  }
}

hipError_t launch_resume_state(const float* x_in, const float* s1_in, const int32_t* rows, int M, int H, float* x,
                               float* s, void* sb, int act, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (act == ACT_F32)
    hipLaunchKernelGGL(k_resume_state<float>, dim3(M), dim3(256), 0, st, x_in, s1_in, rows, H, x, s, (float*)sb);
  else
    hipLaunchKernelGGL(k_resume_state<bf16_t>, dim3(M), dim3(256), 0, st, x_in, s1_in, rows, H, x, s, (bf16_t*)sb);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* s, const int32_t* rows, int M, int H, float* y, hipStream_t st) {
  const size_t n = (size_t)M * H;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_scatter_rows, dim3(blocks), dim3(256), 0, st, s, rows, H, n, y);
  return hipGetLastError();
}

hipError_t launch_update(const UpdateArgs& u, hipStream_t st) {
  if (u.M == 0) return hipSuccess;
  const bool few = u.M < 512;
  const bool vec = !few && u.y_bf16 && u.splits == 1 && u.H % 8 == 0 && u.H <= 8 * 1024;
  if (u.state_act && (!vec || u.act != ACT_BF16 || !u.sb || !u.s16)) return hipErrorInvalidValue;
  if (u.state_act && u.H % 512 == 0 && u.H / 512 <= 8) {
    const dim3 grid((u.M + 3) / 4);
    switch (u.H / 512) {
      case 1: hipLaunchKernelGGL(k_update_wave<1>, grid, dim3(256), 0, st, u); break;
      case 2: hipLaunchKernelGGL(k_update_wave<2>, grid, dim3(256), 0, st, u); break;
      case 3: hipLaunchKernelGGL(k_update_wave<3>, grid, dim3(256), 0, st, u); break;
      case 4: hipLaunchKernelGGL(k_update_wave<4>, grid, dim3(256), 0, st, u); break;
      case 5: hipLaunchKernelGGL(k_update_wave<5>, grid, dim3(256), 0, st, u); break;
      case 6: hipLaunchKernelGGL(k_update_wave<6>, grid, dim3(256), 0, st, u); break;
      case 7: hipLaunchKernelGGL(k_update_wave<7>, grid, dim3(256), 0, st, u); break;
      default: hipLaunchKernelGGL(k_update_wave<8>, grid, dim3(256), 0, st, u); break;
    }
    return hipGetLastError();
  }
  if (vec) {
    const int per = u.H / 8;  // threads carrying 8 channels each
    if (u.act == ACT_F32) {
      if (per <= 320) hipLaunchKernelGGL((k_update_vec<float, 320>), dim3(u.M), dim3(320), 0, st, u);
      else if (per <= 512) hipLaunchKernelGGL((k_update_vec<float, 512>), dim3(u.M), dim3(512), 0, st, u);
      else hipLaunchKernelGGL((k_update_vec<float, 1024>), dim3(u.M), dim3(1024), 0, st, u);
    } else {
      if (per <= 320) hipLaunchKernelGGL((k_update_vec<bf16_t, 320>), dim3(u.M), dim3(320), 0, st, u);
      else if (per <= 512) hipLaunchKernelGGL((k_update_vec<bf16_t, 512>), dim3(u.M), dim3(512), 0, st, u);
      else hipLaunchKernelGGL((k_update_vec<bf16_t, 1024>), dim3(u.M), dim3(1024), 0, st, u);
    }
    return hipGetLastError();
  }
  if (few && !u.y_bf16 && u.H % 256 == 0 && u.H <= 4096) {
    if (u.act == ACT_F32) hipLaunchKernelGGL(k_update_split4<float>, dim3(u.M), dim3(u.H / 4), 0, st, u);
    else hipLaunchKernelGGL(k_update_split4<bf16_t>, dim3(u.M), dim3(u.H / 4), 0, st, u);
    return hipGetLastError();
  }
  if (u.act == ACT_F32) {
    if (few) hipLaunchKernelGGL((k_update<float, 1024>), dim3(u.M), dim3(1024), 0, st, u);
    else hipLaunchKernelGGL((k_update<float, 512>), dim3(u.M), dim3(512), 0, st, u);
  } else {
    if (few) hipLaunchKernelGGL((k_update<bf16_t, 1024>), dim3(u.M), dim3(1024), 0, st, u);
    else hipLaunchKernelGGL((k_update<bf16_t, 512>), dim3(u.M), dim3(512), 0, st, u);
  }
  return hipGetLastError();
}

hipError_t launch_stage_input(const float* x_in, float* s, void* sb, int M, int H, int act,
                              hipStream_t st, const int32_t* rows, void* s16) {
  const size_t n = (size_t)M * H;
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  if (act == ACT_F32)
    hipLaunchKernelGGL(k_stage_input<float>, dim3(blocks), dim3(256), 0, st, x_in, s, (float*)sb, n, rows, H,
                       (_Float16*)s16);
  else
    hipLaunchKernelGGL(k_stage_input<bf16_t>, dim3(blocks), dim3(256), 0, st, x_in, s, (bf16_t*)sb, n, rows, H,
                       (_Float16*)s16);
  return hipGetLastError();
}

}  // namespace dory
