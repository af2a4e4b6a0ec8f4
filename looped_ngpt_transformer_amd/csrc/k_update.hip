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
  const bool need_x = u.bnd == BND_LOOP_CONTINUE;
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
  if (u.bnd == BND_LOOP_CONTINUE || u.bnd == BND_LOOP_FINAL) {  // s_t = N(F(u_t))
    const float n2 = inv_norm(norm_sp * norm_sp);
    scale *= n2;
    norm_sp *= n2;
  }
  if (u.bnd == BND_LOOP_CONTINUE) {  // u = N(s_t + x)
    const float dot = (tot[4] + tot[5] * ny) * scale;  // s_t . x
    const float n3 = inv_norm(norm_sp * norm_sp + 2.f * dot + tot[6]);
    scale *= n3;
    add_x = n3;
  } else if (u.bnd == BND_SAVE_X) {  // x = s'; u = N(s' + s')
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

template <typename SB>
__global__ __launch_bounds__(256) void k_stage_input(const float* x, float* s, SB* sb, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const float v = x[i];
    s[i] = v;
    st<SB>(sb, i, v);
  }
}

hipError_t launch_update(const UpdateArgs& u, hipStream_t st) {
  if (u.M == 0) return hipSuccess;
  const bool few = u.M < 512;
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
                              hipStream_t st) {
  const size_t n = (size_t)M * H;
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  if (act == ACT_F32)
    hipLaunchKernelGGL(k_stage_input<float>, dim3(blocks), dim3(256), 0, st, x_in, s, (float*)sb, n);
  else
    hipLaunchKernelGGL(k_stage_input<bf16_t>, dim3(blocks), dim3(256), 0, st, x_in, s, (bf16_t*)sb, n);
  return hipGetLastError();
}

}  // namespace dory
