// Fused nGPT residual update and loop boundary (one work-group per row).
//
// s <- N((1 - a) * s + a * N(y))  — the nGPT update ("Dory1.0-4B" paper summary,
// nGPT prerequisite; arXiv summary §2: normalised sublayer output blended with the
// normalised residual by per-channel rates, then normalised). y arrives as split-K
// partial sums. The L2 norm the pages put before the output and down projections (arXiv
// §2) scales y's row by a positive factor, which N(y) removes, so it needs no work.
// Loop boundaries (paper summary, core-method equation): at the end of the input block
// x is saved and u_1 = N(x + x); at the end of loop t, s_t = N(.) and, unless t = k,
// u_{t+1} = N(s_t + x).
//
// All of the row's loads (partials, state, rates, x) are issued first; the 2560-wide
// reductions are wave shuffles plus one LDS exchange, the row stays in registers.
#include "common.h"
#include "kernels.h"

namespace dory {

// THREADS per row: 256 for many rows, 1024 for few rows (decode) so that each row's
// loads are spread over more waves.
template <typename SB, int UPD_THREADS>
__global__ __launch_bounds__(UPD_THREADS) void k_update(UpdateArgs u) {
  constexpr int UPD_MAXPER = 4096 / UPD_THREADS;  // H <= 4096
  __shared__ float red[UPD_THREADS / WAVE];
  const int m = blockIdx.x;
  const int H = u.H;
  const size_t row = (size_t)m * H;
  const bool need_x = u.bnd == BND_LOOP_CONTINUE;
  float v[UPD_MAXPER], sv[UPD_MAXPER], av[UPD_MAXPER], xv[UPD_MAXPER];
  float sq = 0.f;
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) {
    const int i = threadIdx.x + k * UPD_THREADS;
    float y = 0.f;
    sv[k] = av[k] = xv[k] = 0.f;
    if (i < H) {
      for (int s = 0; s < u.splits; ++s) y += u.y[(size_t)s * u.M * H + row + i];
      sv[k] = u.s[row + i];
      av[k] = u.alpha[i];
      if (need_x) xv[k] = u.x[row + i];
    }
    v[k] = y;
    sq += y * y;
  }
  const float ny = inv_norm(block_sum<UPD_THREADS / WAVE>(sq, red));
  sq = 0.f;
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) {
    const float t = (1.f - av[k]) * sv[k] + av[k] * (v[k] * ny);  // zero beyond H
    v[k] = t;
    sq += t * t;
  }
  float n = inv_norm(block_sum<UPD_THREADS / WAVE>(sq, red));
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) v[k] *= n;

  if (u.bnd == BND_LOOP_CONTINUE || u.bnd == BND_LOOP_FINAL) {  // s_t = N(F(u_t))
    sq = 0.f;
#pragma unroll
    for (int k = 0; k < UPD_MAXPER; ++k) sq += v[k] * v[k];
    n = inv_norm(block_sum<UPD_THREADS / WAVE>(sq, red));
#pragma unroll
    for (int k = 0; k < UPD_MAXPER; ++k) v[k] *= n;
  }
  if (u.bnd == BND_SAVE_X || u.bnd == BND_LOOP_CONTINUE) {  // u = N(s + x)
    sq = 0.f;
#pragma unroll
    for (int k = 0; k < UPD_MAXPER; ++k) {
      const int i = threadIdx.x + k * UPD_THREADS;
      if (i < H) {
        float x;
        if (u.bnd == BND_SAVE_X) {
          x = v[k];
          u.x[row + i] = x;
        } else {
          x = xv[k];
        }
        v[k] += x;
        sq += v[k] * v[k];
      }
    }
    n = inv_norm(block_sum<UPD_THREADS / WAVE>(sq, red));
#pragma unroll
    for (int k = 0; k < UPD_MAXPER; ++k) v[k] *= n;
  }
  SB* sb = (SB*)u.sb;
#pragma unroll
  for (int k = 0; k < UPD_MAXPER; ++k) {
    const int i = threadIdx.x + k * UPD_THREADS;
    if (i < H) {
      u.s_out[row + i] = v[k];
      if (sb) st<SB>(sb, row + i, v[k]);
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
    else hipLaunchKernelGGL((k_update<float, 256>), dim3(u.M), dim3(256), 0, st, u);
  } else {
    if (few) hipLaunchKernelGGL((k_update<bf16_t, 1024>), dim3(u.M), dim3(1024), 0, st, u);
    else hipLaunchKernelGGL((k_update<bf16_t, 256>), dim3(u.M), dim3(256), 0, st, u);
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
