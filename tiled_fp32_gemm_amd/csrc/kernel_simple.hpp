// kernel_simple.hpp -- the basic shared-memory tiled product.
//
// The inner loop the pages start from: a T x T workgroup stages a T x T tile
// of A and of B in shared memory, then each thread accumulates one element of
// C as sum += As[ty][k] * Bs[k][tx] ("CUDA in depth (4): accessing shared
// memory efficiently", section on too many shared-memory reads, with the
// As/Bs declaration of its section on the common tile pitfall).  That costs
// 2 T^3 shared-memory loads per T x T tile and K step and is kept as the
// correctness and ablation baseline for the register-tiled kernels.
//
// With T = 16 and 64-lane waves, a quarter-wave shares ty: its As reads are
// one broadcast word and its Bs reads 16 consecutive words.  Loads are 32-bit
// with zero fill outside the matrix; one stage, two barriers per K step.
#pragma once

#include "common.hpp"

namespace sg {

constexpr int kSimpleT = 16;

__global__ void __launch_bounds__(256) sgemm_simple_kernel(GemmArgs g) {
  constexpr int T = kSimpleT;
  __shared__ float As[T][T];
  __shared__ float Bs[T][T];

  int tm, tn;
  tile_of_workgroup(g, tm, tn);
  const int tx = (int)threadIdx.x & (T - 1), ty = (int)threadIdx.x / T;
  const int row = tm * T + ty, col = tn * T + tx;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.B, g.b_bytes);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.C, g.c_bytes);

  float sum = 0.0f;
  for (int k0 = 0; k0 < g.K; k0 += T) {
    const bool a_ok = row < g.M && k0 + tx < g.K;
    const bool b_ok = k0 + ty < g.K && col < g.N;
    As[ty][tx] = load1(ra, a_ok ? ((uint32_t)row * (uint32_t)g.lda + (uint32_t)(k0 + tx)) * 4u : kOob);
    Bs[ty][tx] = load1(rb, b_ok ? ((uint32_t)(k0 + ty) * (uint32_t)g.ldb + (uint32_t)col) * 4u : kOob);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < T; ++k) sum = __builtin_fmaf(As[ty][k], Bs[k][tx], sum);
    __syncthreads();
  }
  const bool ok = row < g.M && col < g.N;
  store1(rc, ok ? ((uint32_t)row * (uint32_t)g.ldc + (uint32_t)col) * 4u : kOob, sum);
}

}  // namespace sg
