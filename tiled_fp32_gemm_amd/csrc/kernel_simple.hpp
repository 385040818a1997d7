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
// with zero fill outside the matrix, through resources moved to each K
// step's corner of A and B; one stage, two barriers per K step.
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
  const int m0 = tm * T, n0 = tn * T;
  const int row = m0 + ty, col = n0 + tx;

  // The tile's corner of A (row m0), B (column n0) and C (m0, n0).
  const float* const At = g.A + (int64_t)m0 * g.lda;
  const uint32_t a_cap =
      cap_bytes((uint64_t)(g.a_bytes - 4 * (int64_t)m0 * g.lda), (uint32_t)kRsrcMax);
  const float* const Bt = g.B + n0;
  const int64_t b_rem = g.b_bytes - 4 * (int64_t)n0;
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(g.C, g.c_bytes, (int64_t)m0 * g.ldc + n0);

  float sum = 0.0f;
  for (int k0 = 0; k0 < g.K; k0 += T) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_slab_a(At, a_cap, k0);
    const __amdgpu_buffer_rsrc_t rb = rsrc_at(Bt, b_rem, (int64_t)k0 * g.ldb);
    const bool a_ok = row < g.M && k0 + tx < g.K;
    const bool b_ok = k0 + ty < g.K && col < g.N;
    As[ty][tx] = load1(ra, a_ok ? ((uint32_t)ty * (uint32_t)g.lda + (uint32_t)tx) * 4u : kOob);
    Bs[ty][tx] = load1(rb, b_ok ? ((uint32_t)ty * (uint32_t)g.ldb + (uint32_t)tx) * 4u : kOob);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < T; ++k) sum = __builtin_fmaf(As[ty][k], Bs[k][tx], sum);
    __syncthreads();
  }
  const bool ok = row < g.M && col < g.N;
  store1(rc, ok ? ((uint32_t)ty * (uint32_t)g.ldc + (uint32_t)tx) * 4u : kOob, sum);
}

}  // namespace sg
