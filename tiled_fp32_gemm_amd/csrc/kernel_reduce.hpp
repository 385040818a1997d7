// kernel_reduce.hpp -- the second pass of split K across workgroups.
//
// C[i][j] = sum over s = 0 .. S-1 of W[s][i][j], added in split order, so the
// result does not depend on which workgroup finished first (run-to-run
// deterministic; no atomics).  W holds S partial M x N tiles with rows of N
// floats.  One thread takes four consecutive elements of a row: 128-bit loads
// of W when N is a multiple of 4, 128-bit stores when C's rows allow them as
// well.  The pass moves (S + 1) M N 4 bytes and is bound by HBM.
#pragma once

#include "common.hpp"

namespace sg {

struct ReduceArgs {
  const float* W;
  float* C;
  uint32_t w_bytes, c_bytes;
  int M, N, ldc, splits;
  int groups_per_row;   // ceil(N / 4)
};

template <bool VEC_W, bool VEC_C>
__global__ void __launch_bounds__(256) sgemm_split_reduce_kernel(ReduceArgs r) {
  const int f = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int row = f / r.groups_per_row;
  if (row >= r.M) return;
  const int col = 4 * (f - row * r.groups_per_row);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(r.W, r.w_bytes);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(r.C, r.c_bytes);
  const uint32_t plane = 4u * (uint32_t)r.M * (uint32_t)r.N;   // bytes per split
  const uint32_t woff = ((uint32_t)row * (uint32_t)r.N + (uint32_t)col) * 4u;
  // Eight splits' loads are in flight at once; they are added one by one.
  constexpr int kBatch = 8;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < r.splits; s0 += kBatch) {
    f32x4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint32_t off = s0 + j < r.splits ? woff + (uint32_t)(s0 + j) * plane : kOob;
      if constexpr (VEC_W) {
        v[j] = load4(rw, off);   // N % 4 == 0: the group lies inside the row
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[j][e] = load1(rw, col + e < r.N && off != kOob ? off + 4u * e : kOob);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < r.splits) acc += v[j];
  }
  const uint32_t coff = ((uint32_t)row * (uint32_t)r.ldc + (uint32_t)col) * 4u;
  if constexpr (VEC_C) {
    store4(rc, coff, acc);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < r.N) store1(rc, coff + 4u * e, acc[e]);
  }
}

}  // namespace sg
