// kernel_reduce.hpp -- the second pass of split K across workgroups.
//
// C[i][j] = sum over s = 0 .. S-1 of W[s][i][j], added in split order, so the
// result does not depend on which workgroup finished first (run-to-run
// deterministic; no atomics).  W holds S partial M x N tiles with rows of N
// floats (less than 2 GiB in all).  A 64-thread workgroup takes 256
// consecutive columns of one row, a thread four of them: 128-bit loads of W
// when N is a multiple of 4, 128-bit stores when C's rows allow them as well.
// C is written through a resource moved to the workgroup's first element, so
// its offsets stay small whatever C's size.  The pass moves (S + 1) M N 4
// bytes and is bound by HBM.
#pragma once

#include "common.hpp"

namespace sg {

constexpr int kReduceThreads = 64;
constexpr int kReduceCols = 4 * kReduceThreads;  // columns per workgroup

struct ReduceArgs {
  const float* W;
  float* C;
  uint32_t w_bytes;
  int64_t c_bytes;
  int M, N, ldc, splits;
  int chunks;   // workgroups per row: ceil(N / kReduceCols)
};

template <bool VEC_W, bool VEC_C>
__global__ void __launch_bounds__(kReduceThreads) sgemm_split_reduce_kernel(ReduceArgs r) {
  const int row = (int)blockIdx.x / r.chunks;
  const int c0 = ((int)blockIdx.x - row * r.chunks) * kReduceCols;
  const int col = 4 * (int)threadIdx.x;   // from c0
  const int n_left = r.N - c0;
  if (col >= n_left) return;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(r.W, r.w_bytes);
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(r.C, r.c_bytes, (int64_t)row * r.ldc + c0);
  const uint32_t plane = 4u * (uint32_t)r.M * (uint32_t)r.N;   // bytes per split
  const uint32_t woff = ((uint32_t)row * (uint32_t)r.N + (uint32_t)(c0 + col)) * 4u;
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
          v[j][e] = load1(rw, col + e < n_left && off != kOob ? off + 4u * e : kOob);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < r.splits) acc += v[j];
  }
  const uint32_t coff = 4u * (uint32_t)col;
  if constexpr (VEC_C) {
    store4(rc, coff, acc);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < n_left) store1(rc, coff + 4u * e, acc[e]);
  }
}

}  // namespace sg
