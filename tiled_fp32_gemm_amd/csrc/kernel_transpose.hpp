// kernel_transpose.hpp -- out = in^T for row-major FP32, staged through LDS.
//
// The pages' one complete kernel is a tiled transpose: a workgroup reads a
// square tile with coalesced row reads, parks it in shared memory, and
// writes it out with coalesced row writes of the transposed tile, so that
// the column access happens in shared memory, where the layout decides
// whether it collides in the banks ("Memory-bank mechanism and accelerated
// compute", section on the transpose kernel, and section on alternatives to
// padding).
//
// gfx950 mapping: a 256-thread workgroup moves a 64 x 64 tile as 16 x 16
// blocks of 4 x 4 floats, with every LDS access 128 bits wide.
//   * Load: thread f (four rounds of 256) reads the 16-byte group (r, c) =
//     (f / 16, f % 16) of the input tile (16 lanes cover one 256-byte row
//     segment) and stores it as LDS unit (r, c).
//   * Store: thread b takes block (i, c) = (b % 16, b / 16): it reads units
//     (4 i + e, c), e = 0..3, transposes the 4 x 4 block in registers and
//     writes four 16-byte groups to output rows 4 c + e' (16 lanes cover one
//     256-byte output row segment).
// Elements outside the matrix read as 0 and are not stored (buffer range
// checks).  The unit layout is a template parameter, because it is the
// experiment.  A 128-bit access is served 16 lanes at a time, and the 16
// lanes of a read share c and e and differ in i:
//
//   kNaive     unit(r, c) = 16 r + c: the 16 reads land in one 16-byte bank
//              group -- 16-way conflicts (the pages' unpadded [32][32]
//              control, scaled to gfx950 and 128-bit accesses).
//   kPadded    unit(r, c) = 17 r + c: one extra 16-byte unit per row, the
//              pages' extra column at the width of the access.  The groups
//              become (4 i + e + c) mod 16: only 4 distinct, so 4-way
//              conflicts remain -- padding by one unit is not enough for
//              128-bit column reads.
//   kSwizzled  unit(r, c) = 16 r + (c ^ ((r / 4) mod 16)): the XOR
//              permutation puts the 16 reads in 16 distinct groups and keeps
//              every row a permutation of its own units, so both the stores
//              and the reads are conflict-free.
#pragma once

#include "common.hpp"

namespace sg {

enum TransposeLayout { kNaive = 1, kPadded = 2, kSwizzled = 3 };

struct TransposeArgs {
  const float* in;
  float* out;
  uint32_t in_bytes, out_bytes;
  int rows, cols;     // of the input
  int ldi, ldo;       // leading dimensions of input and output
  int tiles_x;        // 64-wide tiles across the input's columns
};

template <int LAYOUT>
struct TileLayout {
  static constexpr int UNITS_PER_ROW = LAYOUT == kPadded ? 17 : 16;
  static constexpr int FLOATS = 64 * UNITS_PER_ROW * 4;
  // Float index of 16-byte unit (r, c) of the tile.
  __device__ static __forceinline__ int at(int r, int c) {
    if constexpr (LAYOUT == kSwizzled)
      return 4 * (16 * r + (c ^ ((r >> 2) & 15)));
    else
      return 4 * (UNITS_PER_ROW * r + c);
  }
};

template <int LAYOUT, bool VEC_IN, bool VEC_OUT>
__global__ void __launch_bounds__(256) sgemm_transpose_kernel(TransposeArgs a) {
  using L = TileLayout<LAYOUT>;
  __shared__ __attribute__((aligned(16))) float tile[L::FLOATS];

  const int tx = (int)blockIdx.x % a.tiles_x, ty = (int)blockIdx.x / a.tiles_x;
  const int x0 = tx * 64, y0 = ty * 64;   // input column and row of the tile
  const int tid = (int)threadIdx.x;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(a.in, a.in_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(a.out, a.out_bytes);

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = q * 256 + tid;
    const int r = f >> 4, c = f & 15;
    const int gr = y0 + r, gc = x0 + 4 * c;
    const uint32_t off = ((uint32_t)gr * (uint32_t)a.ldi + (uint32_t)gc) * 4u;
    f32x4 v;
    if constexpr (VEC_IN) {
      v = load4(rin, (gr < a.rows && gc < a.cols) ? off : kOob);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = load1(rin, (gr < a.rows && gc + e < a.cols) ? off + 4u * e : kOob);
    }
    *reinterpret_cast<f32x4*>(&tile[L::at(r, c)]) = v;
  }
  __syncthreads();  // every thread reaches it, edge tiles included

  const int i = tid & 15, c = tid >> 4;
  f32x4 blk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    blk[e] = *reinterpret_cast<const f32x4*>(&tile[L::at(4 * i + e, c)]);
  const int ocol = y0 + 4 * i;
#pragma unroll
  for (int e = 0; e < 4; ++e) {   // output row x0 + 4 c + e
    const int orow = x0 + 4 * c + e;
    const f32x4 v = {blk[0][e], blk[1][e], blk[2][e], blk[3][e]};
    const uint32_t off = ((uint32_t)orow * (uint32_t)a.ldo + (uint32_t)ocol) * 4u;
    if constexpr (VEC_OUT) {
      store4(rout, (orow < a.cols && ocol < a.rows) ? off : kOob, v);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        store1(rout, (orow < a.cols && ocol + w < a.rows) ? off + 4u * w : kOob, v[w]);
    }
  }
}

}  // namespace sg
