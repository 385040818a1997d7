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
// gfx950 mapping: a 256-thread workgroup moves a tile of 64 input rows by
// 128 input columns, 8192 floats, as 16-byte groups, with every LDS access
// 128 bits wide.
//   * Load: thread f (eight rounds of 256) reads the 16-byte group (r, c) =
//     (f / 32, f % 32) of the input tile (32 lanes cover one 512-byte row
//     segment) and stores it as LDS unit (r, c).
//   * Store: thread b (two rounds of 256) takes the 4 x 4 block (i, c) =
//     (b % 16, b / 16): it reads units (4 i + e, c), e = 0..3, transposes the
//     block in registers and writes four 16-byte groups to output rows
//     4 c + e' (16 lanes cover one 256-byte output row segment).
// The tile is twice as wide as it is tall so that input rows are read in
// 512-byte runs: with buffers rotated past the 256 MiB last-level cache this
// moved 8192^2 from 4.1 to 5.0 TB/s and 16384^2 from 4.6 to 5.1 TB/s on
// MI355X, where a plain device copy reaches 4.7-5.3 TB/s.
// Elements outside the matrix read as 0 and are not stored (buffer range
// checks); each tile reads and writes through resources moved to its own
// corner, so offsets stay below 2^31 whatever the size of the matrices.  The unit layout is a template parameter, because it is the
// experiment.  A 128-bit access is served 16 lanes at a time, and the 16
// lanes of a read share c and e and differ in i:
//
//   kNaive     unit(r, c) = 32 r + c: the 16 reads land in one 16-byte bank
//              group -- 16-way conflicts (the pages' unpadded [32][32]
//              control, scaled to gfx950 and 128-bit accesses).
//   kPadded    unit(r, c) = 33 r + c: one extra 16-byte unit per row, the
//              pages' extra column at the width of the access.  The groups
//              become (4 i + e + c) mod 16: only 4 distinct, so 4-way
//              conflicts remain -- padding by one unit is not enough for
//              128-bit column reads.
//   kSwizzled  unit(r, c) = 32 r + (c ^ (r / 4)): the XOR permutation puts
//              the 16 reads in 16 distinct groups and keeps every row a
//              permutation of its own units, so both the stores and the
//              reads are conflict-free.
#pragma once

#include "common.hpp"

namespace sg {

enum TransposeLayout { kNaive = 1, kPadded = 2, kSwizzled = 3 };

constexpr int kTransposeRows = 64;    // input rows per tile
constexpr int kTransposeCols = 128;   // input columns per tile

struct TransposeArgs {
  const float* in;
  float* out;
  int64_t in_bytes, out_bytes;   // bytes each matrix spans
  int rows, cols;     // of the input
  int ldi, ldo;       // leading dimensions of input and output
  int tiles_x;        // tiles across the input's columns
};

template <int LAYOUT>
struct TileLayout {
  static constexpr int UNITS = kTransposeCols / 4;  // 16-byte units per tile row
  static constexpr int UNITS_PER_ROW = LAYOUT == kPadded ? UNITS + 1 : UNITS;
  static constexpr int FLOATS = kTransposeRows * UNITS_PER_ROW * 4;
  // Float index of 16-byte unit (r, c) of the tile.
  __device__ static __forceinline__ int at(int r, int c) {
    if constexpr (LAYOUT == kSwizzled)
      return 4 * (UNITS * r + (c ^ (r >> 2)));
    else
      return 4 * (UNITS_PER_ROW * r + c);
  }
};

template <int LAYOUT, bool VEC_IN, bool VEC_OUT>
__global__ void __launch_bounds__(256) sgemm_transpose_kernel(TransposeArgs a) {
  using L = TileLayout<LAYOUT>;
  constexpr int UNITS = L::UNITS;
  constexpr int LOADS = kTransposeRows * UNITS / 256;            // 8
  constexpr int BLOCKS = kTransposeRows * kTransposeCols / 16 / 256;  // 2
  static_assert(kTransposeRows / 4 == 16, "a 16-lane phase spans one block column");
  __shared__ __attribute__((aligned(16))) float tile[L::FLOATS];

  const int tx = (int)blockIdx.x % a.tiles_x, ty = (int)blockIdx.x / a.tiles_x;
  const int x0 = tx * kTransposeCols, y0 = ty * kTransposeRows;  // input column, row
  const int tid = (int)threadIdx.x;
  // Resources from the tile's corner of the input (row y0, column x0) and
  // of the output (row x0, column y0); offsets below are counted from there.
  const __amdgpu_buffer_rsrc_t rin = rsrc_at(a.in, a.in_bytes, (int64_t)y0 * a.ldi + x0);
  const __amdgpu_buffer_rsrc_t rout = rsrc_at(a.out, a.out_bytes, (int64_t)x0 * a.ldo + y0);

  f32x4 v[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int f = q * 256 + tid;
    const int r = f / UNITS, c = f % UNITS;
    const int gr = y0 + r, gc = x0 + 4 * c;
    const uint32_t off = ((uint32_t)r * (uint32_t)a.ldi + (uint32_t)(4 * c)) * 4u;
    if constexpr (VEC_IN) {
      v[q] = load4(rin, (gr < a.rows && gc < a.cols) ? off : kOob);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[q][e] = load1(rin, (gr < a.rows && gc + e < a.cols) ? off + 4u * e : kOob);
    }
  }
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int f = q * 256 + tid;
    *reinterpret_cast<f32x4*>(&tile[L::at(f / UNITS, f % UNITS)]) = v[q];
  }
  __syncthreads();  // every thread reaches it, edge tiles included

#pragma unroll
  for (int bq = 0; bq < BLOCKS; ++bq) {
    const int b = bq * 256 + tid;
    const int i = b & 15, c = b >> 4;
    f32x4 blk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      blk[e] = *reinterpret_cast<const f32x4*>(&tile[L::at(4 * i + e, c)]);
    const int ocol = y0 + 4 * i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // output row x0 + 4 c + e
      const int orow = x0 + 4 * c + e;
      const f32x4 o = {blk[0][e], blk[1][e], blk[2][e], blk[3][e]};
      const uint32_t off = ((uint32_t)(4 * c + e) * (uint32_t)a.ldo + (uint32_t)(4 * i)) * 4u;
      if constexpr (VEC_OUT) {
        store4(rout, (orow < a.cols && ocol < a.rows) ? off : kOob, o);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          store1(rout, (orow < a.cols && ocol + w < a.rows) ? off + 4u * w : kOob, o[w]);
      }
    }
  }
}

}  // namespace sg
