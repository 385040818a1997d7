// kernel_fma.hpp -- FP32 GEMM on the vector ALUs with register tiles.
//
// Register tiling as the pages describe it: each thread keeps a TM x TN block
// of C in registers and, per k, reads TM values of A and TN values of B from
// shared memory once and uses each for TN (resp. TM) multiply-adds, so the
// shared-memory loads per multiply-add fall from 2 (1x1) to (TM + TN) /
// (TM * TN) = 0.25 for 8x8 ("CUDA in depth (4): accessing shared memory
// efficiently", sections on register tiling and on going from 1x1 to 2x2).
//
// gfx950 mapping.  A 256-thread workgroup owns a 128 x 128 tile of C; thread
// (ty, tx) of the 16 x 16 grid owns rows {4ty..4ty+3, 64+4ty..64+4ty+3} and the
// same pattern of columns, so its A and B values for one k come in as four
// 128-bit LDS reads.  Within a wave tx = lane % 16 and ty = 4 * wave + lane / 16:
// a quarter-wave (16 lanes) shares ty, so its A reads are one broadcast word
// group, and its B reads are 256 contiguous bytes: no bank is hit twice.
//
// LDS layouts (gfx950: 64 banks of 4 bytes):
//   As[BK][BM+4]  A transposed on the way in (k-major), so a thread's rows are
//                 contiguous for a given k.  The 4 values of a 128-bit global
//                 load go to 4 different k rows (the pages' split store,
//                 "CUDA in depth (5)", sections on shared-memory transpose and
//                 on vectorised shared-memory stores); with rows of 132 floats
//                 the 64 lanes of each 32-bit store hit 64 distinct banks.
//   Bs[BK][BN+4]  B as in memory, stored with 128-bit writes.
// Staging is the same double-buffered scheme as the matrix-core kernel.
#pragma once

#include "common.hpp"

namespace sg {

struct FmaCfg {
  static constexpr int BM = 128, BN = 128, BK = 16, NT = 256;
  static constexpr int RA = BM + 4, RB = BN + 4;
  static constexpr int A_STAGE = BK * RA, B_STAGE = BK * RB;
  static constexpr int LDS_FLOATS = 2 * (A_STAGE + B_STAGE);
  static constexpr int A_SLOTS = BM * BK / 4 / NT;  // 2
  static constexpr int B_SLOTS = BK * BN / 4 / NT;  // 2
};

// KU: how many k steps of a slab are unrolled together; WPE: the waves per
// SIMD the register allocation must leave room for.  Unrolling all 16 steps
// lets the compiler hoist every LDS read of the slab and needs ~356
// registers (one wave per SIMD); 8 steps with room for two waves per SIMD
// runs 1.7x faster on MI355X (88 against 51 TFLOP/s at 4096^3).
template <bool VEC_A, bool VEC_B, bool VEC_C, int KU = 8, int WPE = 2>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
sgemm_fma_kernel(GemmArgs g) {
  using Cfg = FmaCfg;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
  constexpr int RA = Cfg::RA, RB = Cfg::RB;

  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS_FLOATS];
  float* const As = lds;                      // [2][BK][RA]
  float* const Bs = lds + 2 * Cfg::A_STAGE;   // [2][BK][RB]

  int tm, tn;
  tile_of_workgroup(g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tx = lane & 15, ty = 4 * wave + (lane >> 4);

  // The tile's corner of each operand (A from row m0, B from column n0, C
  // from (m0, n0)); each slab moves A and B on to its own first column and
  // row, so lane offsets are counted from the slab's corner.
  const float* const At = g.A + (int64_t)m0 * g.lda;
  const uint32_t a_cap =
      cap_bytes((uint64_t)(g.a_bytes - 4 * (int64_t)m0 * g.lda), (uint32_t)kRsrcMax);
  const float* const Bt = g.B + n0;
  const int64_t b_rem = g.b_bytes - 4 * (int64_t)n0;
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(g.C, g.c_bytes, (int64_t)m0 * g.ldc + n0);

  // A slot: row (f % 16) + 16 (f / 64), k group (f / 16) % 4, f = s NT + tid.
  uint32_t a_off[Cfg::A_SLOTS];
  bool a_row_ok[Cfg::A_SLOTS];
  int a_k[Cfg::A_SLOTS], a_row[Cfg::A_SLOTS];
#pragma unroll
  for (int s = 0; s < Cfg::A_SLOTS; ++s) {
    const int f = s * NT + tid;
    const int row = (f & 15) + ((f >> 6) << 4), kq = (f >> 4) & 3;
    a_row[s] = row;
    a_k[s] = 4 * kq;
    a_row_ok[s] = row < g.M - m0;
    a_off[s] = ((uint32_t)row * (uint32_t)g.lda + 4u * kq) * 4u;
  }
  uint32_t b_off[Cfg::B_SLOTS];
  int b_k[Cfg::B_SLOTS], b_j[Cfg::B_SLOTS], b_lds[Cfg::B_SLOTS];
#pragma unroll
  for (int s = 0; s < Cfg::B_SLOTS; ++s) {
    const int f = s * NT + tid;
    const int k = f / (BN / 4), jq = f % (BN / 4);
    b_k[s] = k;
    b_j[s] = n0 + 4 * jq;
    b_off[s] = ((uint32_t)k * (uint32_t)g.ldb + (uint32_t)(4 * jq)) * 4u;
    b_lds[s] = k * RB + 4 * jq;
  }

  f32x4 sa[Cfg::A_SLOTS], sb[Cfg::B_SLOTS];
  auto load_slab = [&](int k0) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_slab_a(At, a_cap, k0);
    const __amdgpu_buffer_rsrc_t rb = rsrc_at(Bt, b_rem, (int64_t)k0 * g.ldb);
#pragma unroll
    for (int s = 0; s < Cfg::A_SLOTS; ++s) {
      const int k = k0 + a_k[s];
      const uint32_t base = a_off[s];
      if constexpr (VEC_A) {
        sa[s] = load4(ra, (a_row_ok[s] && k < g.K) ? base : kOob);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sa[s][e] = load1(ra, (a_row_ok[s] && k + e < g.K) ? base + 4u * e : kOob);
      }
    }
#pragma unroll
    for (int s = 0; s < Cfg::B_SLOTS; ++s) {
      const bool k_ok = (k0 + b_k[s]) < g.K;
      const uint32_t base = b_off[s];
      if constexpr (VEC_B) {
        sb[s] = load4(rb, (k_ok && b_j[s] < g.N) ? base : kOob);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sb[s][e] = load1(rb, (k_ok && b_j[s] + e < g.N) ? base + 4u * e : kOob);
      }
    }
  };
  auto store_slab = [&](int st) {
    float* as = As + st * Cfg::A_STAGE;
    float* bs = Bs + st * Cfg::B_STAGE;
#pragma unroll
    for (int s = 0; s < Cfg::A_SLOTS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) as[(a_k[s] + e) * RA + a_row[s]] = sa[s][e];
#pragma unroll
    for (int s = 0; s < Cfg::B_SLOTS; ++s)
      *reinterpret_cast<f32x4*>(bs + b_lds[s]) = sb[s];
  };

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

  const int nslab = (g.K + BK - 1) / BK;
  if (nslab > 0) {
    load_slab(0);
    store_slab(0);
  }
  __syncthreads();

  for (int t = 0; t < nslab; ++t) {
    const int cur = t & 1;
    const bool more = (t + 1) < nslab;
    if (more) load_slab((t + 1) * BK);
    const float* as = As + cur * Cfg::A_STAGE;
    const float* bs = Bs + cur * Cfg::B_STAGE;
#pragma unroll KU
    for (int k = 0; k < BK; ++k) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(as + k * RA + 4 * ty);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(as + k * RA + 64 + 4 * ty);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(bs + k * RB + 4 * tx);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(bs + k * RB + 64 + 4 * tx);
      const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    if (more) store_slab(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: row 4ty + i (+64) and columns 4tx..4tx+3 (+64) from the
  // tile's corner; a quarter-wave writes 256 contiguous bytes of one row.
  const int m_left = g.M - m0, n_left = g.N - n0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4;
    const bool row_ok = row < m_left;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = 64 * h + 4 * tx;
      const uint32_t off = ((uint32_t)row * (uint32_t)g.ldc + (uint32_t)col) * 4u;
      if constexpr (VEC_C) {
        const f32x4 v = {acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2],
                         acc[i][4 * h + 3]};
        store4(rc, (row_ok && col < n_left) ? off : kOob, v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          store1(rc, (row_ok && col + e < n_left) ? off + 4u * e : kOob,
                 acc[i][4 * h + e]);
      }
    }
  }
}

}  // namespace sg
