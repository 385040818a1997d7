// kernel_ladder.hpp -- the pages' optimisation steps as kernels of their own,
// for the ablation ladder: each step changes one thing against the one
// before, so that its effect on time and on LDS bank conflicts can be
// measured in isolation.
//
//   sgemm_naive_kernel   no shared memory: each thread reads a row of A and
//                        a column of B from global memory for its one output
//                        (the starting point that tiling improves on, "CUDA
//                        in depth (4): accessing shared memory efficiently",
//                        opening recap of the global-memory tiling parts).
//   sgemm_ladder_kernel<TM, TN, AL, BL, VEC>
//                        a 256-thread workgroup (16 x 16 threads) computes a
//                        16 TM x 16 TN tile of C, each thread a TM x TN
//                        register tile ("CUDA in depth (4)", sections on
//                        register tiling and on going from 1x1 to 2x2: per k a
//                        thread reads TM values of A and TN of B and does
//                        TM TN multiply-adds).  K is walked in 16-deep slabs
//                        through one LDS stage (load, barrier, compute,
//                        barrier).  The options:
//     VEC  128-bit global loads of 4-float groups instead of four 32-bit
//          ones ("CUDA in depth (5): vectorized load and shared-memory
//          layout", sections on scalar-load waste and on vector loads);
//     AL   the layout of A, stored k-major (transposed on the way in, the
//          same page's shared-memory transpose, so that a thread's rows are
//          contiguous for one k): kAUnpadded As[16][BM]; kAPadded
//          As[16][BM + 4] (the pages' extra column at the width of a 16-byte
//          group); kASwizzled As[16][BM] with the row index XORed by
//          16 ((k / 4) mod 4) ("Memory-bank mechanism and accelerated
//          compute", section on alternatives to padding);
//     BL   the layout of B: kBRows Bs[16][BN + 4], rows as in memory, which
//          the compute loop reads as contiguous groups; or B transposed on
//          the way in, Bs[BN][16] (kBCols) or Bs[BN][17] (kBColsPadded), the
//          two shapes of the pages' B-tile example ("CUDA in depth (5)",
//          section on the B-tile example), which this compute loop reads
//          down a column.
// The last FMA step of the ladder, double buffering, is the product FMA
// kernel itself (kernel_fma.hpp).
//
// On 64 banks of 4 bytes (a 128-bit access served 16 lanes at a time), for
// the 8 x 8 tile: a 32-bit store of A's k-major split store puts its 64
// lanes on 16 rows x 4 k rows; unpadded, lanes four k rows apart share a bank
// (4-way); padded by 4 floats or XOR-swizzled they hit 64 distinct banks.
// Reading B transposed without padding, the 16 threads of a quarter-wave
// read column 4 tx + j at one k, 64 floats apart: one bank (16-way); with a
// 17-float pitch they are spread.
#pragma once

#include "common.hpp"

namespace sg {

__global__ void __launch_bounds__(256) sgemm_naive_kernel(GemmArgs g) {
  int tm, tn;
  tile_of_workgroup(g, tm, tn);
  const int tx = (int)threadIdx.x & 15, ty = (int)threadIdx.x >> 4;
  const int m0 = tm * 16, n0 = tn * 16;
  const int row = m0 + ty, col = n0 + tx;
  // The tile's corner of A (row m0), B (column n0) and C (m0, n0); A and B
  // move on by 16 values of k at a time.
  const float* const At = g.A + (int64_t)m0 * g.lda;
  const uint32_t a_cap =
      cap_bytes((uint64_t)(g.a_bytes - 4 * (int64_t)m0 * g.lda), (uint32_t)kRsrcMax);
  const float* const Bt = g.B + n0;
  const int64_t b_rem = g.b_bytes - 4 * (int64_t)n0;
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(g.C, g.c_bytes, (int64_t)m0 * g.ldc + n0);
  const bool row_ok = row < g.M, col_ok = col < g.N;
  float sum = 0.0f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_slab_a(At, a_cap, k0);
    const __amdgpu_buffer_rsrc_t rb = rsrc_at(Bt, b_rem, (int64_t)k0 * g.ldb);
    const int kn = min(16, g.K - k0);
    for (int k = 0; k < kn; ++k) {
      const float a = load1(ra, row_ok ? ((uint32_t)ty * (uint32_t)g.lda + (uint32_t)k) * 4u : kOob);
      const float b = load1(rb, col_ok ? ((uint32_t)k * (uint32_t)g.ldb + (uint32_t)tx) * 4u : kOob);
      sum = __builtin_fmaf(a, b, sum);
    }
  }
  store1(rc, (row_ok && col_ok) ? ((uint32_t)ty * (uint32_t)g.ldc + (uint32_t)tx) * 4u : kOob, sum);
}

enum LadderALayout { kAUnpadded = 0, kAPadded = 1, kASwizzled = 2 };
enum LadderBLayout { kBRows = 0, kBCols = 1, kBColsPadded = 2 };

template <int TM, int TN, int AL, int BL>
struct LadderCfg {
  static constexpr int BM = 16 * TM, BN = 16 * TN, BK = 16, NT = 256;
  static constexpr int RA = AL == kAPadded ? BM + 4 : BM;       // A row pitch
  static constexpr int RB = BL == kBRows ? BN + 4 : (BL == kBCols ? BK : BK + 1);
  static constexpr int A_FLOATS = BK * RA;
  static constexpr int B_FLOATS = BL == kBRows ? BK * RB : BN * RB;
  static constexpr int A_GROUPS = BM * BK / 4, B_GROUPS = BK * BN / 4;  // 4-float groups
  static constexpr int A_SLOTS = (A_GROUPS + NT - 1) / NT;
  static constexpr int B_SLOTS = (B_GROUPS + NT - 1) / NT;
  // A thread's rows come in groups of RG consecutive rows, 16 RG apart
  // (8 x 8: rows 4 ty + 0..3 and 64 + 4 ty + 0..3), and its columns alike.
  static constexpr int RG = TM < 4 ? TM : 4, NGM = TM / RG;
  static constexpr int CG = TN < 4 ? TN : 4, NGN = TN / CG;
  static_assert(TM == 1 || TM == 2 || TM == 4 || TM == 8, "register tile rows");
  static_assert(TN == 1 || TN == 2 || TN == 4 || TN == 8, "register tile columns");
  static_assert(AL != kASwizzled || BM % 64 == 0, "the swizzle flips row bits 4-5");
};

template <int N>
struct FloatVec;
template <> struct FloatVec<1> { typedef float type; };
template <> struct FloatVec<2> { typedef float type __attribute__((ext_vector_type(2))); };
template <> struct FloatVec<4> { typedef f32x4 type; };

template <int TM, int TN, int AL, int BL, bool VEC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
sgemm_ladder_kernel(GemmArgs g) {
  using Cfg = LadderCfg<TM, TN, AL, BL>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
  constexpr int RA = Cfg::RA, RB = Cfg::RB, RG = Cfg::RG, CG = Cfg::CG;
  using AVec = typename FloatVec<RG>::type;
  using BVec = typename FloatVec<CG>::type;

  __shared__ __attribute__((aligned(16))) float As[Cfg::A_FLOATS];
  __shared__ __attribute__((aligned(16))) float Bs[Cfg::B_FLOATS];

  int tm, tn;
  tile_of_workgroup(g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tx = lane & 15, ty = 4 * wave + (lane >> 4);

  // The tile's corner of A (row m0), B (column n0) and C (m0, n0); each
  // slab moves A and B on to its own first column and row.
  const float* const At = g.A + (int64_t)m0 * g.lda;
  const uint32_t a_cap =
      cap_bytes((uint64_t)(g.a_bytes - 4 * (int64_t)m0 * g.lda), (uint32_t)kRsrcMax);
  const float* const Bt = g.B + n0;
  const int64_t b_rem = g.b_bytes - 4 * (int64_t)n0;
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(g.C, g.c_bytes, (int64_t)m0 * g.ldc + n0);

  // Column of As that holds tile row r at slab depth k.
  auto a_col = [](int r, int k) {
    if constexpr (AL == kASwizzled) return r ^ (16 * ((k >> 2) & 3));
    else return r;
  };

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < g.K; k0 += BK) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_slab_a(At, a_cap, k0);
    const __amdgpu_buffer_rsrc_t rb = rsrc_at(Bt, b_rem, (int64_t)k0 * g.ldb);
    // A group f: tile row (f % 16) + 16 (f / 64), k quad (f / 16) % 4.
#pragma unroll
    for (int s = 0; s < Cfg::A_SLOTS; ++s) {
      const int f = s * NT + tid;
      if (f < Cfg::A_GROUPS) {
        const int row = (f & 15) + ((f >> 6) << 4), kq = (f >> 4) & 3;
        const int gr = m0 + row, gk = k0 + 4 * kq;
        const uint32_t off = ((uint32_t)row * (uint32_t)g.lda + (uint32_t)(4 * kq)) * 4u;
        f32x4 v;
        if constexpr (VEC) {
          v = load4(ra, (gr < g.M && gk < g.K) ? off : kOob);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = load1(ra, (gr < g.M && gk + e < g.K) ? off + 4u * e : kOob);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) As[(4 * kq + e) * RA + a_col(row, 4 * kq + e)] = v[e];
      }
    }
    // B group f: slab row f / (BN / 4), columns 4 (f % (BN / 4)) + 0..3.
#pragma unroll
    for (int s = 0; s < Cfg::B_SLOTS; ++s) {
      const int f = s * NT + tid;
      if (f < Cfg::B_GROUPS) {
        const int k = f / (BN / 4), jq = f % (BN / 4);
        const int gk = k0 + k, gc = n0 + 4 * jq;
        const uint32_t off = ((uint32_t)k * (uint32_t)g.ldb + (uint32_t)(4 * jq)) * 4u;
        f32x4 v;
        if constexpr (VEC) {
          v = load4(rb, (gk < g.K && gc < g.N) ? off : kOob);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = load1(rb, (gk < g.K && gc + e < g.N) ? off + 4u * e : kOob);
        }
        if constexpr (BL == kBRows) {
          *reinterpret_cast<f32x4*>(&Bs[k * RB + 4 * jq]) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) Bs[(4 * jq + e) * RB + k] = v[e];
        }
      }
    }
    __syncthreads();

#pragma unroll 8
    for (int k = 0; k < BK; ++k) {
      float a[TM], b[TN];
#pragma unroll
      for (int gi = 0; gi < Cfg::NGM; ++gi) {
        const int r = gi * 16 * RG + RG * ty;
        const AVec v = *reinterpret_cast<const AVec*>(&As[k * RA + a_col(r, k)]);
        if constexpr (RG == 1) {
          a[gi] = v;
        } else {
#pragma unroll
          for (int e = 0; e < RG; ++e) a[gi * RG + e] = v[e];
        }
      }
#pragma unroll
      for (int gj = 0; gj < Cfg::NGN; ++gj) {
        const int c = gj * 16 * CG + CG * tx;
        if constexpr (BL == kBRows) {
          const BVec v = *reinterpret_cast<const BVec*>(&Bs[k * RB + c]);
          if constexpr (CG == 1) {
            b[gj] = v;
          } else {
#pragma unroll
            for (int e = 0; e < CG; ++e) b[gj * CG + e] = v[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < CG; ++e) b[gj * CG + e] = Bs[(c + e) * RB + k];
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  // Row i of the thread: group i / RG, offset i % RG; columns alike.  With 4
  // columns per group and aligned rows of C a group is one 128-bit store.
  const bool vc = (((uintptr_t)g.C & 15u) == 0) && (g.ldc % 4 == 0) && (g.N % 4 == 0);
  const int m_left = g.M - m0, n_left = g.N - n0;   // rows, columns from the corner
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = (i / RG) * 16 * RG + RG * ty + i % RG;
    const bool row_ok = row < m_left;
#pragma unroll
    for (int gj = 0; gj < Cfg::NGN; ++gj) {
      const int col = gj * 16 * CG + CG * tx;
      const uint32_t off = ((uint32_t)row * (uint32_t)g.ldc + (uint32_t)col) * 4u;
      bool done = false;
      if constexpr (CG == 4) {
        if (vc) {
          const f32x4 v = {acc[i][4 * gj], acc[i][4 * gj + 1], acc[i][4 * gj + 2],
                           acc[i][4 * gj + 3]};
          store4(rc, (row_ok && col < n_left) ? off : kOob, v);
          done = true;
        }
      }
      if (!done) {
#pragma unroll
        for (int e = 0; e < CG; ++e)
          store1(rc, (row_ok && col + e < n_left) ? off + 4u * e : kOob, acc[i][gj * CG + e]);
      }
    }
  }
}

}  // namespace sg
