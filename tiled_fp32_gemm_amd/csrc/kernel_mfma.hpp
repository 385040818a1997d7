// kernel_mfma.hpp -- FP32 GEMM on the gfx950 matrix cores.
//
// Data path (the one the pages lay out for a tiled GEMM: global memory ->
// vectorised coalesced load -> registers -> shared memory in a chosen layout
// -> register fragments -> multiply-add; "CUDA in depth (5)", section on the
// GEMM data path), mapped onto CDNA4:
//
//  * One workgroup owns a BM x BN tile of C and walks K in slabs of BK (16 or
//    32) floats.
//    Its waves split the tile into WM x WN wave tiles, each a grid of 32 x 32
//    blocks computed by v_mfma_f32_32x32x2_f32 (FP32 in, FP32 fused
//    multiply-add, accumulators in registers).
//  * Global -> registers: 128-bit buffer loads (VEC_A / VEC_B) or, when a row
//    is not 16-byte aligned, four 32-bit loads per 4-float group; elements
//    outside the matrix read as 0 through the buffer range check.  Each slab
//    reads through resources moved to its own corner (A: the tile's first
//    row and the slab's first column; B: the slab's first row and the tile's
//    first column), so the per-lane offsets do not grow with K.
//  * Registers -> LDS, double buffered: the loads for slab t+1 are issued
//    before the matrix instructions of slab t and written to the other LDS
//    stage after them, with one barrier per slab.
//  * LDS layouts, chosen for gfx950's 64 banks of 4 bytes:
//      As[BM][BK+4] A rows, k contiguous (BK used, 4 pad).  A row is BK + 4
//                   floats, an odd number of 16-byte units (5 or 9): sixteen
//                   consecutive rows start at sixteen different 16-byte bank
//                   groups, so the 128-bit stores and reads below, which give
//                   consecutive lanes consecutive rows, touch each bank once
//                   per 16 lanes.
//      Bs[16][BN+4] B rows as in memory (j contiguous).  128-bit stores are
//                   256 contiguous bytes per 16 lanes; 32-bit reads give
//                   lanes 0-31 one row and lanes 32-63 the row 8 below, and
//                   8 * (BN + 4) = 32 (mod 64) puts the two halves on
//                   disjoint banks.
//  * Split K inside the workgroup (KS > 1, for shapes with too few tiles to
//    fill the chip): KS wave groups each compute the same BM x BN tile over
//    their own share of every slab's sub-slabs, and the partial tiles are
//    summed through LDS at the end.
//  * The k order inside each 16-deep sub-slab is regrouped: MFMA step p (0..7)
//    takes k = p from lanes 0-31 and k = 8 + p from lanes 32-63.  Every k is
//    still used exactly once for A and B alike, and each lane's eight A values
//    are contiguous in As, so they come in as two 128-bit reads (the pages'
//    "segmented storage matching the register tile's read order",
//    "CUDA in depth (5)", section on why data is re-laid out in shared memory).
//
// MFMA operand layout (32x32x2, one block): lane l supplies A[l % 32][l / 32]
// and B[l / 32][l % 32]; accumulator element r of lane l is
// C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].
#pragma once

#include "common.hpp"

namespace sg {

template <int BM, int BN, int WM, int WN, int BK_ = 16, int KS_ = 1>
struct MfmaCfg {
  static constexpr int BK = BK_;
  static constexpr int KS = KS_;       // wave groups sharing each slab
  static constexpr int SUB = BK / 16;  // 16-deep sub-slabs per slab
  static constexpr int SUB_G = SUB / KS;  // ... per wave group
  static constexpr int CPR = BK / 4;   // 4-float groups per A tile row
  static constexpr int WAVES_M = BM / WM;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int SPATIAL = WAVES_M * WAVES_N;  // waves per group
  static constexpr int NT = 64 * SPATIAL * KS;
  static constexpr int TA = WM / 32;  // 32x32 blocks per wave along M
  static constexpr int TB = WN / 32;  // ... along N
  static constexpr int RA = BK + 4;   // As row stride (floats)
  static constexpr int RB = BN + 4;   // Bs row stride (floats)
  static constexpr int A_STAGE = BM * RA;
  static constexpr int B_STAGE = BK * RB;
  static constexpr int STAGE_FLOATS = 2 * (A_STAGE + B_STAGE);
  static constexpr int RED_FLOATS = (KS - 1) * BM * BN;  // partial tiles
  static constexpr int LDS_FLOATS =
      STAGE_FLOATS > RED_FLOATS ? STAGE_FLOATS : RED_FLOATS;
  static constexpr int A_SLOTS = BM * BK / 4 / NT;  // 4-float groups per thread
  static constexpr int B_SLOTS = BK * BN / 4 / NT;
  static_assert(BM % WM == 0 && BN % WN == 0, "wave tiles must divide the tile");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is made of 32x32 blocks");
  static_assert(BM % 16 == 0, "A staging covers 16 rows per wave");
  static_assert(A_SLOTS * NT * 4 == BM * BK, "A tile must split evenly");
  static_assert(B_SLOTS * NT * 4 == BK * BN, "B tile must split evenly");
  static_assert((8 * RB) % 64 == 32, "B read halves must use disjoint banks");
  static_assert((RA / 4) % 2 == 1, "A row stride must be an odd number of 16B");
  static_assert(BK % 16 == 0 && BK <= 64, "slabs are whole 16-deep sub-slabs");
  static_assert(SUB % KS == 0, "each wave group takes whole sub-slabs");
};

// One 4-float group of the A slab: slot s of thread t covers A tile row
// (f % 16) + 16 * (f / (16 * CPR)) and k = 4 * ((f / 16) % CPR),
// f = s * NT + t, so the 16 lanes of each quarter-wave hold 16 consecutive
// rows at one k group.
template <class Cfg>
__device__ __forceinline__ void a_slot(int f, int& row, int& kq) {
  row = (f & 15) + (f / (16 * Cfg::CPR)) * 16;
  kq = (f >> 4) % Cfg::CPR;
}

template <int BM, int BN, int WM, int WN, int BK_, bool VEC_A, bool VEC_B,
          int KS_ = 1>
__global__ void __launch_bounds__(64 * (BM / WM) * (BN / WN) * KS_)
sgemm_mfma_kernel(GemmArgs g) {
  using Cfg = MfmaCfg<BM, BN, WM, WN, BK_, KS_>;
  constexpr int BK = Cfg::BK, NT = Cfg::NT, TA = Cfg::TA, TB = Cfg::TB;
  constexpr int KS = Cfg::KS, SUB_G = Cfg::SUB_G;
  constexpr int RA = Cfg::RA, RB = Cfg::RB;

  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS_FLOATS];
  float* const As = lds;                       // [2][BM][RA]
  float* const Bs = lds + 2 * Cfg::A_STAGE;    // [2][BK][RB]

  int tm, tn;
  tile_of_workgroup(g, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = wave / Cfg::SPATIAL, sw = wave % Cfg::SPATIAL;
  const int wm0 = (sw / Cfg::WAVES_N) * WM;
  const int wn0 = (sw % Cfg::WAVES_N) * WN;
  const int li = lane & 31, lh = lane >> 5;

  // The tile's corner of each operand (A from row m0, B from column n0, C
  // from (m0, n0)); rows and columns below are counted from there.
  const float* const At = g.A + (int64_t)m0 * g.lda;
  const uint32_t a_cap =
      cap_bytes((uint64_t)(g.a_bytes - 4 * (int64_t)m0 * g.lda), (uint32_t)kRsrcMax);
  const float* const Bt = g.B + n0;
  const int64_t b_rem = g.b_bytes - 4 * (int64_t)n0;
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(g.C, g.c_bytes, (int64_t)m0 * g.ldc + n0);

  // Per-slot byte offsets from a slab's corner and the LDS positions they
  // fill.
  uint32_t a_off[Cfg::A_SLOTS];
  bool a_row_ok[Cfg::A_SLOTS];
  int a_k[Cfg::A_SLOTS], a_lds[Cfg::A_SLOTS];
#pragma unroll
  for (int s = 0; s < Cfg::A_SLOTS; ++s) {
    int row, kq;
    a_slot<Cfg>(s * NT + tid, row, kq);
    a_row_ok[s] = row < g.M - m0;
    a_k[s] = 4 * kq;
    a_off[s] = ((uint32_t)row * (uint32_t)g.lda + 4u * kq) * 4u;
    a_lds[s] = row * RA + 4 * kq;
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

  // Global -> registers for the slab starting at k0 (< K).
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

  // Registers -> LDS stage `st`.
  auto store_slab = [&](int st) {
    float* as = As + st * Cfg::A_STAGE;
    float* bs = Bs + st * Cfg::B_STAGE;
#pragma unroll
    for (int s = 0; s < Cfg::A_SLOTS; ++s)
      *reinterpret_cast<f32x4*>(as + a_lds[s]) = sa[s];
#pragma unroll
    for (int s = 0; s < Cfg::B_SLOTS; ++s)
      *reinterpret_cast<f32x4*>(bs + b_lds[s]) = sb[s];
  };

  f32x16 acc[TA][TB];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

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
#pragma unroll
    for (int uu = 0; uu < SUB_G; ++uu) {
      const int u = grp * SUB_G + uu;  // this wave group's sub-slabs
      f32x4 af[TA][2];
#pragma unroll
      for (int i = 0; i < TA; ++i) {
        const float* p = as + (wm0 + 32 * i + li) * RA + 16 * u + 8 * lh;
        af[i][0] = *reinterpret_cast<const f32x4*>(p);
        af[i][1] = *reinterpret_cast<const f32x4*>(p + 4);
      }
      float bf[TB][8];
#pragma unroll
      for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int j = 0; j < TB; ++j)
          bf[j][p] = bs[(16 * u + 8 * lh + p) * RB + wn0 + 32 * j + li];

#pragma unroll
      for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int i = 0; i < TA; ++i)
#pragma unroll
          for (int j = 0; j < TB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                af[i][p >> 2][p & 3], bf[j][p], acc[i][j], 0, 0, 0);
    }

    if (more) store_slab(cur ^ 1);
    __syncthreads();
  }

  // Split K across wave groups: groups 1..KS-1 leave their partial tiles in
  // LDS (lane-contiguous, so conflict-free), group 0 adds them in group order
  // (a fixed order, so the result is run-to-run deterministic) and stores.
  if constexpr (KS > 1) {
    float* red = lds;  // the staging stages are free after the last barrier
    constexpr int PER_WAVE = TA * TB * 16 * 64;
    if (grp > 0) {
      float* dst = red + ((grp - 1) * Cfg::SPATIAL + sw) * PER_WAVE + lane;
#pragma unroll
      for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((i * TB + j) * 16 + r) * 64] = acc[i][j][r];
    }
    __syncthreads();
    if (grp > 0) return;  // no barrier follows
#pragma unroll
    for (int q = 1; q < KS; ++q) {
      const float* src = red + ((q - 1) * Cfg::SPATIAL + sw) * PER_WAVE + lane;
#pragma unroll
      for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] += src[((i * TB + j) * 16 + r) * 64];
    }
  }

  // Epilogue: each lane writes column wn0 + 32 j + li (from the tile's
  // corner) of 16 rows per block; lanes 0-31 cover 128 contiguous bytes of
  // one row.
#pragma unroll
  for (int i = 0; i < TA; ++i) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int col = wn0 + 32 * j + li;
      const bool col_ok = col < g.N - n0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        const bool ok = col_ok && row < g.M - m0;
        store1(rc, ok ? ((uint32_t)row * (uint32_t)g.ldc + (uint32_t)col) * 4u : kOob,
               acc[i][j][r]);
      }
    }
  }
}

}  // namespace sg
