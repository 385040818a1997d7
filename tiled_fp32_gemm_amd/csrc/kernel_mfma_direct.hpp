// kernel_mfma_direct.hpp -- FP32 MFMA GEMM with direct global->LDS staging.
//
// Same MFMA microkernel, k regrouping and epilogue as kernel_mfma.hpp, but
// the slabs go from global memory straight into LDS with the gfx950
// buffer-load-to-LDS form (16 bytes per lane), bypassing registers.  That is
// the nearest CDNA4 counterpart of the asynchronous copy the pages mention
// ("Memory-bank mechanism and accelerated compute", section on alternatives
// to padding); here it removes the staging registers and the LDS store
// instructions, and one slab is in flight while the other is computed (two
// LDS stages).
//
// Alignment and edges.  The load-to-LDS form takes 16 bytes from any
// 4-byte-aligned address and range-checks each 4-byte word against the
// resource, so rows of any alignment and leading dimension are loaded as
// whole 4-float groups.  A lane's offset inside a slab never changes: each
// slab moves the two resources instead (A's base to the tile's first row and
// the slab's first column, B's to the slab's first row and the tile's first
// column, their sizes shrunk to match), so a load is one instruction with no
// per-lane address arithmetic.  The range check then does the edges:
//   * A groups of rows >= M and B groups starting at a column >= N get the
//     offset kOob once, and read zeros in every slab;
//   * B rows k >= K lie past the end of the moved B resource and read zeros
//     (when K is shorter than one slab they get kOob instead, since their
//     offsets could reach 2^31);
//   * a B group reaching past column N-1 brings in values that only feed C
//     columns >= N, which are never stored;
//   * A words at k >= K of a row below M-1 are inside the allocation (the
//     next row, a padding column that may hold NaN or Inf): in the last slab,
//     when it is partial, the lane that loaded such a group overwrites those
//     words with 0 in LDS before the slab's barrier.  This is the pages' rule
//     that an edge writes 0 for invalid elements ("CUDA in depth (5)",
//     section on edges).
// The last slab, which loads nothing, and the one before it, whose successor
// loads nothing, are peeled off the main loop, so the loads between the
// matrix instructions need no branch and every wait count in the loop is
// the same.
//
// A direct load writes lane l's 16 bytes at base + 16 l, so each layout is
// chosen as a permutation of 16-byte units that keeps every load instruction
// lane-linear and every read conflict-free on 64 banks of 4 bytes:
//
//   A stage (BM x BK): rows in blocks of 16; inside a block the BK/4 k
//     groups follow each other, row fastest: unit(r, c) = 4 BK (r / 16) +
//     16 c + r % 16.  A load instruction covers 16 rows x 64 contiguous
//     bytes of global memory; an MFMA fragment read by 16 consecutive lanes
//     (16 consecutive rows, one k group) is 256 contiguous bytes.
//   B stage (BK x BN): rows as in memory with the 16-byte units of rows whose
//     bit 3 is set XOR-swizzled by 8: unit(k, q) = k BN/4 + (q ^ 8 [k & 8]).
//     The B reads give lanes 0-31 row 16 s + p and lanes 32-63 row
//     16 s + 8 + p of sub-slab s; the swizzle puts the two halves on the two
//     disjoint halves of the banks (the pages' XOR swizzle idea,
//     "Memory-bank mechanism and accelerated compute", section on
//     alternatives to padding, applied at 16-byte granularity so that the
//     128-bit units stay whole).  With one 32-column block per wave a lane
//     reads one word per row; with two, block j takes the wave's columns
//     2 i + j (i = lane mod 32) instead of 32 j + i, so a lane's two words
//     of a row are adjacent and come in one 64-bit read (32 lanes: 256
//     contiguous bytes), and its two C values of a row leave in one 64-bit
//     store.
//
// Pipeline.  Slabs rotate through STAGES LDS stages, so that STAGES - 1
// slabs are in flight.  Every variant the library launches uses two: on
// MI355X three and four stages timed level or slower for the small tiles as
// well, whose slabs compute briefly.  A wave reads its MFMA
// fragments one 8-deep chunk ahead of the matrix instructions that use them,
// into two register sets of one chunk each (the registers one 16-deep
// sub-slab would take), and the slab barrier sits before the last chunk's
// matrix instructions: before it, each wave waits for its own loads of slab
// t + 1 and its reads of slab t's last chunk; after it, slab t's last chunk
// computes from registers while slab t + 1's first chunk is read and slab
// t + 2 is loaded into the stage slab t has left.  The matrix pipe thus has
// a chunk of every wave's work queued across each barrier and each slab's
// first fragment reads, which with the fragments read after the barrier
// left it idle (measured on MI355X: +1 to +2% at 4096^3 and 8192^3 for the
// 256 x 256 tile, +2 to +6% for the smaller tiles on mid-size shapes).  With one wave group a
// slab's loads go out one at a time among the last chunk's matrix
// instructions: issued together, the loads of all waves land in LDS at the
// same moment and hold up the fragment reads.  With K split inside the
// workgroup a wave's chunk is short, and the loads go out at once.
//
// Split K inside the workgroup (KS > 1, for shapes with too few tiles to fill
// the chip): KS wave groups compute the same tile over their own sub-slabs
// of every slab; the partial tiles are summed through LDS in group order.
//
// Split K across workgroups (SPLIT, for grids that even the smallest tiles
// leave under-filled): workgroup (s, tile) computes the tile over the s-th
// range of k_split values of K into a partial buffer; sgemm_split_reduce
// (kernel_reduce.hpp) then adds the partials in split order.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace sg {

template <int BM, int BN, int WM, int WN, int BK_ = 32, int KS_ = 1, int STAGES_ = 2>
struct DirectCfg {
  static constexpr int BK = BK_, KS = KS_;
  static constexpr int STAGES = STAGES_;    // slab buffers in LDS
  static constexpr int SUB = BK / 16;       // 16-deep sub-slabs per slab
  static constexpr int SUB_G = SUB / KS;    // ... per wave group
  static constexpr int CPR = BK / 4;        // 16-byte k groups per A row
  static constexpr int WAVES_N = BN / WN;
  static constexpr int SPATIAL = (BM / WM) * (BN / WN);  // waves per group
  static constexpr int NT = 64 * SPATIAL * KS;
  static constexpr int TA = WM / 32, TB = WN / 32;
  static constexpr int A_STAGE = BM * BK;   // floats
  static constexpr int B_STAGE = BK * BN;
  static constexpr int STAGE_FLOATS = STAGES * (A_STAGE + B_STAGE);
  static constexpr int RED_FLOATS = (KS - 1) * BM * BN;
  static constexpr int LDS_FLOATS =
      STAGE_FLOATS > RED_FLOATS ? STAGE_FLOATS : RED_FLOATS;
  static constexpr int A_SLOTS = BM * BK / 4 / NT;
  static constexpr int B_SLOTS = BK * BN / 4 / NT;
  static constexpr int LOADS = A_SLOTS + B_SLOTS;  // vector loads per slab
  static_assert(A_SLOTS * NT * 4 == BM * BK && B_SLOTS * NT * 4 == BK * BN,
                "slabs must split into whole 64-lane load instructions");
  static_assert(BM % 32 == 0 && BN >= 64 && BN % 64 == 0, "tile shape");
  static_assert(LOADS < 64, "wait count must fit the 6-bit field");
  static_assert(BK % 16 == 0, "slabs of whole sub-slabs");
  static_assert(SUB % KS == 0, "each wave group takes whole sub-slabs");
  static_assert(STAGES >= 2 && (STAGES - 2) * LOADS < 64, "stages");
};

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima; the
// 6-bit vector-memory count is split over bits 3:0 and 15:14).
template <int n>
struct VmWait {
  static_assert(n >= 0 && n < 64, "vector-memory count is 6 bits");
  static constexpr int imm = (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14);
};

// s_waitcnt immediate that waits for every LDS access of this wave (lgkmcnt
// 0, the other counts at their maxima).
constexpr int kLdsWait = 0xF | (0x7 << 4) | (0x3 << 14);

template <int BM, int BN, int WM, int WN, int BK_ = 32, int KS_ = 1, int STAGES_ = 2,
          bool SPLIT = false>
__global__ void __launch_bounds__(64 * (BM / WM) * (BN / WN) * KS_)
sgemm_mfma_direct_kernel(GemmArgs g_in) {
  using Cfg = DirectCfg<BM, BN, WM, WN, BK_, KS_, STAGES_>;
  constexpr int S = Cfg::STAGES;
  constexpr int BK = Cfg::BK, NT = Cfg::NT, TA = Cfg::TA, TB = Cfg::TB;
  constexpr int CPR = Cfg::CPR;
  constexpr int KS = Cfg::KS, SUB_G = Cfg::SUB_G;
  constexpr int QB = BN / 4;  // 16-byte units per B row

  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS_FLOATS];
  float* const As = lds;                                // [STAGES][A_STAGE]
  float* const Bs = lds + Cfg::STAGES * Cfg::A_STAGE;   // [STAGES][B_STAGE]

  // Split K across workgroups: this workgroup's K range becomes the whole
  // product of a narrower A and a shorter B, its tile goes to the partial
  // buffer.  Everything below then reads g as for an unsplit product.
  GemmArgs g = g_in;
  int tm, tn;
  if constexpr (SPLIT) {
    int split;
    tile_split_of_workgroup(g_in, tm, tn, split);
    const int kb = split * g_in.k_split;
    g.K = min(g_in.k_split, g_in.K - kb);
    g.A = g_in.A + kb;
    g.a_bytes = g_in.a_bytes - 4 * (int64_t)kb;
    g.B = g_in.B + (int64_t)kb * g_in.ldb;
    g.b_bytes = g_in.b_bytes - 4 * (int64_t)kb * g_in.ldb;
    g.C = g_in.W + (int64_t)split * g_in.M * g_in.N;
    g.ldc = g_in.N;
    g.c_bytes = 4 * (int64_t)g_in.M * g_in.N;
  } else {
    tile_of_workgroup(g, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Wave group and place in the group (with one group, the wave itself:
  // said outright, since the compiler cannot know that wave < SPATIAL).
  const int grp = KS == 1 ? 0 : wave / Cfg::SPATIAL;
  const int sw = KS == 1 ? wave : wave % Cfg::SPATIAL;
  const int wm0 = (sw / Cfg::WAVES_N) * WM;
  const int wn0 = (sw % Cfg::WAVES_N) * WN;
  const int li = lane & 31, lh = lane >> 5;

  // The tile's corner of each operand: A from row m0, B from column n0, C
  // from (m0, n0).  Rows and columns below are counted from there.
  const float* const At = g.A + (int64_t)m0 * g.lda;
  const uint32_t a_cap =
      cap_bytes((uint64_t)(g.a_bytes - 4 * (int64_t)m0 * g.lda), (uint32_t)kRsrcMax);
  const float* const Bt = g.B + n0;
  const int64_t b_rem = g.b_bytes - 4 * (int64_t)n0;
  const int m_left = g.M - m0, n_left = g.N - n0;
  const __amdgpu_buffer_rsrc_t rc = rsrc_at(g.C, g.c_bytes, (int64_t)m0 * g.ldc + n0);

  // Unit u = s NT + 64 wave + lane of each load instruction, and the offset
  // of the global 4-float group it takes in every slab (kOob when outside
  // the matrix in M or N).  a_unit gives the row and k group of A slot s.
  auto a_unit = [&](int s, int ln, int& row, int& c) {
    const int u = s * NT + 64 * wave + ln;
    row = (u / (16 * CPR)) * 16 + (u & 15);
    c = (u >> 4) % CPR;
  };
  uint32_t a_off[Cfg::A_SLOTS];
#pragma unroll
  for (int s = 0; s < Cfg::A_SLOTS; ++s) {
    int row, c;
    a_unit(s, lane, row, c);
    a_off[s] = row < m_left ? ((uint32_t)row * (uint32_t)g.lda + 4u * c) * 4u : kOob;
  }
  uint32_t b_off[Cfg::B_SLOTS];
#pragma unroll
  for (int s = 0; s < Cfg::B_SLOTS; ++s) {
    const int u = s * NT + 64 * wave + lane;
    const int k = u / QB, q = (u % QB) ^ ((k & 8) ? 8 : 0);
    // Rows k < min(K, BK) lie less than 2^31 bytes from a slab's first row
    // (checked on the host).  With K >= BK that is every row; with K < BK
    // there is one slab, and its rows past K, which may lie further away,
    // get kOob rather than an offset that would wrap.
    b_off[s] = (4 * q < n_left && k < g.K)
                   ? ((uint32_t)k * (uint32_t)g.ldb + (uint32_t)(4 * q)) * 4u
                   : kOob;
  }
  // The resources of the slab starting at k0 (< K: slabs from K on are
  // never loaded): A moved by k0 columns, B by k0 rows, each size shrunk to
  // match.
  auto rsrc_a = [&](int k0) { return rsrc_slab_a(At, a_cap, k0); };
  auto rsrc_b = [&](int k0) { return rsrc_at(Bt, b_rem, (int64_t)k0 * g.ldb); };

  // Issue direct load l (the A slots, then the B slots) of a slab with
  // resources (qa, qb) into stage st.
  auto issue_one = [&](int l, __amdgpu_buffer_rsrc_t qa, __amdgpu_buffer_rsrc_t qb, int st) {
#pragma unroll
    for (int s = 0; s < Cfg::A_SLOTS; ++s) {
      if (l != s) continue;
      float* dst = As + st * Cfg::A_STAGE + 4 * (s * NT + 64 * wave);
      load4_to_lds(qa, dst, a_off[s]);
    }
#pragma unroll
    for (int s = 0; s < Cfg::B_SLOTS; ++s) {
      if (l != Cfg::A_SLOTS + s) continue;
      float* dst = Bs + st * Cfg::B_STAGE + 4 * (s * NT + 64 * wave);
      load4_to_lds(qb, dst, b_off[s]);
    }
  };
  auto issue = [&](__amdgpu_buffer_rsrc_t qa, __amdgpu_buffer_rsrc_t qb, int st) {
#pragma unroll
    for (int l = 0; l < Cfg::LOADS; ++l) issue_one(l, qa, qb, st);
  };

  f32x16 acc[TA][TB];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nslab = (g.K + BK - 1) / BK;
  const bool k_tail = g.K % BK != 0;  // the last slab reaches past k = K

  // Zeroes this lane's own A words at k >= K of slab t in stage st, once its
  // loads have landed (rows >= M read zeros already): each 16-byte unit that
  // reaches past K is read and written back whole, so that the 16 lanes an
  // LDS access serves together (16 rows of one k group, 16 consecutive
  // units) touch every bank once.  Runs once per tile: the lane's unit is
  // worked out again here rather than kept in registers through the loop.
  auto fix_tail = [&](int t, int st) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int s = 0; s < Cfg::A_SLOTS; ++s) {
      int row, c;
      a_unit(s, ln, row, c);
      const int k = t * BK + 4 * c;
      if (k + 4 > g.K && row < m_left) {
        f32x4* unit =
            reinterpret_cast<f32x4*>(As + st * Cfg::A_STAGE + 4 * (s * NT + 64 * wave + ln));
        f32x4 v = *unit;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (k + e >= g.K) v[e] = 0.0f;
        *unit = v;
      }
    }
  };

  // Spread the loads only where a slab's compute is long (one wave group):
  // with split K a slab lasts a few hundred cycles per wave, and issuing its
  // successor's loads any later costs more than the burst does.
  constexpr bool kSpread = KS == 1;

  // With two 32-column blocks per wave, block j takes the wave's columns
  // 2 li + j rather than 32 j + li: a lane's two B words of a k step are
  // then adjacent (one 64-bit LDS read) and so are its two C words of a row
  // (one 64-bit store).
  constexpr bool kPairB = TB == 2;

  // The chunk pipeline described at the top of the file.
  constexpr int NCH = 2 * SUB_G;  // chunks per slab of this wave group
  struct Frag {
    f32x4 a[TA];      // k group 2 lh + (c & 1) of sub-slab c >> 1
    float b[TB][4];   // 4 k steps
  };
  // Chunk c of the slab in stage st: k steps 4 (c & 1) .. 4 (c & 1) + 3 of
  // this wave group's sub-slab c >> 1, in the lane layout of the loop
  // below.
  auto read_chunk = [&](Frag& f, int st, int c) {
    const float* as = As + st * Cfg::A_STAGE;
    const float* bs = Bs + st * Cfg::B_STAGE;
    const int sub = grp * SUB_G + (c >> 1), h = c & 1;
#pragma unroll
    for (int i = 0; i < TA; ++i) {
      const int row = wm0 + 32 * i + li;
      const float* p = as + 4 * ((row >> 4) * (16 * CPR) + (row & 15));
      f.a[i] = *reinterpret_cast<const f32x4*>(p + 4 * 16 * (4 * sub + 2 * lh + h));
    }
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int k = 16 * sub + 8 * lh + 4 * h + pp;
      if constexpr (kPairB) {
        // Columns 2 li and 2 li + 1 of the wave's 64: one 64-bit read.
        const int col = wn0 + 2 * li;
        const int q = (col >> 2) ^ (lh ? 8 : 0);
        const f32x2 v = *reinterpret_cast<const f32x2*>(bs + 4 * (k * QB + q) + (col & 3));
        f.b[0][pp] = v[0];
        f.b[1][pp] = v[1];
      } else {
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          const int col = wn0 + 32 * j + li;
          const int q = (col >> 2) ^ (lh ? 8 : 0);
          f.b[j][pp] = bs[4 * (k * QB + q) + (col & 3)];
        }
      }
    }
  };
  // The matrix instructions of a chunk; with LOADS set, load l of the
  // slab (qa, qb) goes into stage st before k step l * 4 / LOADS.
  // With pin_first set, the first k step's instructions stay where they are
  // written; the rest may move (see step).
  auto mfma_chunk = [&](const Frag& f, auto loads, __amdgpu_buffer_rsrc_t qa,
                        __amdgpu_buffer_rsrc_t qb, int st, auto pin_first) {
    constexpr bool kLoads = decltype(loads)::value;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      if constexpr (kLoads) {
#pragma unroll
        for (int l = 0; l < Cfg::LOADS; ++l)
          if (pp == l * 4 / Cfg::LOADS) issue_one(l, qa, qb, st);
      }
#pragma unroll
      for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i][pp], f.b[j][pp],
                                                           acc[i][j], 0, 0, 0);
      if constexpr (decltype(pin_first)::value)
        if (pp == 0) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Chunks 0 .. NCH-2 of slab t (stage st), each after the read of the
  // next; the scheduling barriers keep each read ahead of the chunk it
  // overlaps.
  Frag fr[2];
  const __amdgpu_buffer_rsrc_t qz = make_rsrc(g.A, 0u);  // for load-free chunks
  auto chunks = [&](int st) {
#pragma unroll
    for (int c = 0; c + 1 < NCH; ++c) {
      read_chunk(fr[(c + 1) & 1], st, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      // With K split over four wave groups, the first k step of the chunk
      // that precedes the slab barrier stays ahead of it (see step).
      mfma_chunk(fr[c & 1], std::false_type(), qz, qz, 0,
                 std::integral_constant<bool, KS == 4>());
    }
  };
  // Slab t (stage st = t mod S; slab j always lives in stage j mod S) when
  // a slab t + 1 follows: its chunks, then this wave's loads of slab t + 1
  // and its reads of the last chunk are waited for, the barrier publishes
  // slab t + 1 and frees stage st, the first chunk of slab t + 1 is read,
  // and the last chunk of slab t computes while (LOADS set) slab t + S is
  // loaded into stage st.  With LOADS set, slabs t + 2 .. t + S - 1 are in
  // flight behind slab t + 1 and stay so across the wait; without, the
  // wait takes every load (the last steps, which load nothing).
  auto step = [&](int t, int st, auto loads) {
    constexpr bool kLoads = decltype(loads)::value;
    // Slab t + S's resources are formed here, among slab t's matrix
    // instructions, rather than between the barrier and the loads.
    const int kn = (t + S) * BK;
    __amdgpu_buffer_rsrc_t qa = qz, qb = qz;
    if constexpr (kLoads) {
      qa = rsrc_a(kn);
      qb = rsrc_b(kn);
    }
    chunks(st);
    // Matrix instructions touch no memory, so the barrier alone does not
    // keep them ahead of it; where they go was measured on MI355X.  With K
    // split over two wave groups, every chunk but the last stays ahead of
    // the barrier (+1 to +5%).  With four groups, whose single accumulator
    // makes a chunk a chain of dependent instructions, only the chunk's
    // first k step does (mfma_chunk's pin_first): the matrix pipe has work
    // across the barrier and the wave still reaches it, and its next loads,
    // early.  With one group the compiler's own placement measured best.
    if constexpr (KS == 2) __builtin_amdgcn_sched_barrier(0);
    const int nst = (t + 1) % S;
    __builtin_amdgcn_s_waitcnt(VmWait<kLoads ? (S - 2) * Cfg::LOADS : 0>::imm);
    if (k_tail && t + 2 == nslab) fix_tail(t + 1, nst);
    __builtin_amdgcn_s_waitcnt(kLdsWait);
    asm volatile("s_barrier" ::: "memory");
    if constexpr (kSpread) {
      read_chunk(fr[0], nst, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk(fr[1], loads, qa, qb, st, std::false_type());
    } else {
      // With K split inside the workgroup a wave's chunk is short: its
      // loads go out at once.
      if constexpr (kLoads) issue(qa, qb, st);
      read_chunk(fr[0], nst, 0);
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk(fr[1], std::false_type(), qz, qz, st, std::false_type());
    }
  };
  if (nslab > 0) {
    // Prologue: slabs 0 .. S - 2 go out at once, into stages 0 .. S - 2;
    // slab 0 is waited for (with every slab behind it, when fewer than
    // S - 2 follow), published, and slab S - 1 goes out.
    issue(rsrc_a(0), rsrc_b(0), 0);
#pragma unroll
    for (int j = 1; j + 1 < S; ++j)
      if (j < nslab) issue(rsrc_a(j * BK), rsrc_b(j * BK), j);
    if (S == 2 || nslab >= S - 1)
      __builtin_amdgcn_s_waitcnt(VmWait<(S - 2) * Cfg::LOADS>::imm);
    else
      __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
    if (k_tail && nslab == 1) fix_tail(0, 0);
    __builtin_amdgcn_s_waitcnt(kLdsWait);
    asm volatile("s_barrier" ::: "memory");
    if (nslab > S - 1) issue(rsrc_a((S - 1) * BK), rsrc_b((S - 1) * BK), S - 1);
    read_chunk(fr[0], 0, 0);
    int t = 0;
    for (; t + S < nslab; ++t) step(t, t % S, std::true_type());
    if constexpr (S == 2) {
      if (t + 1 < nslab) {
        step(t, t % S, std::false_type());
        ++t;
      }
    } else {
      for (; t + 1 < nslab; ++t) step(t, t % S, std::false_type());
    }
    chunks(t % S);
    mfma_chunk(fr[1], std::false_type(), qz, qz, 0, std::false_type());
  }

  if constexpr (KS > 1) {
    // Groups 1..KS-1 leave their partial tiles in LDS (lane-contiguous, so
    // conflict-free) and group 0 adds them in group order (a fixed order, so
    // the result is run-to-run deterministic).  The barrier first lets every
    // wave finish reading the last stage.
    __syncthreads();
    float* red = lds;
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

  // The lane's place in C, worked out again rather than kept in registers
  // through the loop (the 256 x 256 tile needs every register it may have).
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int li_c = ln & 31, lh_c = ln >> 5;
  if constexpr (kPairB) {
    const int col = wn0 + 2 * li_c;   // and col + 1, from the tile's corner
    // Inside C's columns the pair goes out as one 64-bit store; at the
    // tile's right edge each word is stored (or dropped) on its own.
    const bool edge = n_left < wn0 + WN;
    const bool ok0 = col < n_left, ok1 = col + 1 < n_left;
    auto store_rows = [&](auto at_edge) {
#pragma unroll
      for (int i = 0; i < TA; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm0 + 32 * i + 8 * (r >> 2) + 4 * lh_c + (r & 3);
          const uint32_t at = ((uint32_t)row * (uint32_t)g.ldc + (uint32_t)col) * 4u;
          const bool row_ok = row < m_left;
          if constexpr (decltype(at_edge)::value) {
            const uint32_t off0 = row_ok && ok0 ? at : kOob;
            const uint32_t off1 = row_ok && ok1 ? at + 4u : kOob;
            if constexpr (SPLIT) {
              store1(rc, off0, acc[i][0][r]);
              store1(rc, off1, acc[i][1][r]);
            } else {
              store1_nt(rc, off0, acc[i][0][r]);
              store1_nt(rc, off1, acc[i][1][r]);
            }
          } else {
            const f32x2 v = {acc[i][0][r], acc[i][1][r]};
            const uint32_t off = row_ok ? at : kOob;
            if constexpr (SPLIT)
              store2(rc, off, v);
            else
              store2_nt(rc, off, v);
          }
        }
      }
    };
    if (edge)
      store_rows(std::true_type());
    else
      store_rows(std::false_type());
    return;
  }
#pragma unroll
  for (int i = 0; i < TA; ++i) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int col = wn0 + 32 * j + li_c;   // from the tile's corner
      const bool col_ok = col < n_left;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm0 + 32 * i + 8 * (r >> 2) + 4 * lh_c + (r & 3);
        const bool ok = col_ok && row < m_left;
        const uint32_t off =
            ok ? ((uint32_t)row * (uint32_t)g.ldc + (uint32_t)col) * 4u : kOob;
        if constexpr (SPLIT)
          store1(rc, off, acc[i][j][r]);
        else
          store1_nt(rc, off, acc[i][j][r]);
      }
    }
  }
}

}  // namespace sg
