// sgemm.hip -- the C ABI of include/sgemm.h: argument checks, kernel choice
// and launch on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/sgemm.h"
#include "kernel_fma.hpp"
#include "kernel_ladder.hpp"
#include "kernel_mfma.hpp"
#include "kernel_mfma_direct.hpp"
#include "kernel_reduce.hpp"
#include "kernel_simple.hpp"
#include "kernel_transpose.hpp"

namespace {

using sg::GemmArgs;

// The kernels address each operand from the corner of their own tile with
// 32-bit byte offsets below 2^31 (kOob = 2^31 marks an element outside the
// matrix), so what is bounded is one tile's span, not an operand's size.
constexpr int64_t kMaxSpanBytes = sg::kRsrcMax;
// Tile origins and sizes are 32-bit ints in the kernels.
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1024;
// The split partials are addressed as one resource from their first byte.
constexpr int64_t kMaxWorkspaceBytes = sg::kRsrcMax;

struct Checked {
  int64_t a_bytes = 0, b_bytes = 0, c_bytes = 0;
  bool launch = false;  // false: M == 0 or N == 0, nothing to do
};

// Bytes spanned by a rows x cols row-major operand with leading dimension ld
// (0 when empty); -1 when the span does not fit in int64.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld) {
  if (rows == 0 || cols == 0) return 0;
  const int64_t lim = INT64_MAX / 4;
  if (rows - 1 > (lim - cols) / ld) return -1;
  return ((rows - 1) * ld + cols) * 4;
}

bool overlaps(const void* p, int64_t pb, const void* q, int64_t qb) {
  if (pb == 0 || qb == 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qb && b < a + (uintptr_t)pb;
}

int check(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
          const float* B, int64_t ldb, const float* C, int64_t ldc, int algo,
          Checked& out) {
  if (algo < SGEMM_ALGO_AUTO || algo > SGEMM_ALGO_MFMA_DIRECT) return SGEMM_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_INVALID_ARG;
  if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_INVALID_ARG;
  // Only what a launch touches is checked: nothing when M or N is 0, and
  // neither A nor B when K is 0.
  const bool touch = M > 0 && N > 0;
  const int64_t ab = touch ? span_bytes(M, K, lda) : 0;
  const int64_t bb = touch ? span_bytes(K, N, ldb) : 0;
  const int64_t cb = touch ? span_bytes(M, N, ldc) : 0;
  struct { const void* p; int64_t bytes; } ops[3] = {{A, ab}, {B, bb}, {C, cb}};
  for (auto& o : ops) {
    if (o.bytes == 0) continue;
    if (o.p == nullptr || ((uintptr_t)o.p & 3u) != 0) return SGEMM_ERR_INVALID_ARG;
  }
  for (auto& o : ops)
    if (o.bytes < 0) return SGEMM_ERR_UNSUPPORTED;   // beyond int64
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_ERR_UNSUPPORTED;
  if (overlaps(C, cb, A, ab) || overlaps(C, cb, B, bb)) return SGEMM_ERR_INVALID_ARG;
  out.a_bytes = ab;
  out.b_bytes = bb;
  out.c_bytes = cb;
  out.launch = (M > 0 && N > 0);
  return SGEMM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// True when rows x width floats with leading dimension ld (the first row
// starting at offset 0) end below kMaxSpanBytes: ((rows - 1) ld + width) 4
// bytes, formed without overflow.
bool span_fits(int64_t rows, int64_t width, int64_t ld) {
  if (rows <= 0 || width <= 0) return true;
  const int64_t lim = kMaxSpanBytes / 4;  // floats
  if (width >= lim) return false;
  if (rows == 1) return true;
  if (ld > (lim - 1 - width) / (rows - 1)) return false;
  return (rows - 1) * ld + width < lim;
}

// Whether a kernel with BM x BN tiles and BK-deep slabs can address this
// product: one tile's rows of A (all K columns, or BK if more) and of C, and
// one slab's rows of B (BN columns past the tile's first), each within
// kMaxSpanBytes of their first element.  ldc is the leading dimension the
// tiles are written with (N for the split partials).
bool tile_fits(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
               int64_t ldc, int bm, int bn, int bk) {
  if (K > 0 && !span_fits(M < bm ? M : bm, K > bk ? K : bk, lda)) return false;
  if (K > 0 && !span_fits(K < bk ? K : bk, bn, ldb)) return false;
  return span_fits(M < bm ? M : bm, bn, ldc);
}

// The grid's work-items, workgroups x threads, must fit in 32 bits.
bool grid_fits(int64_t workgroups, int threads) {
  return workgroups >= 0 && workgroups < ((int64_t(1) << 32) / threads);
}

typedef void (*KernelFn)(GemmArgs);
typedef void (*KernelFnT)(sg::TransposeArgs);
typedef void (*KernelFnR)(sg::ReduceArgs);

struct Plan {
  sgemm_plan info;
  KernelFn fn;
  int k_split;  // with info.splits > 1: K per split
};

bool vec_a_ok(const float* A, int64_t lda, int64_t K) {
  return aligned16(A) && lda % 4 == 0 && K % 4 == 0;
}
bool vec_b_ok(const float* B, int64_t ldb, int64_t N) {
  return aligned16(B) && ldb % 4 == 0 && N % 4 == 0;
}

// One launchable configuration of a kernel family.
struct Variant {
  const char* name;
  int tile_m, tile_n, tile_k, threads, lds_bytes;
  int stages;               // LDS slab buffers (STAGES - 1 slabs in flight)
  KernelFn vv, sv, vs, ss;  // by (A 128-bit?, B 128-bit?); null: unsupported
  KernelFn split;           // the split-K-across-workgroups form, or null
};

template <int BM, int BN, int WM, int WN, int BK>
Variant reg_variant(const char* name) {
  using Cfg = sg::MfmaCfg<BM, BN, WM, WN, BK>;
  return {name, BM, BN, BK, Cfg::NT, Cfg::LDS_FLOATS * 4, 2,
          sg::sgemm_mfma_kernel<BM, BN, WM, WN, BK, true, true>,
          sg::sgemm_mfma_kernel<BM, BN, WM, WN, BK, false, true>,
          sg::sgemm_mfma_kernel<BM, BN, WM, WN, BK, true, false>,
          sg::sgemm_mfma_kernel<BM, BN, WM, WN, BK, false, false>, nullptr};
}

// The LDS-direct kernel takes rows of any 4-byte alignment, so one kernel
// serves every load form.
template <int BM, int BN, int WM, int WN, int BK, int KS, int ST = 2>
Variant direct_variant(const char* name) {
  using Cfg = sg::DirectCfg<BM, BN, WM, WN, BK, KS, ST>;
  const KernelFn f = sg::sgemm_mfma_direct_kernel<BM, BN, WM, WN, BK, KS, ST>;
  return {name, BM, BN, Cfg::BK, Cfg::NT, Cfg::LDS_FLOATS * 4, ST, f, f, f, f,
          sg::sgemm_mfma_direct_kernel<BM, BN, WM, WN, BK, KS, ST, true>};
}

// Matrix-core configurations, large to small tiles, with the planner's two
// inputs for each:
//   eff  the fraction of a CU's FP32 matrix peak the variant sustains with
//        its pipes busy (fitted, with the constants below, to MI355X timings
//        of every variant on 196 shapes from 96 to 65536 per side; after the
//        kernels' chunk pipeline the 128 x 128 value alone was raised, which
//        brings the picks within 0.6% of the fastest variant on average over
//        170 re-timed shapes);
//   occ  the workgroups a CU holds at once, from the kernel's LDS bytes and
//        its registers per lane (512 per SIMD lane, at most 8 waves per
//        SIMD) as compiled for gfx950.
// The large tiles cut L2 traffic per flop; the small ones, and those that
// split K over wave groups, keep more of the chip busy on small, ragged or
// short-K shapes.
struct Candidate {
  Variant v;
  double eff;
  int occ;
};

const Candidate* mfma_candidates(bool direct, int& n) {
  static const Candidate reg[3] = {
      {reg_variant<256, 128, 64, 64, 16>("mfma_256x128x16"), 0.86, 2},
      {reg_variant<128, 128, 64, 32, 16>("mfma_128x128x16"), 0.81, 3},
      {reg_variant<64, 64, 32, 32, 16>("mfma_64x64x16"), 0.77, 8}};
  // LDS-direct: 32-deep slabs in two stages (one slab in flight) halve the
  // barriers per flop against 16-deep slabs in three stages.  "ks" names the
  // number of wave groups that split each slab.
  static const Candidate lds[8] = {
      {direct_variant<256, 256, 64, 64, 32, 1>("mfma_lds_256x256x32"), 0.929, 1},
      {direct_variant<128, 128, 32, 64, 32, 1>("mfma_lds_128x128x32"), 0.895, 2},
      {direct_variant<64, 128, 32, 64, 32, 1>("mfma_lds_64x128x32"), 0.901, 3},
      {direct_variant<64, 128, 32, 64, 32, 2>("mfma_lds_64x128x32_ks2"), 0.805, 3},
      {direct_variant<64, 64, 32, 32, 32, 1>("mfma_lds_64x64x32"), 0.837, 5},
      {direct_variant<64, 64, 32, 32, 32, 2>("mfma_lds_64x64x32_ks2"), 0.830, 4},
      {direct_variant<32, 64, 32, 32, 32, 2>("mfma_lds_32x64x32_ks2"), 0.799, 6},
      {direct_variant<32, 64, 32, 32, 64, 4>("mfma_lds_32x64x64_ks4"), 0.807, 3}};
  n = direct ? 8 : 3;
  return direct ? lds : reg;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kCUs = 256;                      // MI355X compute units
constexpr double kPeakPerCU = 157.3e12 / kCUs;  // FP32 matrix flop/s per CU
constexpr double kSaturate = 1.28;   // waves per SIMD that keep the pipes busy
constexpr double kSlabFloor = 0.61e-6;  // s: a slab's wait for its loads
constexpr double kRoundCost = 4.4e-6;   // s: fill and drain of one round
constexpr double kWriteBW = 4.52e12;    // B/s: C stores of a final round

// Estimated seconds of variant c on an M x N x K product.  Workgroups are
// spread evenly over the CUs, so the busiest CU computes n = ceil(tiles /
// CUs) tiles (charging partial-tile padding and the idle CUs of the last
// round, i.e. wave quantisation), in rounds of up to occ resident ones.  In a
// round of r tiles every slab takes the longer of its compute (r tiles'
// flops at eff of the CU's peak, in proportion below kSaturate waves per
// SIMD) and the latency of its loads; each round adds a fixed cost; and the
// C tiles of the final round, which all CUs store at once, are charged at
// the chip's write bandwidth.
double estimate_grid(const Candidate& c, int64_t tiles, int64_t K) {
  const Variant& v = c.v;
  const int64_t n = cdiv(tiles, kCUs);
  const int64_t slabs = K > v.tile_k ? cdiv(K, v.tile_k) : 1;
  const double waves = v.threads / 64.0;
  const double slab_flops = 2.0 * v.tile_m * v.tile_n * v.tile_k;
  auto round = [&](int64_t r) {
    const double simd = r * waves / 4.0;
    const double busy = simd >= kSaturate ? 1.0 : simd / kSaturate;
    const double compute = r * slab_flops / (kPeakPerCU * c.eff * busy);
    return (double)slabs * (compute > kSlabFloor ? compute : kSlabFloor) + kRoundCost;
  };
  const int64_t full = n / c.occ, rest = n % c.occ;
  double t = (double)full * round(c.occ) + (rest > 0 ? round(rest) : 0.0);
  const int64_t last = rest > 0 ? rest : c.occ;
  const int64_t cus = tiles < kCUs ? tiles : kCUs;
  t += (double)last * cus * v.tile_m * v.tile_n * 4.0 / kWriteBW;
  return t;
}

double estimate(const Candidate& c, int64_t M, int64_t N, int64_t K) {
  return estimate_grid(c, cdiv(M, c.v.tile_m) * cdiv(N, c.v.tile_n), K);
}

// Whether candidate c can address the product (tile spans, grid size).
bool candidate_fits(const Candidate& c, int64_t M, int64_t N, int64_t K,
                    int64_t lda, int64_t ldb, int64_t ldc) {
  const Variant& v = c.v;
  return tile_fits(M, N, K, lda, ldb, ldc, v.tile_m, v.tile_n, v.tile_k) &&
         grid_fits(cdiv(M, v.tile_m) * cdiv(N, v.tile_n), v.threads);
}

// The candidate with the least estimated time among those that fit; ties
// keep the earlier (larger-tile) one.  Null when none fits.
const Candidate* choose_mfma(int64_t M, int64_t N, int64_t K, int64_t lda,
                             int64_t ldb, int64_t ldc, bool direct) {
  int n;
  const Candidate* c = mfma_candidates(direct, n);
  const Candidate* best = nullptr;
  double best_t = 0;
  for (int i = 0; i < n; ++i) {
    if (!candidate_fits(c[i], M, N, K, lda, ldb, ldc)) continue;
    const double t = estimate(c[i], M, N, K);
    if (best == nullptr || t < best_t * 0.995) {
      best = &c[i];
      best_t = t;
    }
  }
  return best;
}

// Split K across workgroups, for grids that leave the chip under-filled:
// S splits of k_split (a multiple of the slab) make S times the workgroups,
// each over a K range of its own, into S partial tiles in the workspace; a
// second pass adds them in split order.  Its cost: the partial products
// (the model above, on tiles x S workgroups of depth k_split), plus the
// reduction's (S + 1) M N 4 bytes at HBM speed and its launch.
constexpr double kReduceFixed = 3.0e-6;  // s
constexpr double kReduceBW = 5.0e12;     // B/s, a device copy's rate
constexpr double kSplitMargin = 0.97;    // split only when clearly faster
// The model over-states the partial pass, whose workgroups see short K and
// fill the CUs evenly; scaled by this (one value, chosen on timings of every
// plan on 64 under-filled shapes and checked on each half of them).
constexpr double kSplitPartial = 0.95;

struct Choice {
  const Candidate* c;
  int splits, k_split;
};

Choice choose_direct(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, int64_t ws_bytes) {
  Choice best = {choose_mfma(M, N, K, lda, ldb, ldc, true), 1, 0};
  if (best.c == nullptr) return best;
  const double t_one = estimate(*best.c, M, N, K);
  if (ws_bytes <= 0 || M == 0 || N == 0 || K < 2) return best;
  int n;
  const Candidate* cs = mfma_candidates(true, n);
  static const int kSplits[] = {2, 3, 4, 6, 8, 12, 16, 24, 32};
  double t_best = 0;
  Choice split = best;
  for (int i = 0; i < n; ++i) {
    const Candidate& c = cs[i];
    const int64_t tiles = cdiv(M, c.v.tile_m) * cdiv(N, c.v.tile_n);
    for (int S : kSplits) {
      const int64_t ks = cdiv(cdiv(K, S), c.v.tile_k) * c.v.tile_k;
      const int64_t se = cdiv(K, ks);  // splits actually used
      if (se < 2) continue;
      const int64_t bytes = se * M * N * 4;
      if (bytes > ws_bytes || bytes >= kMaxWorkspaceBytes) continue;
      // The partial products read A and B as the product does and write
      // tiles with rows of N floats.
      if (!tile_fits(M, N, ks, lda, ldb, N, c.v.tile_m, c.v.tile_n, c.v.tile_k) ||
          !grid_fits(tiles * se, c.v.threads) || !grid_fits(M * cdiv(N, sg::kReduceCols),
                                                            sg::kReduceThreads))
        continue;
      const double t = kSplitPartial * estimate_grid(c, tiles * se, ks) + kReduceFixed +
                       (double)(se + 1) * M * N * 4.0 / kReduceBW;
      if (split.splits == 1 || t < t_best) {
        split = {&c, (int)se, (int)ks};
        t_best = t;
      }
    }
  }
  if (split.splits > 1 && t_best < t_one * kSplitMargin) return split;
  return best;
}

KernelFn fma_fn(bool va, bool vb, bool vc) {
  const int idx = (va ? 4 : 0) | (vb ? 2 : 0) | (vc ? 1 : 0);
  static const KernelFn table[8] = {
      sg::sgemm_fma_kernel<false, false, false>, sg::sgemm_fma_kernel<false, false, true>,
      sg::sgemm_fma_kernel<false, true, false>,  sg::sgemm_fma_kernel<false, true, true>,
      sg::sgemm_fma_kernel<true, false, false>,  sg::sgemm_fma_kernel<true, false, true>,
      sg::sgemm_fma_kernel<true, true, false>,   sg::sgemm_fma_kernel<true, true, true>};
  return table[idx];
}

void set_name(sgemm_plan& p, const char* base, bool va, bool vb) {
  snprintf(p.kernel, sizeof(p.kernel), "%s_%s%s", base, va ? "va" : "sa",
           vb ? "vb" : "sb");
}

// Chooses the kernel and fills the launch geometry for checked arguments.
Plan plan_for(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
              const float* B, int64_t ldb, const float* C, int64_t ldc,
              int algo, int64_t ws_bytes = 0) {
  Plan p;
  memset(&p, 0, sizeof(p));
  p.info.splits = 1;
  // With K == 0 neither A nor B is read, so any load form will do.
  const bool va = K == 0 || vec_a_ok(A, lda, K);
  const bool vb = K == 0 || vec_b_ok(B, ldb, N);
  const bool vc = aligned16(C) && ldc % 4 == 0 && N % 4 == 0;
  if (algo == SGEMM_ALGO_AUTO) algo = SGEMM_ALGO_MFMA_DIRECT;
  p.info.algo = algo;
  p.info.vec_a = va;
  p.info.vec_b = vb;
  if (algo == SGEMM_ALGO_SIMPLE) {
    p.info.tile_m = p.info.tile_n = p.info.tile_k = sg::kSimpleT;
    p.info.threads = sg::kSimpleT * sg::kSimpleT;
    p.info.lds_bytes = 2 * sg::kSimpleT * sg::kSimpleT * 4;
    p.info.vec_a = p.info.vec_b = 0;
    p.info.wg_per_cu = 8;  // 8 waves per SIMD at 44 registers per lane
    p.fn = sg::sgemm_simple_kernel;
    snprintf(p.info.kernel, sizeof(p.info.kernel), "simple_16x16x16");
  } else if (algo == SGEMM_ALGO_FMA) {
    p.info.tile_m = p.info.tile_n = 128;
    p.info.tile_k = 16;
    p.info.threads = sg::FmaCfg::NT;
    p.info.lds_bytes = sg::FmaCfg::LDS_FLOATS * 4;
    p.info.wg_per_cu = 4;  // 116 registers per lane: 4 waves per SIMD
    p.fn = fma_fn(va, vb, vc);
    set_name(p.info, "fma_128x128x16", va, vb);
  } else {
    Choice ch = {nullptr, 1, 0};
    if (algo == SGEMM_ALGO_MFMA_DIRECT) ch = choose_direct(M, N, K, lda, ldb, ldc, ws_bytes);
    else ch.c = choose_mfma(M, N, K, lda, ldb, ldc, false);
    if (ch.c == nullptr) return p;  // no tile can address this product
    const Candidate& cand = *ch.c;
    const Variant& v = cand.v;
    p.info.wg_per_cu = cand.occ;
    p.info.tile_m = v.tile_m;
    p.info.tile_n = v.tile_n;
    p.info.tile_k = v.tile_k;
    p.info.threads = v.threads;
    p.info.lds_bytes = v.lds_bytes;
    if (ch.splits > 1) {
      p.fn = v.split;
      p.k_split = ch.k_split;
      p.info.splits = ch.splits;
      p.info.workspace_bytes = (int64_t)ch.splits * M * N * 4;
      snprintf(p.info.kernel, sizeof(p.info.kernel), "%s_split%d", v.name, ch.splits);
    } else {
      p.fn = va ? (vb ? v.vv : v.vs) : (vb ? v.sv : v.ss);
      set_name(p.info, v.name, va, vb);
    }
  }
  p.info.workgroups = (M > 0 && N > 0)
                          ? cdiv(M, p.info.tile_m) * cdiv(N, p.info.tile_n) * p.info.splits
                          : 0;
  // The fixed-tile families (the matrix-core ones were chosen among fitting
  // candidates above).
  if (p.info.splits == 1 &&
      (!tile_fits(M, N, K, lda, ldb, ldc, p.info.tile_m, p.info.tile_n, p.info.tile_k) ||
       !grid_fits(p.info.workgroups, p.info.threads)))
    p.fn = nullptr;
  return p;
}

// Kernel arguments for checked operands and a launch of fn over the tiles
// of C.
int launch_gemm(KernelFn fn, int64_t M, int64_t N, int64_t K, const float* A,
                int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                const Checked& c, int tile_m, int tile_n, int threads,
                hipStream_t stream, int splits = 1, int k_split = 0,
                float* W = nullptr) {
  GemmArgs g;
  g.A = A;
  g.B = B;
  g.C = C;
  g.a_bytes = c.a_bytes;
  g.b_bytes = c.b_bytes;
  g.c_bytes = c.c_bytes;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  // A leading dimension only matters past the first row of an operand that
  // is read or written; there the checks bound it below 2^29.
  g.lda = (int)(M > 1 && K > 0 ? lda : (K > 1 ? K : 1));
  g.ldb = (int)(K > 1 ? ldb : (N > 1 ? N : 1));
  g.ldc = (int)(M > 1 ? ldc : (N > 1 ? N : 1));
  g.tiles_m = (int)cdiv(M, tile_m);
  g.tiles_n = (int)cdiv(N, tile_n);
  g.group_m = g.tiles_m < 8 ? g.tiles_m : 8;
  g.splits = splits;
  g.k_split = k_split;
  g.W = W;

  void* kargs[] = {&g};
  const hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(fn),
      dim3((unsigned)((int64_t)g.tiles_m * g.tiles_n * splits)), dim3(threads), kargs, 0,
      stream);
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

// C = the sum of the splits partial products in W, in split order.
int launch_reduce(const float* W, int splits, int64_t M, int64_t N, float* C,
                  int64_t ldc, const Checked& c, hipStream_t stream) {
  sg::ReduceArgs r;
  r.W = W;
  r.C = C;
  r.w_bytes = (uint32_t)(splits * M * N * 4);
  r.c_bytes = c.c_bytes;
  r.M = (int)M;
  r.N = (int)N;
  r.ldc = (int)(M > 1 ? ldc : (N > 1 ? N : 1));
  r.splits = splits;
  r.chunks = (int)cdiv(N, sg::kReduceCols);
  const bool vw = aligned16(W) && N % 4 == 0;
  const bool vc = vw && aligned16(C) && r.ldc % 4 == 0;
  static const KernelFnR table[3] = {sg::sgemm_split_reduce_kernel<false, false>,
                                     sg::sgemm_split_reduce_kernel<true, false>,
                                     sg::sgemm_split_reduce_kernel<true, true>};
  const KernelFnR fn = table[vc ? 2 : (vw ? 1 : 0)];
  void* kargs[] = {&r};
  const hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(fn), dim3((unsigned)(M * r.chunks)),
      dim3(sg::kReduceThreads), kargs, 0, stream);
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

// The workspace of sgemm_ws_noalloc: a file-scope device array, of which
// every device the library runs on holds its own copy (at its own address)
// until the process ends.  In host code `scratch` is only a handle for
// hipGetSymbolAddress; the kernels get the device address from scratch_of.
constexpr int64_t kScratchBytes = SGEMM_NOALLOC_MAX_BYTES;
}  // namespace

static __device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  float* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

// The device address of device dev's scratch, looked up once per device
// with dev current (made current for the lookup when it is not, and the
// caller's device restored); null when HIP reports an error.
float* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot, dev] {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
      slot.ptr = static_cast<float*>(p);
    if (cur != dev && hipSetDevice(cur) != hipSuccess) slot.ptr = nullptr;
  });
  return slot.ptr;
}

// The device a launch on stream runs on: the stream's own, or for the null
// stream the current device.
bool stream_device(hipStream_t stream, int& dev) {
  if (stream == nullptr) return hipGetDevice(&dev) == hipSuccess;
  hipDevice_t d = -1;
  if (hipStreamGetDevice(stream, &d) != hipSuccess) return false;
  dev = (int)d;
  return true;
}

// The ablation ladder.  Each step changes one thing against the one before;
// the vector-ALU steps 0-10 run the kernels of kernel_ladder.hpp (and the
// pages' basic tiled loop, kernel_simple.hpp), the last three the product
// families.  Steps with 128-bit loads fall back to 32-bit ones when A or B
// rows are not 16-byte aligned.
struct LadderStep {
  const char* name;
  KernelFn vec, sca;  // 128-bit / 32-bit load forms (same for the others)
  int tile_m, tile_n;
  int algo;           // >= 0: the step is the product family sgemm_ex(algo)
};

template <int TM, int TN, int AL, int BL, bool VEC>
LadderStep ladder_step(const char* name) {
  return {name, sg::sgemm_ladder_kernel<TM, TN, AL, BL, VEC>,
          sg::sgemm_ladder_kernel<TM, TN, AL, BL, false>, 16 * TM, 16 * TN, -1};
}

const LadderStep* ladder_steps(int& n) {
  static const LadderStep steps[] = {
      {"naive_global", sg::sgemm_naive_kernel, sg::sgemm_naive_kernel, 16, 16, -1},
      {"lds_tile_16", sg::sgemm_simple_kernel, sg::sgemm_simple_kernel, 16, 16, -1},
      ladder_step<1, 1, sg::kAPadded, sg::kBRows, false>("reg_1x1"),
      ladder_step<2, 2, sg::kAPadded, sg::kBRows, false>("reg_2x2"),
      ladder_step<4, 4, sg::kAPadded, sg::kBRows, false>("reg_4x4"),
      ladder_step<8, 8, sg::kAPadded, sg::kBRows, false>("reg_8x8"),
      ladder_step<8, 8, sg::kAPadded, sg::kBRows, true>("reg_8x8_vec128"),
      ladder_step<8, 8, sg::kAUnpadded, sg::kBRows, true>("reg_8x8_vec128_a_unpadded"),
      ladder_step<8, 8, sg::kASwizzled, sg::kBRows, true>("reg_8x8_vec128_a_xor"),
      ladder_step<8, 8, sg::kAPadded, sg::kBCols, true>("reg_8x8_vec128_b_transposed"),
      ladder_step<8, 8, sg::kAPadded, sg::kBColsPadded, true>(
          "reg_8x8_vec128_b_transposed_padded"),
      {"reg_8x8_vec128_double_buffer", nullptr, nullptr, 0, 0, SGEMM_ALGO_FMA},
      {"mfma_register_staging", nullptr, nullptr, 0, 0, SGEMM_ALGO_MFMA},
      {"mfma_direct_to_lds", nullptr, nullptr, 0, 0, SGEMM_ALGO_MFMA_DIRECT}};
  n = (int)(sizeof(steps) / sizeof(steps[0]));
  return steps;
}

}  // namespace

extern "C" {

int sgemm_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
             const float* B, int64_t ldb, float* C, int64_t ldc,
             hipStream_t stream, int algo) {
  Checked c;
  const int st = check(M, N, K, A, lda, B, ldb, C, ldc, algo, c);
  if (st != SGEMM_OK || !c.launch) return st;
  const Plan p = plan_for(M, N, K, A, lda, B, ldb, C, ldc, algo);
  if (p.fn == nullptr) return SGEMM_ERR_UNSUPPORTED;  // no kernel for this form

  return launch_gemm(p.fn, M, N, K, A, lda, B, ldb, C, ldc, c, p.info.tile_m,
                     p.info.tile_n, p.info.threads, stream);
}

int sgemm_ladder_steps(void) {
  int n;
  ladder_steps(n);
  return n;
}

const char* sgemm_ladder_name(int step) {
  int n;
  const LadderStep* s = ladder_steps(n);
  return (step >= 0 && step < n) ? s[step].name : nullptr;
}

int sgemm_ladder(int step, int64_t M, int64_t N, int64_t K, const float* A,
                 int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                 hipStream_t stream) {
  int n;
  const LadderStep* steps = ladder_steps(n);
  if (step < 0 || step >= n) return SGEMM_ERR_INVALID_ARG;
  const LadderStep& ls = steps[step];
  if (ls.algo >= 0) return sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, ls.algo);
  Checked c;
  const int st = check(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_AUTO, c);
  if (st != SGEMM_OK || !c.launch) return st;
  // Every vector-ALU step walks K in 16-deep slabs.
  if (!tile_fits(M, N, K, lda, ldb, ldc, ls.tile_m, ls.tile_n, 16) ||
      !grid_fits(cdiv(M, ls.tile_m) * cdiv(N, ls.tile_n), 256))
    return SGEMM_ERR_UNSUPPORTED;
  const bool vec = K == 0 || (vec_a_ok(A, lda, K) && vec_b_ok(B, ldb, N));
  return launch_gemm(vec ? ls.vec : ls.sca, M, N, K, A, lda, B, ldb, C, ldc, c,
                     ls.tile_m, ls.tile_n, 256, stream);
}

int sgemm_ws(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
             const float* B, int64_t ldb, float* C, int64_t ldc,
             hipStream_t stream, void* workspace, int64_t workspace_bytes) {
  if (workspace_bytes < 0 || (workspace_bytes > 0 && workspace == nullptr) ||
      ((uintptr_t)workspace & 3u))
    return SGEMM_ERR_INVALID_ARG;
  Checked c;
  const int st = check(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_AUTO, c);
  if (st != SGEMM_OK || !c.launch) return st;
  const Plan p = plan_for(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_MFMA_DIRECT,
                          workspace_bytes);
  if (p.fn == nullptr) return SGEMM_ERR_UNSUPPORTED;
  if (p.info.splits == 1)
    return launch_gemm(p.fn, M, N, K, A, lda, B, ldb, C, ldc, c, p.info.tile_m,
                       p.info.tile_n, p.info.threads, stream);
  float* W = static_cast<float*>(workspace);
  const int64_t wb = p.info.workspace_bytes;
  if (overlaps(W, wb, A, c.a_bytes) || overlaps(W, wb, B, c.b_bytes) ||
      overlaps(W, wb, C, c.c_bytes))
    return SGEMM_ERR_INVALID_ARG;
  const int e = launch_gemm(p.fn, M, N, K, A, lda, B, ldb, W, N, c, p.info.tile_m,
                            p.info.tile_n, p.info.threads, stream, p.info.splits,
                            p.k_split, W);
  if (e != SGEMM_OK) return e;
  return launch_reduce(W, p.info.splits, M, N, C, ldc, c, stream);
}

int sgemm_ws_noalloc(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                     const float* B, int64_t ldb, float* C, int64_t ldc,
                     hipStream_t stream, int64_t workspace_bytes) {
  if (workspace_bytes < 0) return SGEMM_ERR_INVALID_ARG;
  if (workspace_bytes > kScratchBytes) return SGEMM_ERR_SCRATCH_LIMIT;
  Checked c;
  const int st = check(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_AUTO, c);
  if (st != SGEMM_OK || !c.launch) return st;
  const Plan p = plan_for(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_MFMA_DIRECT,
                          workspace_bytes);
  if (p.fn == nullptr) return SGEMM_ERR_UNSUPPORTED;
  if (p.info.splits == 1)
    return launch_gemm(p.fn, M, N, K, A, lda, B, ldb, C, ldc, c, p.info.tile_m,
                       p.info.tile_n, p.info.threads, stream);
  int dev = -1;
  if (!stream_device(stream, dev)) return SGEMM_ERR_LAUNCH;
  float* const W = scratch_of(dev);
  if (W == nullptr) return SGEMM_ERR_LAUNCH;
  const int64_t wb = p.info.workspace_bytes;
  if (overlaps(W, wb, A, c.a_bytes) || overlaps(W, wb, B, c.b_bytes) ||
      overlaps(W, wb, C, c.c_bytes))
    return SGEMM_ERR_INVALID_ARG;
  const int e = launch_gemm(p.fn, M, N, K, A, lda, B, ldb, W, N, c, p.info.tile_m,
                            p.info.tile_n, p.info.threads, stream, p.info.splits,
                            p.k_split, W);
  if (e != SGEMM_OK) return e;
  return launch_reduce(W, p.info.splits, M, N, C, ldc, c, stream);
}

int64_t sgemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  // Contiguous operands (lda = K, ldb = ldc = N).
  const Choice ch = choose_direct(M, N, K, K > 1 ? K : 1, N, N, kMaxWorkspaceBytes);
  return ch.c != nullptr && ch.splits > 1 ? (int64_t)ch.splits * M * N * 4 : 0;
}

int sgemm_plan_query_ws(int64_t M, int64_t N, int64_t K, const float* A,
                        int64_t lda, const float* B, int64_t ldb, const float* C,
                        int64_t ldc, int64_t workspace_bytes, sgemm_plan* plan) {
  if (plan == nullptr || workspace_bytes < 0) return SGEMM_ERR_INVALID_ARG;
  Checked c;
  const int st = check(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_AUTO, c);
  if (st != SGEMM_OK) return st;
  const Plan p = plan_for(M, N, K, A, lda, B, ldb, C, ldc, SGEMM_ALGO_MFMA_DIRECT,
                          workspace_bytes);
  if (c.launch && p.fn == nullptr) return SGEMM_ERR_UNSUPPORTED;
  *plan = p.info;
  return SGEMM_OK;
}

int sgemm(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
          const float* B, int64_t ldb, float* C, int64_t ldc,
          hipStream_t stream) {
  return sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_ALGO_AUTO);
}

int sgemm_plan_query(int64_t M, int64_t N, int64_t K, const float* A,
                     int64_t lda, const float* B, int64_t ldb, const float* C,
                     int64_t ldc, int algo, sgemm_plan* plan) {
  if (plan == nullptr) return SGEMM_ERR_INVALID_ARG;
  Checked c;
  const int st = check(M, N, K, A, lda, B, ldb, C, ldc, algo, c);
  if (st != SGEMM_OK) return st;
  const Plan p = plan_for(M, N, K, A, lda, B, ldb, C, ldc, algo);
  if (c.launch && p.fn == nullptr) return SGEMM_ERR_UNSUPPORTED;
  *plan = p.info;
  return SGEMM_OK;
}

int sgemm_transpose_ex(int64_t rows, int64_t cols, const float* in,
                       int64_t ldi, float* out, int64_t ldo,
                       hipStream_t stream, int layout) {
  if (layout < SGEMM_TRANSPOSE_AUTO || layout > SGEMM_TRANSPOSE_SWIZZLED)
    return SGEMM_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0) return SGEMM_ERR_INVALID_ARG;
  if (ldi < (cols > 1 ? cols : 1) || ldo < (rows > 1 ? rows : 1))
    return SGEMM_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return SGEMM_OK;
  const int64_t ib = span_bytes(rows, cols, ldi), ob = span_bytes(cols, rows, ldo);
  if (in == nullptr || out == nullptr || ((uintptr_t)in & 3u) || ((uintptr_t)out & 3u))
    return SGEMM_ERR_INVALID_ARG;
  if (ib < 0 || ob < 0) return SGEMM_ERR_UNSUPPORTED;   // beyond int64
  if (overlaps(in, ib, out, ob)) return SGEMM_ERR_INVALID_ARG;
  // A tile reads rows of the input and writes rows of the output from its
  // corner with 32-bit offsets.
  const int64_t tiles = cdiv(cols, sg::kTransposeCols) * cdiv(rows, sg::kTransposeRows);
  if (rows > kMaxDim || cols > kMaxDim || !grid_fits(tiles, 256) ||
      !span_fits(rows < sg::kTransposeRows ? rows : sg::kTransposeRows,
                 sg::kTransposeCols, ldi) ||
      !span_fits(cols < sg::kTransposeCols ? cols : sg::kTransposeCols,
                 sg::kTransposeRows, ldo))
    return SGEMM_ERR_UNSUPPORTED;

  sg::TransposeArgs a;
  a.in = in;
  a.out = out;
  a.in_bytes = ib;
  a.out_bytes = ob;
  a.rows = (int)rows;
  a.cols = (int)cols;
  a.ldi = (int)(rows > 1 ? ldi : (cols > 1 ? cols : 1));
  a.ldo = (int)(cols > 1 ? ldo : (rows > 1 ? rows : 1));
  a.tiles_x = (int)cdiv(cols, sg::kTransposeCols);
  const bool vi = aligned16(in) && a.ldi % 4 == 0 && cols % 4 == 0;
  const bool vo = aligned16(out) && a.ldo % 4 == 0 && rows % 4 == 0;
  if (layout == SGEMM_TRANSPOSE_AUTO) layout = SGEMM_TRANSPOSE_SWIZZLED;
  static const KernelFnT table[3][4] = {
#define SG_T(L) {sg::sgemm_transpose_kernel<L, false, false>,   \
                 sg::sgemm_transpose_kernel<L, false, true>,    \
                 sg::sgemm_transpose_kernel<L, true, false>,    \
                 sg::sgemm_transpose_kernel<L, true, true>}
      SG_T(sg::kNaive), SG_T(sg::kPadded), SG_T(sg::kSwizzled)
#undef SG_T
  };
  const KernelFnT fn = table[layout - 1][(vi ? 2 : 0) | (vo ? 1 : 0)];
  void* kargs[] = {&a};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                       dim3((unsigned)tiles), dim3(256), kargs,
                                       0, stream);
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_transpose(int64_t rows, int64_t cols, const float* in, int64_t ldi,
                    float* out, int64_t ldo, hipStream_t stream) {
  return sgemm_transpose_ex(rows, cols, in, ldi, out, ldo, stream,
                            SGEMM_TRANSPOSE_AUTO);
}

const char* sgemm_status_string(int status) {
  switch (status) {
    case SGEMM_OK: return "success";
    case SGEMM_ERR_INVALID_ARG: return "invalid argument";
    case SGEMM_ERR_UNSUPPORTED:
      return "unsupported: a dimension of 2^31 - 1024 or more, one tile's rows of an "
             "operand spanning 2 GiB or more, or a grid of 2^32 work-items or more";
    case SGEMM_ERR_LAUNCH: return "kernel launch failed";
    case SGEMM_ERR_SCRATCH_LIMIT:
      return "workspace request beyond the 32 MiB static scratch of sgemm_ws_noalloc";
    default: return "unknown status";
  }
}

int sgemm_version(void) { return SGEMM_VERSION; }

}  // extern "C"
