// sgemm.hip -- the C ABI of include/sgemm.h: argument checks, kernel choice
// and launch on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/sgemm.h"
#include "kernel_fma.hpp"
#include "kernel_mfma.hpp"
#include "kernel_simple.hpp"

namespace {

using sg::GemmArgs;

constexpr int64_t kMaxOperandBytes = int64_t(1) << 31;  // 32-bit offsets, kOob

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
  if (algo < SGEMM_ALGO_AUTO || algo > SGEMM_ALGO_MFMA) return SGEMM_ERR_INVALID_ARG;
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
    if (o.bytes < 0 || o.bytes >= kMaxOperandBytes) return SGEMM_ERR_UNSUPPORTED;
  if (overlaps(C, cb, A, ab) || overlaps(C, cb, B, bb)) return SGEMM_ERR_INVALID_ARG;
  out.a_bytes = ab;
  out.b_bytes = bb;
  out.c_bytes = cb;
  out.launch = (M > 0 && N > 0);
  return SGEMM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

typedef void (*KernelFn)(GemmArgs);

struct Plan {
  sgemm_plan info;
  KernelFn fn;
};

template <int BM, int BN, int WM, int WN>
KernelFn mfma_fn(bool va, bool vb) {
  if (va && vb) return sg::sgemm_mfma_kernel<BM, BN, WM, WN, true, true>;
  if (va) return sg::sgemm_mfma_kernel<BM, BN, WM, WN, true, false>;
  if (vb) return sg::sgemm_mfma_kernel<BM, BN, WM, WN, false, true>;
  return sg::sgemm_mfma_kernel<BM, BN, WM, WN, false, false>;
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

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void set_name(sgemm_plan& p, const char* fam, bool va, bool vb) {
  snprintf(p.kernel, sizeof(p.kernel), "%s_%dx%dx%d_%s%s", fam, p.tile_m,
           p.tile_n, p.tile_k, va ? "va" : "sa", vb ? "vb" : "sb");
}

// Chooses the kernel and fills the launch geometry for checked arguments.
Plan plan_for(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
              const float* B, int64_t ldb, const float* C, int64_t ldc,
              int algo) {
  Plan p;
  memset(&p, 0, sizeof(p));
  const bool va = aligned16(A) && lda % 4 == 0 && K % 4 == 0;
  const bool vb = aligned16(B) && ldb % 4 == 0 && N % 4 == 0;
  const bool vc = aligned16(C) && ldc % 4 == 0 && N % 4 == 0;
  if (algo == SGEMM_ALGO_AUTO) algo = SGEMM_ALGO_MFMA;
  p.info.algo = algo;
  p.info.tile_k = 16;
  if (algo == SGEMM_ALGO_SIMPLE) {
    p.info.tile_m = p.info.tile_n = sg::kSimpleT;
    p.info.threads = sg::kSimpleT * sg::kSimpleT;
    p.info.lds_bytes = 2 * sg::kSimpleT * sg::kSimpleT * 4;
    p.fn = sg::sgemm_simple_kernel;
    snprintf(p.info.kernel, sizeof(p.info.kernel), "simple_16x16x16");
  } else if (algo == SGEMM_ALGO_FMA) {
    p.info.tile_m = p.info.tile_n = 128;
    p.info.threads = sg::FmaCfg::NT;
    p.info.lds_bytes = sg::FmaCfg::LDS_FLOATS * 4;
    p.info.vec_a = va;
    p.info.vec_b = vb;
    p.fn = fma_fn(va, vb, vc);
    set_name(p.info, "fma", va, vb);
  } else {
    // 128 x 128 tiles when they give every CU at least one; 64 x 64 tiles
    // otherwise (small and ragged shapes), so that fewer CUs sit idle.
    const int64_t t128 = cdiv(M, 128) * cdiv(N, 128);
    if (t128 >= 256) {
      using Cfg = sg::MfmaCfg<128, 128, 64, 64>;
      p.info.tile_m = p.info.tile_n = 128;
      p.info.threads = Cfg::NT;
      p.info.lds_bytes = Cfg::LDS_FLOATS * 4;
      p.fn = mfma_fn<128, 128, 64, 64>(va, vb);
    } else {
      using Cfg = sg::MfmaCfg<64, 64, 32, 32>;
      p.info.tile_m = p.info.tile_n = 64;
      p.info.threads = Cfg::NT;
      p.info.lds_bytes = Cfg::LDS_FLOATS * 4;
      p.fn = mfma_fn<64, 64, 32, 32>(va, vb);
    }
    p.info.vec_a = va;
    p.info.vec_b = vb;
    set_name(p.info, "mfma", va, vb);
  }
  p.info.workgroups = (M > 0 && N > 0)
                          ? cdiv(M, p.info.tile_m) * cdiv(N, p.info.tile_n)
                          : 0;
  return p;
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

  GemmArgs g;
  g.A = A;
  g.B = B;
  g.C = C;
  g.a_bytes = (uint32_t)c.a_bytes;
  g.b_bytes = (uint32_t)c.b_bytes;
  g.c_bytes = (uint32_t)c.c_bytes;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  // A leading dimension only matters past the first row; keep it in range.
  g.lda = (int)(M > 1 ? lda : (K > 1 ? K : 1));
  g.ldb = (int)(K > 1 ? ldb : (N > 1 ? N : 1));
  g.ldc = (int)(M > 1 ? ldc : (N > 1 ? N : 1));
  g.tiles_m = (int)cdiv(M, p.info.tile_m);
  g.tiles_n = (int)cdiv(N, p.info.tile_n);
  g.group_m = g.tiles_m < 8 ? g.tiles_m : 8;

  void* kargs[] = {&g};
  const hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(p.fn),
                      dim3((unsigned)p.info.workgroups), dim3(p.info.threads),
                      kargs, 0, stream);
  return e == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
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
  *plan = plan_for(M, N, K, A, lda, B, ldb, C, ldc, algo).info;
  return SGEMM_OK;
}

const char* sgemm_status_string(int status) {
  switch (status) {
    case SGEMM_OK: return "success";
    case SGEMM_ERR_INVALID_ARG: return "invalid argument";
    case SGEMM_ERR_UNSUPPORTED: return "unsupported: an operand spans 2 GiB or more";
    case SGEMM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int sgemm_version(void) { return SGEMM_VERSION; }

}  // extern "C"
