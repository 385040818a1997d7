// probe.hip -- the clock probe and version query of include/sgemm_probe.h.
// A measurement aid for the benchmark; it holds no GEMM.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/sgemm_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS per workgroup that leaves room for one workgroup per CU (160 KiB).
constexpr int kProbeLdsFloats = 96 * 1024 / 4;

__global__ void __launch_bounds__(64 * SGEMM_PROBE_WAVES)
mfma_clock_probe_kernel(int iters, uint64_t* stamps) {
  __shared__ float pin[kProbeLdsFloats];  // reserved, see above
  const int tid = (int)threadIdx.x;
  // Operand values do not matter; they are per-lane so nothing folds.
  const float a = (float)(tid & 7) * 0.125f, b = 1.0f / 64.0f;
  // Four accumulators, each updated every fourth instruction, so no
  // instruction waits for the one before it.
  constexpr int kAcc = 4;
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  // Each lane touches its own word only; volatile keeps the reservation.
  volatile float* const vpin = pin;
  vpin[tid] = a;
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < SGEMM_PROBE_MFMA_PER_ITER; ++j)
      acc[j % kAcc] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j % kAcc], 0, 0, 0);
  }
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  float s = vpin[tid];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (tid == 0) {
    uint64_t* o = stamps + 5 * (size_t)blockIdx.x;
    o[0] = c0;
    o[1] = w0;
    o[2] = c1;
    o[3] = w1;
    o[4] = (uint64_t)__float_as_uint(s);
  }
}

}  // namespace

extern "C" {

int sgemm_probe_mfma_clock(hipStream_t stream, int iters, uint64_t* stamps) {
  if (iters < 1 || stamps == nullptr || ((uintptr_t)stamps & 7u) != 0) return 1;
  void* kargs[] = {&iters, &stamps};
  const hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(mfma_clock_probe_kernel),
      dim3(SGEMM_PROBE_WORKGROUPS), dim3(64 * SGEMM_PROBE_WAVES), kargs, 0, stream);
  return e == hipSuccess ? 0 : 3;
}

int sgemm_probe_versions(int* wall_clock_khz, int* runtime_version,
                         int* driver_version) {
  if (wall_clock_khz != nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(wall_clock_khz, hipDeviceAttributeWallClockRate, dev) !=
            hipSuccess)
      return 3;
  }
  if (runtime_version != nullptr && hipRuntimeGetVersion(runtime_version) != hipSuccess)
    return 3;
  if (driver_version != nullptr && hipDriverGetVersion(driver_version) != hipSuccess)
    return 3;
  return 0;
}

}  // extern "C"
