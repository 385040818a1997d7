/*
 * sgemm_probe.h -- measurement aids for the benchmark of libsgemm (not part
 * of the product: libsgemm_probe.so holds no GEMM).
 *
 * The pages' measurement recipe fixes the clocks and the tool versions
 * before timing anything ("Memory-bank mechanism and accelerated compute",
 * section on turning derivations into measurements, first step).  A GPU's
 * shader clock is not fixed by the caller: it ramps with load and varies
 * between hosts.  These calls let a benchmark record the clock its kernels
 * actually ran at, and the runtime and driver versions.
 */
#ifndef SGEMM_PROBE_H
#define SGEMM_PROBE_H

#include <stdint.h>

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of the clock probe: one per compute unit of an MI355X. */
#define SGEMM_PROBE_WORKGROUPS 256
/* Waves per workgroup: four per SIMD. */
#define SGEMM_PROBE_WAVES 16
/* v_mfma_f32_32x32x2_f32 instructions each wave issues per iteration. */
#define SGEMM_PROBE_MFMA_PER_ITER 16
/* Cycles one v_mfma_f32_32x32x2_f32 holds its SIMD's matrix pipe (16
 * passes of 4 cycles: 32 x 32 x 2 multiply-adds at 64 flop per cycle per
 * SIMD, i.e. the 256 flop per cycle per CU of the FP32 matrix peak). */
#define SGEMM_PROBE_MFMA_CYCLES 64

/* Enqueues the clock probe on stream: SGEMM_PROBE_WORKGROUPS workgroups of
 * SGEMM_PROBE_WAVES waves, each reserving enough LDS that a compute unit
 * holds only one, so that every CU runs exactly one; every wave issues
 * iters x SGEMM_PROBE_MFMA_PER_ITER independent FP32 matrix instructions and
 * nothing else.  Each SIMD's matrix pipe is then busy for
 *   iters x SGEMM_PROBE_MFMA_PER_ITER x (SGEMM_PROBE_WAVES / 4) x
 *   SGEMM_PROBE_MFMA_CYCLES cycles,
 * so the launch's duration gives the clock the matrix pipes ran at.
 * stamps: device memory for 5 x SGEMM_PROBE_WORKGROUPS uint64 (caller
 * owned, 8-byte aligned); workgroup w writes, from its first wave, clock64()
 * and wall_clock64() before its loop (stamps[5w], stamps[5w + 1]) and after
 * it (stamps[5w + 2], stamps[5w + 3]), and a value derived from the
 * accumulators (stamps[5w + 4]) so that the work cannot be optimised away.
 * Returns 0, 1 for iters < 1 or a null or misaligned stamps, 3 when the
 * launch fails.  No synchronisation. */
int sgemm_probe_mfma_clock(hipStream_t stream, int iters, uint64_t *stamps);

/* The rate of wall_clock64() in kHz (hipDeviceAttributeWallClockRate of the
 * current device), the HIP runtime version and the driver version
 * (hipRuntimeGetVersion, hipDriverGetVersion).  Returns 0, or 3 when HIP
 * reports an error; any output pointer may be NULL. */
int sgemm_probe_versions(int *wall_clock_khz, int *runtime_version,
                         int *driver_version);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_PROBE_H */
