/*
 * sgemm.h -- single-precision matrix product C = A·B on an AMD Instinct
 * MI355X (gfx950), row-major, behind a plain C ABI.
 *
 * The operation.  For 0 <= i < M and 0 <= j < N
 *
 *      C[i*ldc + j] = sum_{k=0}^{K-1} A[i*lda + k] * B[k*ldb + j]
 *
 * This is the textbook product that the tiled kernels of the pages reach by
 * other data movement only: tiling, shared-memory layout, vectorised loads and
 * register tiles change where data travels, not the result ("CUDA in depth
 * (5): vectorized load and shared-memory layout", section on the GEMM data
 * path).  Row-major storage with leading dimensions that set where each row
 * begins, possibly wider than the logical row, is the convention of the same
 * page's section on leading dimensions.  There is no alpha or beta: C is
 * overwritten.  Summation order is the kernel's own; results are
 * run-to-run deterministic (no atomics, no split-K races) and agree with the
 * exact sum within 1e-5 * sum_k |A[i][k]| |B[k][j]| for finite inputs.
 *
 * Arguments common to every entry point.
 *   M, N, K   logical sizes; C is M x N, A is M x K, B is K x N.  >= 0.
 *   A, lda    device pointer to A[0][0]; row i starts at A + i*lda.
 *             lda >= max(1, K).  Columns K..lda-1 are never read.
 *   B, ldb    device pointer to B[0][0]; row k starts at B + k*ldb.
 *             ldb >= max(1, N).  Columns N..ldb-1 are never read.
 *   C, ldc    device pointer to C[0][0]; row i starts at C + i*ldc.
 *             ldc >= max(1, N).  Columns N..ldc-1 are never written.
 *   stream    HIP stream the kernels are enqueued on (0 = null stream).
 *
 * Ownership and ordering.  All three matrices are device memory owned by the
 * caller; the library neither allocates, frees nor retains them.  Calls return
 * once the work is enqueued, without synchronising: the buffers must stay
 * valid until the stream has passed the call.  C must not overlap A or B (the
 * same no-overlap contract the pages state for their tiled transpose kernel,
 * "Memory-bank mechanism and accelerated compute", section on the transpose
 * kernel).  Pointers must be 4-byte aligned; any alignment and any leading
 * dimension are accepted, and the 128-bit load path is chosen internally when
 * the pointer is 16-byte aligned and the leading dimension and row length are
 * multiples of 4 (same pages, sections on contiguity and alignment and on
 * leading dimensions).
 *
 * Errors.  Arguments are checked before any HIP call; a rejected call
 * enqueues nothing and leaves C untouched.
 *   SGEMM_ERR_INVALID_ARG  negative size; leading dimension too small; a
 *                          null or misaligned (not 4-byte) pointer for a
 *                          non-empty operand; C overlapping A or B; an
 *                          unknown algo.
 *   SGEMM_ERR_UNSUPPORTED  M, N or K of 2^31 - 1024 or more; or, for every
 *                          tile the kernel family offers, one tile's rows
 *                          of A (all K columns) or of C, or one K slab's
 *                          rows of B, would span 2 GiB or more (the kernels
 *                          address an operand from the corner of their own
 *                          tile with 32-bit byte offsets, so operands
 *                          themselves may be of any size: this needs a
 *                          leading dimension of millions of floats, e.g.
 *                          lda >= 2^24 with 32 or more rows of A, or one
 *                          row of A of 2^29 floats); or a grid of 2^32
 *                          work-items or more.  sgemm_plan_query answers
 *                          the same.
 *   SGEMM_ERR_LAUNCH       the HIP launch reported an error.
 * M == 0 or N == 0 returns SGEMM_OK with nothing enqueued; K == 0 writes
 * C = 0 (the empty sum).
 *
 * Thread safety.  Stateless and reentrant; concurrent calls on different
 * streams are independent.
 */
#ifndef SGEMM_H
#define SGEMM_H

#include <stddef.h>
#include <stdint.h>

/* The HIP stream handle type, identical to the one hip_runtime_api.h
 * declares (a repeated identical typedef is valid C11 and C++). */
struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_VERSION 130 /* 1.3.0 */

/* Status codes. */
#define SGEMM_OK 0
#define SGEMM_ERR_INVALID_ARG 1
#define SGEMM_ERR_UNSUPPORTED 2
#define SGEMM_ERR_LAUNCH 3
#define SGEMM_ERR_SCRATCH_LIMIT 4   /* sgemm_ws_noalloc only */

/* Kernel families (sgemm_ex).
 *   AUTO    the fastest family, MFMA_DIRECT, with the tile size (and the
 *           split of K across wave groups) chosen from the shape.
 *   SIMPLE  one output per thread from 16x16 shared tiles, the basic tiled
 *           inner loop of "CUDA in depth (4): accessing shared memory
 *           efficiently", section on too many shared-memory reads.
 *   FMA     8x8 register tile per thread with vector FMA instructions, the
 *           register tiling of the same page (sections on register tiling and
 *           on going from 1x1 to 2x2), double-buffered, 128-bit loads.
 *   MFMA    the same register staging feeding the gfx950 FP32 matrix
 *           instruction (32x32x2, fused multiply-add in FP32, round to
 *           nearest even); any alignment.
 *   MFMA_DIRECT  the same matrix instructions with slabs loaded from global
 *           memory straight into LDS in 16-byte groups (any 4-byte
 *           alignment; the groups that straddle k = K are zero-filled in
 *           LDS).  Bitwise equal to MFMA when K is not split across wave
 *           groups; otherwise the partial sums of the groups are added in a
 *           fixed order. */
#define SGEMM_ALGO_AUTO 0
#define SGEMM_ALGO_SIMPLE 1
#define SGEMM_ALGO_FMA 2
#define SGEMM_ALGO_MFMA 3
#define SGEMM_ALGO_MFMA_DIRECT 4

/* C = A·B with the AUTO kernel family.  See the top of this file for the
 * arguments, layout, ownership and errors.  Returns a status code. */
int sgemm(int64_t M, int64_t N, int64_t K,
          const float *A, int64_t lda,
          const float *B, int64_t ldb,
          float *C, int64_t ldc,
          hipStream_t stream);

/* As sgemm(), with the kernel family named by algo (SGEMM_ALGO_*); an unknown
 * algo is SGEMM_ERR_INVALID_ARG.  Every family computes the same product. */
int sgemm_ex(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             hipStream_t stream, int algo);

/* What a call with these arguments would launch, without launching it.  The
 * checks and return codes are those of sgemm_ex; on SGEMM_OK *plan is filled
 * (kernel name, workgroup tile, grid).  plan must not be NULL.  AUTO picks
 * the LDS-direct tile (and K split) with the least estimated time for
 * M x N x K: wave quantisation over the 256 CUs, resident workgroups per CU,
 * slab load latency and the final C stores, with rates measured on MI355X. */
typedef struct sgemm_plan {
    int algo;            /* family actually used (AUTO resolved) */
    int tile_m, tile_n;  /* C tile per workgroup */
    int tile_k;          /* K slab staged through LDS per step */
    int threads;         /* threads per workgroup */
    int vec_a, vec_b;    /* 1 if A / B rows take 128-bit loads */
    int64_t workgroups;  /* grid size (0 when nothing is launched) */
    int lds_bytes;       /* LDS per workgroup */
    int wg_per_cu;       /* workgroups one CU holds at once (LDS and
                            registers of the kernel as built for gfx950) */
    int splits;          /* K ranges run by separate workgroups: 1, or > 1
                            for a split plan (sgemm_plan_query_ws) */
    int64_t workspace_bytes; /* workspace the plan uses (0 unless split) */
    char kernel[64];     /* kernel name, NUL-terminated */
} sgemm_plan;

int sgemm_plan_query(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     const float *C, int64_t ldc,
                     int algo, sgemm_plan *plan);

/* C = A·B with K split across workgroups when that is faster: for a C too
 * small to fill the 256 CUs with its tiles but a long K, S workgroups per C
 * tile each multiply one range of K (the per-tile product of "CUDA in depth
 * (4): accessing shared memory efficiently", section on too many
 * shared-memory reads, over a part of the k sum) into partial tiles in
 * workspace, and a second kernel adds the S partials in the order s = 0..S-1
 * into C.  The result is deterministic from run to run and within the sgemm
 * tolerance, but is not bitwise equal to sgemm() for such shapes (the k sum
 * is grouped differently).  Without a split (the shape fills the chip, or
 * workspace_bytes is below what the best split needs) this is exactly
 * sgemm(), bit for bit, and the workspace is not touched.
 *   workspace        device memory owned by the caller, 4-byte aligned, not
 *                    overlapping A, B or C; its contents on entry do not
 *                    matter and are overwritten (S x M x N floats; a split
 *                    is only planned while these stay below 2 GiB).  It must
 *                    stay allocated until the enqueued kernels finish, and
 *                    calls that share one workspace must be ordered (one
 *                    stream), or they race.  May be NULL when
 *                    workspace_bytes is 0.
 *   workspace_bytes  its size; 0 allows no split.
 * Other arguments, checks and return codes are sgemm's; a negative size, a
 * NULL workspace of nonzero size, a misaligned or overlapping workspace is
 * SGEMM_ERR_INVALID_ARG.  No allocation; two kernel launches on stream. */
int sgemm_ws(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             hipStream_t stream, void *workspace, int64_t workspace_bytes);

/* Bytes of the static scratch sgemm_ws_noalloc splits K into, per device. */
#define SGEMM_NOALLOC_MAX_BYTES (32 << 20)

/* sgemm_ws for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a file-scope device array of SGEMM_NOALLOC_MAX_BYTES that the
 * library holds on each device it runs on until the process ends (its
 * address is looked up once per device, on the first call that splits K on
 * it; the device is the stream's, or the current one for the null stream);
 * the call itself allocates nothing and frees nothing.
 *   workspace_bytes  the room the plan may take from the scratch, as
 *                    sgemm_ws's workspace_bytes (0 allows no split), at most
 *                    SGEMM_NOALLOC_MAX_BYTES; more is SGEMM_ERR_SCRATCH_LIMIT
 *                    and a negative value SGEMM_ERR_INVALID_ARG, before any
 *                    HIP call.
 * The plan, the kernels and the result are those of sgemm_ws with a
 * workspace of workspace_bytes, bit for bit.  Every call on a device shares
 * that device's one scratch, which keeps the last call's partials (each
 * split call overwrites all it reads): calls that overlap on one device (on
 * different streams, or from different threads without ordering) race and
 * must not be made.  Under HIP graph capture, make one split call on the
 * device before capturing, so that the address lookup (a HIP runtime query,
 * not a stream operation) is not made inside the capture; the captured
 * launches then read and write the scratch at replay, in stream order.
 * Other arguments, checks and return codes are sgemm_ws's; SGEMM_ERR_LAUNCH
 * also when the scratch's address cannot be had. */
int sgemm_ws_noalloc(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     hipStream_t stream, int64_t workspace_bytes);

/* The workspace size with which sgemm_ws takes its fastest plan for
 * M x N x K (0 when the best plan does not split K, or for an invalid or
 * empty shape).  Host only; no HIP call. */
int64_t sgemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The plan sgemm_ws would take with this workspace size (plan->splits and
 * plan->workspace_bytes give the split).  Checks as for sgemm_plan_query
 * with AUTO; a negative workspace_bytes or NULL plan is
 * SGEMM_ERR_INVALID_ARG. */
int sgemm_plan_query_ws(int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda,
                        const float *B, int64_t ldb,
                        const float *C, int64_t ldc,
                        int64_t workspace_bytes, sgemm_plan *plan);

/* out = in^T: in is rows x cols (row i at in + i*ldi, ldi >= max(1, cols)),
 * out is cols x rows (row j at out + j*ldo, ldo >= max(1, rows)); out[j][i]
 * = in[i][j], bit for bit.  This is the pages' tiled transpose ("Memory-bank
 * mechanism and accelerated compute", section on the transpose kernel):
 * coalesced row reads and row writes, with the column access done inside an
 * LDS tile of 64 input rows by 128 input columns.  Device pointers owned by
 * the caller, 4-byte aligned, not
 * overlapping; any leading dimension; enqueued on stream without
 * synchronising.  Errors as for sgemm (checked before any HIP call);
 * rows == 0 or cols == 0 is a no-op; SGEMM_ERR_UNSUPPORTED when rows or cols
 * is 2^31 - 1024 or more, when 64 input rows or 128 output rows would span
 * 2 GiB or more, or when the grid would reach 2^32 work-items. */
int sgemm_transpose(int64_t rows, int64_t cols,
                    const float *in, int64_t ldi,
                    float *out, int64_t ldo,
                    hipStream_t stream);

/* LDS tile layouts for sgemm_transpose_ex (all give the same result).  The
 * tile is kept as 16-byte units and every LDS access is 128 bits wide; the
 * column-wise reads of 4 x 4 blocks are where the layouts differ:
 *   NAIVE     64 x 16 units, the unpadded control: the 16 lanes served
 *             together read one 16-byte bank group (16-way conflicts).
 *   PADDED    64 x 17 units, one extra unit per row, the pages' extra column
 *             at the access width ("Memory-bank mechanism and accelerated
 *             compute", section 'one extra column'): 4-way conflicts remain.
 *   SWIZZLED  64 x 16 units, unit c of row r stored at c ^ ((r / 4) % 16)
 *             (same page, section on alternatives to padding):
 *             conflict-free; AUTO uses it. */
#define SGEMM_TRANSPOSE_AUTO 0
#define SGEMM_TRANSPOSE_NAIVE 1
#define SGEMM_TRANSPOSE_PADDED 2
#define SGEMM_TRANSPOSE_SWIZZLED 3

/* As sgemm_transpose with an explicit LDS layout; an unknown layout is
 * SGEMM_ERR_INVALID_ARG. */
int sgemm_transpose_ex(int64_t rows, int64_t cols,
                       const float *in, int64_t ldi,
                       float *out, int64_t ldo,
                       hipStream_t stream, int layout);

/* Static English text for a status code (never NULL). */
const char *sgemm_status_string(int status);

/* SGEMM_VERSION of the built library. */
int sgemm_version(void);

/* The ablation ladder: the pages' optimisations as separate kernels, each
 * step changing one thing against the step before, for measurement
 * ("CUDA in depth (4): accessing shared memory efficiently", sections on too
 * many shared-memory reads, register tiling and going from 1x1 to 2x2;
 * "CUDA in depth (5): vectorized load and shared-memory layout", sections on
 * vector loads, the B-tile example and padding with transpose; "Memory-bank
 * mechanism and accelerated compute", sections on one extra column and on
 * alternatives to padding).  Every step computes C = A.B as sgemm does and
 * takes the same arguments, checks and return codes; it is not the product
 * path (call sgemm for that).
 *   0  naive_global        one output per thread, no shared memory
 *   1  lds_tile_16         16 x 16 tiles in LDS, one output per thread
 *   2  reg_1x1             the same tiling, A stored k-major (transposed)
 *   3  reg_2x2             2 x 2 outputs per thread (32 x 32 tile)
 *   4  reg_4x4             4 x 4 (64 x 64 tile)
 *   5  reg_8x8             8 x 8 (128 x 128 tile), 32-bit loads
 *   6  reg_8x8_vec128      + 128-bit loads (32-bit where rows are unaligned)
 *   7  .._a_unpadded      A without its 4-float padding (bank conflicts)
 *   8  .._a_xor           A XOR-swizzled instead of padded
 *   9  .._b_transposed    B stored transposed, Bs[BN][16] (bank conflicts)
 *   10 .._b_transposed_padded  ... as Bs[BN][17]
 *   11 reg_8x8_vec128_double_buffer  = sgemm_ex(..., SGEMM_ALGO_FMA)
 *   12 mfma_register_staging         = sgemm_ex(..., SGEMM_ALGO_MFMA)
 *   13 mfma_direct_to_lds            = sgemm_ex(..., SGEMM_ALGO_MFMA_DIRECT)
 * sgemm_ladder_name returns NULL and sgemm_ladder SGEMM_ERR_INVALID_ARG for
 * a step outside [0, sgemm_ladder_steps()). */
int sgemm_ladder_steps(void);
const char *sgemm_ladder_name(int step);
int sgemm_ladder(int step, int64_t M, int64_t N, int64_t K,
                 const float *A, int64_t lda,
                 const float *B, int64_t ldb,
                 float *C, int64_t ldc,
                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_H */
