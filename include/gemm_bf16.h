/*
 * gemm_bf16.h -- C ABI of libgemm_bf16.so, a tiled bf16 GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation is the matrix product that the page "读书笔记-《面向机器学习系统的现代 GPU
 * 编程》" builds in its section "9 步优化" (steps 1-3 define it: output tiles, a loop over K
 * blocks accumulating into one fp32 accumulator, a 2-D grid of tiles; steps 4-9 only make it
 * faster), with both operands in the k-major layout named in that page's section
 * "三个核心概念：scope、layout、dispatch":
 *
 *     C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[j*ldb + k]      0 <= i < M, 0 <= j < N
 *
 * i.e. C = A * B^T with A (M x K) and B (N x K) row-major bf16, each product exact and the
 * sum accumulated in fp32; C (M x N, row-major) is OVERWRITTEN (no alpha/beta).  The order
 * of the fp32 additions is not specified, but it is fixed, so repeated calls with the same
 * arguments give bitwise identical results (gemm_bf16_splitk and gemm_bf16_streamk, which cut
 * K across workgroups, add the pieces in a fixed order too).
 *
 * Memory and ownership.  A, B and C are device pointers (e.g. from hipMalloc or a torch
 * tensor's data_ptr() on ROCm) owned by the caller; the library keeps no pointer after a call
 * returns and allocates no memory in any call.  bf16 values are raw 16-bit patterns
 * (uint16_t).  Pitches (lda, ldb, ldc) and batch strides are in ELEMENTS.  A and B must be
 * 2-byte aligned, C 4-byte (fp32 out) or 2-byte (bf16 out) aligned; 4-byte aligned operands
 * with even pitches (and strides) take the fast kernels, any K; anything else a slower
 * general kernel with the same result semantics.  C must not overlap A or B.
 *
 * Streams.  `stream` is a hipStream_t passed as void*; NULL is the default stream.  Calls are
 * asynchronous: they enqueue kernels and return.  A device fault surfaces at the caller's
 * next synchronisation, not in the return value.
 *
 * Errors.  Every function returns GEMM_OK (0) or a GEMM_ERR_* code; argument errors are
 * detected on the host before anything is enqueued, and nothing is written then.  No C++
 * exception crosses this interface.  gemm_bf16_status_string() names a code.
 */
#ifndef GEMM_BF16_H
#define GEMM_BF16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GEMM_OK 0
#define GEMM_ERR_ARG 1         /* negative size, pitch < required, bad stride or variant  */
#define GEMM_ERR_NULL 2        /* NULL pointer for an operand with a nonzero extent        */
#define GEMM_ERR_DTYPE 3       /* out_dtype is not GEMM_OUT_FP32 or GEMM_OUT_BF16          */
#define GEMM_ERR_ARCH 4        /* current device is not gfx950, or no device               */
#define GEMM_ERR_LAUNCH 5      /* the HIP runtime rejected the kernel launch              */
#define GEMM_ERR_UNSUPPORTED 6 /* the requested variant cannot run these arguments         */
#define GEMM_ERR_SCRATCH 7     /* the call needs more than the library's static scratch    */

/* Output element types. */
#define GEMM_OUT_FP32 0        /* C is float                                              */
#define GEMM_OUT_BF16 1        /* C is bf16, rounded to nearest even from the fp32 sum   */

/* Kernel variants (gemm_bf16_variant): the rungs of the page's nine-step ladder as built
 * for gfx950.  GEMM_VARIANT_AUTO is what gemm_bf16 uses. */
#define GEMM_VARIANT_AUTO 0
#define GEMM_VARIANT_SIMPLE 1      /* steps 1-3: LDS-tiled 64x64, K loop, 2-D grid, fp32 VALU */
#define GEMM_VARIANT_MFMA 2        /* MFMA register-blocked accumulators, one LDS stage       */
#define GEMM_VARIANT_PIPELINED 3   /* steps 4-5: direct-to-LDS swizzled multi-stage ring       */
#define GEMM_VARIANT_PERSISTENT 4  /* step 6: + persistent workgroups, XCD-aware tile order    */
#define GEMM_VARIANT_SPECIALIZED 5 /* steps 7-9: producer/consumer waves sharing the B tile    */
#define GEMM_VARIANT_GEMV 6        /* skinny M (M <= 16): bandwidth-bound decode path         */
#define GEMM_VARIANT_PINGPONG 7    /* steps 7-9: two wave groups alternate load / MFMA phases  */
#define GEMM_VARIANT_RING8 8       /* steps 4-6, separate A and B rings, loads spread, 8 waves */
#define GEMM_VARIANT_RING4 9       /* the same with 4 waves of 128x128 register tiles          */
#define GEMM_VARIANT_DTV 10        /* ring4's tile with A loaded into MFMA registers, B in LDS */
#define GEMM_VARIANT_ROLES 11      /* step 7 with fixed roles: 4 load-only, 4 MFMA-only waves  */

/* Operand layouts (gemm_bf16_layout).  The page "读书笔记-《面向机器学习系统的现代 GPU
 * 编程》", section "三个核心概念：scope、layout、dispatch", names the two ways a GEMM
 * operand can be stored: contiguous along the reduction dimension (k-major) or along the
 * output dimension (mn-major).
 *   GEMM_LAYOUT_K_MAJOR   A(i, k) = A[i * lda + k] (A is M x K), B(j, k) = B[j * ldb + k]
 *                         (B is N x K): pitch >= K.  What every other entry point takes.
 *   GEMM_LAYOUT_MN_MAJOR  A(i, k) = A[k * lda + i] (A is stored K x M, pitch >= M),
 *                         B(j, k) = B[k * ldb + j] (B stored K x N, pitch >= N): with an
 *                         MN-major B, C = A * B for a row-major K x N matrix B. */
#define GEMM_LAYOUT_K_MAJOR 0
#define GEMM_LAYOUT_MN_MAJOR 1

/*
 * C = A * B^T for one problem (definition above).
 *   M, N, K      >= 0.  M == 0 or N == 0: nothing is done.  K == 0: C is set to zero (the
 *                empty sum).
 *   A, lda       M x K bf16, row pitch lda >= max(K, 1).
 *   B, ldb       N x K bf16, row pitch ldb >= max(K, 1).
 *   C, ldc       M x N output, row pitch ldc >= max(N, 1); element type from out_dtype.
 *   out_dtype    GEMM_OUT_FP32 or GEMM_OUT_BF16.
 *   stream       hipStream_t or NULL.
 * Returns GEMM_OK or GEMM_ERR_{ARG,NULL,DTYPE,ARCH,LAUNCH}.
 */
int gemm_bf16(int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda,
              const void* B, int64_t ldb,
              void* C, int64_t ldc,
              int out_dtype, void* stream);

/*
 * `batch` independent problems of one shape: item b uses A + b*strideA, B + b*strideB and
 * C + b*strideC (strides in elements, >= 0; A or B may be shared with stride 0).  Output
 * items must not overlap: strideC >= (M-1)*ldc + N when batch > 1.  The whole batch is one
 * launch whose tile scheduler enumerates (item, tile row, tile column).
 * batch <= 65535.  Other arguments and errors as gemm_bf16.
 */
int gemm_bf16_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, int64_t strideA,
                              const void* B, int64_t ldb, int64_t strideB,
                              void* C, int64_t ldc, int64_t strideC,
                              int out_dtype, void* stream);

/*
 * As gemm_bf16_strided_batched, forcing one GEMM_VARIANT_* kernel (for ablations and the
 * measurements of each rung).  A variant whose preconditions the arguments do not meet
 * (GEMV with M > 16, or with A, B not 16-byte aligned or lda, ldb, K not multiples of 8;
 * the pipelined, persistent and specialized variants need 4-byte aligned A and B and even
 * lda, ldb and strides; the ping-pong and DTV variants 16-byte aligned A and B and lda, ldb,
 * strides and K multiples of 8) returns GEMM_ERR_UNSUPPORTED and does nothing.
 * An unknown variant returns GEMM_ERR_ARG.
 */
int gemm_bf16_variant(int variant, int64_t batch, int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, int64_t strideA,
                      const void* B, int64_t ldb, int64_t strideB,
                      void* C, int64_t ldc, int64_t strideC,
                      int out_dtype, void* stream);

/*
 * Host-only argument check of gemm_bf16_strided_batched (pass batch = 1 and zero strides
 * for a single problem).  Touches no device and no pointer target: usable without a GPU.
 * Returns GEMM_OK or GEMM_ERR_{ARG,NULL,DTYPE}.
 */
int gemm_bf16_validate(int64_t batch, int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, int64_t strideA,
                       const void* B, int64_t ldb, int64_t strideB,
                       const void* C, int64_t ldc, int64_t strideC,
                       int out_dtype);

/*
 * Host-only: the kernel gemm_bf16_variant(variant, ...) would launch for these arguments
 * on a device with `num_cus` compute units (pass 0 for the MI355X's 256), and its launch
 * shape.  Pointers are used only for their alignment.  On success *kernel_id receives a
 * kernel id (see gemm_bf16_kernel_name), *grid_x the number of workgroups and *block the
 * threads per workgroup; any output pointer may be NULL.  Returns the status the call would
 * return before launching.
 */
int gemm_bf16_plan(int variant, int64_t batch, int64_t M, int64_t N, int64_t K,
                   const void* A, int64_t lda, int64_t strideA,
                   const void* B, int64_t ldb, int64_t strideB,
                   const void* C, int64_t ldc, int64_t strideC,
                   int out_dtype, int num_cus,
                   int* kernel_id, int64_t* grid_x, int* block);

/*
 * C[i][j] = sum_k A(i, k) * B(j, k) with each operand in the layout a_layout / b_layout
 * (GEMM_LAYOUT_*), through kernel variant `variant` (GEMM_VARIANT_AUTO to let the library
 * choose); otherwise as gemm_bf16_variant: same pointers, strides, output, streams and
 * status codes, C row-major with pitch ldc, batch items strideA / strideB / strideC
 * elements apart.  With both layouts K-major this is gemm_bf16_variant.  With an MN-major
 * operand, AUTO runs the ring kernel (4 waves, 256 x 256 tiles) when A and B are 4-byte
 * aligned with even pitches and strides and the MN-major operand's extent (M for A, N for
 * B) is a multiple of 8, and the general 64 x 64 kernel otherwise; of the forced variants
 * only GEMM_VARIANT_SIMPLE and GEMM_VARIANT_RING4 accept MN-major operands (others return
 * GEMM_ERR_UNSUPPORTED).  An unknown layout returns GEMM_ERR_ARG.
 */
int gemm_bf16_layout(int a_layout, int b_layout, int variant, int64_t batch,
                     int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, int64_t strideA,
                     const void* B, int64_t ldb, int64_t strideB,
                     void* C, int64_t ldc, int64_t strideC,
                     int out_dtype, void* stream);

/* gemm_bf16_validate for gemm_bf16_layout's arguments (host-only). */
int gemm_bf16_layout_validate(int a_layout, int b_layout, int64_t batch,
                              int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, int64_t strideA,
                              const void* B, int64_t ldb, int64_t strideB,
                              const void* C, int64_t ldc, int64_t strideC,
                              int out_dtype);

/* gemm_bf16_plan for gemm_bf16_layout's arguments (host-only). */
int gemm_bf16_layout_plan(int a_layout, int b_layout, int variant, int64_t batch,
                          int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda, int64_t strideA,
                          const void* B, int64_t ldb, int64_t strideB,
                          const void* C, int64_t ldc, int64_t strideC,
                          int out_dtype, int num_cus,
                          int* kernel_id, int64_t* grid_x, int* block);

/*
 * Split K (for problems with too few output tiles to fill the device, but a long K).  The
 * page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "9 步优化", builds the
 * output of one tile as the sum over the K blocks of their partial products (step 2) and
 * hands tiles to a fixed pool of persistent workgroups (step 6).  Here a work item of that
 * pool is (tile, K range): the K blocks of 64 are cut into `S` contiguous ranges; each work
 * item writes its range's fp32 partial sum to the workspace, and a second kernel adds the S
 * partials of each element in range order (0, 1, ..., S-1) and rounds once to out_dtype.
 * The result is deterministic (the same bits on every run with the same S) and differs from
 * gemm_bf16_layout only in the order of the fp32 additions.
 *   splits           S >= 1 to force (capped at the number of K blocks, ceil(K / 64)), or 0
 *                    to let the library choose.  Automatic S: 1 unless the call would run
 *                    a tiled MFMA kernel (not the skinny-M path) whose tiles cover at most
 *                    half of the compute units; then S = min(CUs / T, floor(nk / 8),
 *                    floor(workspace_bytes / (batch * M * N * 4))), at least 1, where T is
 *                    the number of 256 x 256 tiles (batch included) and nk = ceil(K / 64):
 *                    one work item per compute unit, at least 8 K blocks per range, and no
 *                    more ranges than the workspace holds.
 *   workspace        device memory owned by the caller, 16-byte aligned, at least
 *                    S * batch * M * N * 4 bytes (see gemm_bf16_splitk_plan for S); only
 *                    used, and may be NULL, when S == 1.  Its contents on entry do not
 *                    matter; it is scratch until the call's work on `stream` completes, so
 *                    calls that share a workspace must be ordered on one stream.
 *   workspace_bytes  its size in bytes.
 * Other arguments as gemm_bf16_layout (every layout).  When S == 1 the call is exactly
 * gemm_bf16_layout(a_layout, b_layout, GEMM_VARIANT_AUTO, ...).  When S > 1 it runs the
 * 4-wave ring kernel, which needs what that kernel needs with the layouts given (4-byte
 * aligned A and B, even pitches and strides; an MN-major extent a multiple of 8): if these
 * do not hold, an explicit splits > 1 returns GEMM_ERR_UNSUPPORTED and splits == 0 falls
 * back to S = 1.  A workspace that is too small or misaligned returns GEMM_ERR_ARG (NULL:
 * GEMM_ERR_NULL); splits < 0 or workspace_bytes < 0: GEMM_ERR_ARG.  Nothing is launched on
 * an error.
 */
int gemm_bf16_splitk(int a_layout, int b_layout, int splits, int64_t batch,
                     int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, int64_t strideA,
                     const void* B, int64_t ldb, int64_t strideB,
                     void* C, int64_t ldc, int64_t strideC,
                     int out_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Host-only plan of gemm_bf16_splitk on a device with `num_cus` compute units (0: 256):
 * *splits_out receives S, *kernel_id the kernel of the first launch and *grid_x its
 * workgroups.  To size a workspace, pass workspace_bytes = INT64_MAX with a non-NULL
 * 16-byte aligned workspace pointer and allocate S * batch * M * N * 4 bytes.  Returns the
 * status gemm_bf16_splitk would return before launching.  Output pointers may be NULL.
 */
int gemm_bf16_splitk_plan(int a_layout, int b_layout, int splits, int64_t batch,
                          int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda, int64_t strideA,
                          const void* B, int64_t ldb, int64_t strideB,
                          const void* C, int64_t ldc, int64_t strideC,
                          int out_dtype, const void* workspace, int64_t workspace_bytes,
                          int num_cus, int* splits_out, int* kernel_id, int64_t* grid_x);

/*
 * Stream-K with atomic work claiming.  The page "读书笔记-《面向机器学习系统的现代 GPU 编程》"
 * hands tiles to persistent workgroups from a scheduler ("9 步优化", step 6) and names atomics
 * as the means for counters and tile claiming ("同步的本质").  Here the 256 x 256 tiles of the
 * 4-wave ring kernel are the work of one persistent workgroup per compute unit, handed out by an
 * atomic counter in the workspace: whole tiles first, then, for the last tiles, stream-K slots
 * of about I / G (tile, K block) iterations each (I the iterations of those tiles, G the
 * workgroups), which cut the tiles along K so that the workgroups end together.  A tile cut
 * into several pieces is summed by whichever piece finishes last: the others write their fp32
 * partials to the workspace, and the last adds them and its own in a fixed order (the pieces'
 * order along K).  The result is deterministic (bitwise the same on every run with the same
 * arguments and device), and differs from gemm_bf16 only in the order of the fp32 additions of
 * the cut tiles.  No workgroup waits for one that has not started: the last piece waits only
 * for pieces that have finished their K loop and have their stores left.  (That wait is bounded;
 * past a limit no such wait reaches, the piece writes its quarter of C as NaN so that a failure
 * shows, and the workspace's counters must then be cleared before it is used again.)
 *   mode   GEMM_STREAMK_AUTO: when there are more tiles than compute units and they do not
 *          divide evenly, stream-K for the last, partly filled wave and the full wave before it;
 *          otherwise whole tiles only.
 *          GEMM_STREAMK_DP: whole tiles only (claimed atomically).  GEMM_STREAMK_ALL: as AUTO,
 *          and with fewer tiles than compute units every tile is cut.
 *   workspace, workspace_bytes  device memory owned by the caller, 256-byte aligned, at least
 *          the size gemm_bf16_streamk_plan returns: 16 KB of counters, then the partials.  The
 *          16 KB of counters must be zero before the first call on a workspace (e.g. hipMemset
 *          once); every call leaves them zero again.  Calls that share a workspace must be
 *          ordered on one stream.
 * Other arguments as gemm_bf16_strided_batched; both operands K-major, 4-byte aligned with even
 * pitches and strides (else GEMM_ERR_UNSUPPORTED).  K == 0 zero-fills C (no workspace used).
 * A workspace that is too small or misaligned: GEMM_ERR_ARG; NULL: GEMM_ERR_NULL.
 */
#define GEMM_STREAMK_AUTO 0
#define GEMM_STREAMK_DP 1
#define GEMM_STREAMK_ALL 2
int gemm_bf16_streamk(int mode, int64_t batch, int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, int64_t strideA,
                      const void* B, int64_t ldb, int64_t strideB,
                      void* C, int64_t ldc, int64_t strideC,
                      int out_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Host-only plan of gemm_bf16_streamk on a device with `num_cus` compute units (0: 256): the
 * workspace size it needs, the tiles computed whole (*dp_tiles) and cut (*sk_tiles), the
 * stream-K slots and the workgroups launched.  Output pointers may be NULL.
 */
int gemm_bf16_streamk_plan(int mode, int64_t batch, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, int64_t strideA,
                           const void* B, int64_t ldb, int64_t strideB,
                           const void* C, int64_t ldc, int64_t strideC,
                           int out_dtype, int num_cus, int64_t* workspace_bytes,
                           int* dp_tiles, int* sk_tiles, int* sk_slots, int64_t* grid_x);

/*
 * gemm_bf16_splitk without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the fp32 partials go to a scratch array the library holds in device memory,
 * GEMM_SCRATCH_BYTES per device, reserved when the library is loaded and kept until the
 * process ends.  Nothing is allocated or freed in the call.
 *   splits   as gemm_bf16_splitk; with 0 the automatic count is limited to what the scratch
 *            holds.  An explicit count whose partials (S * batch * M * N * 4 bytes, S capped
 *            at ceil(K / 64)) exceed GEMM_SCRATCH_BYTES returns GEMM_ERR_SCRATCH and launches
 *            nothing.
 * Other arguments, results and errors as gemm_bf16_splitk; the result is bitwise that of
 * gemm_bf16_splitk with the same S.  Every call on one device uses that device's one scratch
 * array, and each call writes every partial it reads (nothing needs to start at zero), but
 * calls that overlap in time on one device race: order them on one stream.
 */
#define GEMM_SCRATCH_BYTES (64ll << 20)
int gemm_bf16_splitk_noalloc(int a_layout, int b_layout, int splits, int64_t batch,
                             int64_t M, int64_t N, int64_t K,
                             const void* A, int64_t lda, int64_t strideA,
                             const void* B, int64_t ldb, int64_t strideB,
                             void* C, int64_t ldc, int64_t strideC,
                             int out_dtype, void* stream);

/* Name of a kernel id from gemm_bf16_plan ("?" if unknown).  Static storage. */
const char* gemm_bf16_kernel_name(int kernel_id);

/* Human-readable name of a status code.  Static storage. */
const char* gemm_bf16_status_string(int status);

/* Library interface version (incremented on any change to this header). */
int gemm_bf16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BF16_H */
