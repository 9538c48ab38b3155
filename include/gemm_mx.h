/*
 * gemm_mx.h — block-scaled 8-bit GEMM in libgemm_bf16.so (MI355X / gfx950).
 *
 * The page "Modern GPU Programming for MLSys：深度解读" (section "背景") names low-precision
 * block-scaled GEMM among the kernel families whose speed decides training and serving.  The
 * pages give no format; this library takes the OCP microscaling (MX) one:
 *
 *   each operand element is an 8-bit float, E4M3 (1 sign, 4 exponent bits with bias 7, 3
 *   mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448) or E5M2 (bias 15, 2
 *   mantissa bits; IEEE-style infinities and NaNs; largest finite 57344), subnormals included;
 *   each run of 32 consecutive k of a row shares one scale, an unsigned 8-bit exponent e
 *   (E8M0) standing for 2^(e - 127) (e = 255 is NaN);
 *
 *   C[i][j] = sum_{k<K} (a(i,k) * 2^(sa(i, k/32) - 127)) * (b(j,k) * 2^(sb(j, k/32) - 127))
 *
 * with a(i,k) = A[i*lda + k], sa(i,q) = A_scale[i*lda_scale + q], b(j,k) = B[j*ldb + k],
 * sb(j,q) = B_scale[j*ldb_scale + q] (A is M x K and B is N x K, both K-contiguous: the GEMM
 * is C = A * B^T as for gemm_bf16), C row-major with pitch ldc, overwritten.
 *
 * Arithmetic.  The sum is accumulated in fp32.  The gfx950 scaled MFMA that the fast kernel
 * uses adds the exact products in groups of 8 consecutive k after truncating each toward zero
 * to a multiple of 2^(E - 13), where E is the largest exponent-field sum (exponents of the two
 * elements plus the two scale exponents) in the group (measured on MI355X), so the result can
 * differ from the exactly rounded sum by up to about 2^-10 of the sum of the products'
 * exponent-field magnitudes, plus the fp32 accumulation error.  Integer-valued inputs whose
 * products and partial sums stay below 2^24 are computed exactly.  Products whose scaled value
 * is outside the fp32 range give inf or lose precision; NaN inputs propagate.
 */
#ifndef GEMM_MX_H
#define GEMM_MX_H

#include <stdint.h>

#include "gemm_bf16.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats (the codes gfx950's scaled MFMA takes for them). */
#define GEMM_MX_E4M3 0
#define GEMM_MX_E5M2 1

/* Kernels of gemm_mx_variant. */
#define GEMM_MX_VARIANT_AUTO 0    /* the library chooses                                       */
#define GEMM_MX_VARIANT_SIMPLE 1  /* general kernel: any argument gemm_mx_validate accepts     */
#define GEMM_MX_VARIANT_RING 2    /* scaled-MFMA ring kernel: K % 128 == 0; A, B, A_scale,
                                     B_scale 4-byte aligned; lda, ldb, lda_scale, ldb_scale
                                     multiples of 4                                           */

/*
 * C = A * B^T in the block-scaled format above.
 *   a_format, b_format  GEMM_MX_E4M3 or GEMM_MX_E5M2 (the two operands may differ).
 *   M, N, K      >= 0, K a multiple of 32.  M == 0 or N == 0: nothing is done; K == 0: C = 0.
 *   A, lda       M x K bytes, row pitch lda >= max(K, 1) bytes.
 *   A_scale, lda_scale  M x K/32 scale bytes, row pitch lda_scale >= max(K/32, 1).
 *   B, ldb, B_scale, ldb_scale  the same for N x K.
 *   C, ldc       M x N output, row pitch ldc >= max(N, 1) elements; out_dtype GEMM_OUT_FP32 or
 *                GEMM_OUT_BF16 (round to nearest even).  C must not overlap the inputs.
 *   stream       hipStream_t or NULL.  Asynchronous; nothing is allocated; device pointers are
 *                the caller's and are not kept.
 * The scaled-MFMA kernel runs when GEMM_MX_VARIANT_RING's conditions hold, else the general
 * kernel (same results up to the summation order).
 * Returns GEMM_OK, GEMM_ERR_ARG (bad format, size, K % 32 != 0, pitch), GEMM_ERR_NULL,
 * GEMM_ERR_DTYPE, GEMM_ERR_ARCH (not gfx950) or GEMM_ERR_LAUNCH; on an error nothing is
 * launched.
 */
int gemm_mx(int a_format, int b_format, int64_t M, int64_t N, int64_t K,
            const void* A, int64_t lda, const void* A_scale, int64_t lda_scale,
            const void* B, int64_t ldb, const void* B_scale, int64_t ldb_scale,
            void* C, int64_t ldc, int out_dtype, void* stream);

/* gemm_mx with the kernel forced (GEMM_MX_VARIANT_*): GEMM_MX_VARIANT_RING on arguments it
 * cannot take returns GEMM_ERR_UNSUPPORTED; an unknown variant GEMM_ERR_ARG. */
int gemm_mx_variant(int variant, int a_format, int b_format, int64_t M, int64_t N, int64_t K,
                    const void* A, int64_t lda, const void* A_scale, int64_t lda_scale,
                    const void* B, int64_t ldb, const void* B_scale, int64_t ldb_scale,
                    void* C, int64_t ldc, int out_dtype, void* stream);

/* Host-only argument check of gemm_mx (touches no device and no pointer target). */
int gemm_mx_validate(int a_format, int b_format, int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, const void* A_scale, int64_t lda_scale,
                     const void* B, int64_t ldb, const void* B_scale, int64_t ldb_scale,
                     const void* C, int64_t ldc, int out_dtype);

/* Host-only: the kernel (see gemm_bf16_kernel_name), workgroups and threads per workgroup
 * that gemm_mx_variant(variant, ...) would launch on a device with num_cus compute units
 * (0: 256).  Pointers are used only for their alignment; output pointers may be NULL. */
int gemm_mx_plan(int variant, int a_format, int b_format, int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda, const void* A_scale, int64_t lda_scale,
                 const void* B, int64_t ldb, const void* B_scale, int64_t ldb_scale,
                 const void* C, int64_t ldc, int out_dtype, int num_cus,
                 int* kernel_id, int64_t* grid_x, int* block);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_MX_H */
