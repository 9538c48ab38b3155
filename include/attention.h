/*
 * attention.h — fused attention forward in libgemm_bf16.so (MI355X / gfx950).
 *
 * The page "Modern GPU Programming for MLSys：深度解读" (its outline of the book's Part IV,
 * Flash Attention 4) and the page "Jak okiełznać Blackwella bez szaleństwa od CUDA" (section
 * "Co znajdziesz w tym samouczku") describe an attention kernel built on the GEMM of
 * gemm_bf16.h: a softmax between two matrix products, evaluated block by block with online
 * rescaling, causal masking and grouped-query attention.  Computed here:
 *
 *   S[i][j] = scale * sum_c Q[b][h][i][c] * K[b][g][j][c],    g = h / (Hq / Hkv)
 *   S[i][j] = -inf where causal and j > i + (Lk - Lq)   (the mask's diagonal ends at the
 *             last query and the last key: for Lq == Lk, key j <= query i)
 *   O[b][h][i][:] = sum_j softmax_j(S[i][j]) * V[b][g][j][:]
 *   LSE[b][h][i]  = log(sum_j exp(S[i][j]))   (natural log; -inf for a row with no key)
 *
 * Q is B x Hq x Lq x d, K and V are B x Hkv x Lk x d, O is B x Hq x Lq x d: contiguous,
 * row-major (the head dimension d innermost), bf16 inputs; O fp32 or bf16 (round to nearest
 * even); LSE fp32 (may be NULL).  Scores and sums in fp32; the probabilities are rounded to
 * bf16 for the second product.  A row with no allowed key gets O = 0.  Nothing is allocated;
 * the call is asynchronous on `stream`; pointers are the caller's device memory.
 */
#ifndef TMM_ATTENTION_H
#define TMM_ATTENTION_H

#include <stdint.h>

#include "gemm_bf16.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VARIANT_AUTO 0    /* the library chooses                                        */
#define ATTN_VARIANT_SIMPLE 1  /* one wave per query row, 64 keys per step (any d <= 256,
                                  d % 8 == 0)                                                */
#define ATTN_VARIANT_MFMA 2    /* MFMA tiles of queries x keys, online softmax in registers
                                  (d = 64 or 128; scale > 0; Q, K, V, O 16-byte aligned)     */
#define ATTN_VARIANT_PIPE 3    /* the same tiles, the next key block's score MFMAs issued
                                  during this block's softmax (same preconditions)           */

/*
 * The attention forward above.
 *   B, Hq, Hkv   >= 1 (B, Hq <= 65535), Hq a multiple of Hkv.
 *   Lq, Lk       >= 0.  Lq == 0: nothing is done; Lk == 0: every row is empty.
 *   d            head dimension, 8 <= d <= 256, d % 8 == 0.
 *   scale        multiplies the scores (1/sqrt(d) for the usual attention).
 *   causal       0 or 1.
 *   out_dtype    GEMM_OUT_FP32 or GEMM_OUT_BF16 (type of O).
 * Returns GEMM_OK, GEMM_ERR_ARG (a size out of range, Hq % Hkv != 0, causal not 0/1, a
 * non-finite scale), GEMM_ERR_NULL (Q, K, V or O NULL with work to do), GEMM_ERR_DTYPE,
 * GEMM_ERR_ARCH or GEMM_ERR_LAUNCH; nothing is launched on an error.
 */
int attention_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                  const void* Q, const void* K, const void* V, void* O, float* LSE,
                  float scale, int causal, int out_dtype, void* stream);

/* attention_fwd with the kernel forced (ATTN_VARIANT_*); a variant that cannot take the
 * arguments returns GEMM_ERR_UNSUPPORTED, an unknown one GEMM_ERR_ARG. */
int attention_fwd_variant(int variant, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                          int64_t Lk, int64_t d, const void* Q, const void* K, const void* V,
                          void* O, float* LSE, float scale, int causal, int out_dtype,
                          void* stream);

/* Host-only argument check of attention_fwd (no device, no pointer target touched). */
int attention_fwd_validate(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                           int64_t d, const void* Q, const void* K, const void* V,
                           const void* O, float scale, int causal, int out_dtype);

/* Host-only: kernel (gemm_bf16_kernel_name), workgroups and threads per workgroup of
 * attention_fwd_variant(variant, ...) on a device with num_cus compute units (0: 256). */
int attention_fwd_plan(int variant, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                       int64_t Lk, int64_t d, const void* Q, const void* K, const void* V,
                       const void* O, float scale, int causal, int out_dtype, int num_cus,
                       int* kernel_id, int64_t* grid_x, int* block);

#ifdef __cplusplus
}
#endif

#endif /* TMM_ATTENTION_H */
