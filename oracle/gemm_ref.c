/*
 * oracle/gemm_ref.c -- CPU oracle for the tiled bf16 GEMM.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load this
 * library.  The product path (tiled_matmul_amd/) never links or calls it, and this file
 * shares no code, header, table or helper with the HIP kernels.
 *
 * What it computes.  The GEMM that the page "读书笔记-《面向机器学习系统的现代 GPU 编程》"
 * develops in its section "9 步优化" (steps 1-3 build it, steps 4-9 only speed it up): an
 * output C of M x N, each element the sum over a contraction index k of A[i][k] * B[j][k],
 * i.e. C = A * B^T with both operands stored K-contiguous (the k-major layout named in that
 * page's section "三个核心概念：scope、layout、dispatch").  The
 * optimised kernels only change *how fast* this is computed, never *what*, so the oracle
 * is the plain definition written out:
 *
 *   step 1  decode every bf16 input (raw 16-bit pattern) to a binary64 number: the 16 bits
 *           become the high half of an IEEE binary32 word, which is then widened exactly;
 *   step 2  for each output (i, j): s = 0, m = 0; for k = 0, 1, ..., K-1 in ascending order
 *           p = a(i,k) * b(j,k);  s += p;  m += |p|;
 *           C[i][j] = s  and  Mag[i][j] = m  (Mag is (|A| |B|^T)[i][j], the quantity the
 *           acceptance bound is stated in).
 *
 * A bf16 x bf16 product has at most 16 significant bits, so p is exact in binary64; s then
 * carries only binary64 rounding error (<= (K-1) 2^-53 Mag), and is exact whenever all
 * partial sums are integers below 2^53.  Rows are distributed over OpenMP threads; within
 * one output the k order is fixed, so the result does not depend on the thread count.
 *
 * Also here: oracle_round_bf16, round-to-nearest-even of a binary64 value to bf16, used to
 * state the exact expected bf16 output of integer-valued test cases.
 *
 * Build (done by __graft_entry__.build()):
 *   gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off -o oracle/liboracle.so oracle/gemm_ref.c -lm
 * No -ffast-math: the k order and IEEE semantics of the sums must be kept.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* step 1: bf16 bit pattern -> binary64 (exact) */
static double decode_bf16(uint16_t h)
{
    uint32_t word = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* Decode a rows x cols block with leading dimension ld into a dense binary64 array. */
static void decode_matrix(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld, double* out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = decode_bf16(X[r * ld + c]);
}

int oracle_version(void) { return 1; }

/*
 * C = A * B^T in binary64, plus Mag = |A| |B|^T.
 *   A: M x K bf16 bit patterns, row pitch lda (elements); B: N x K, row pitch ldb.
 *   rows == NULL: every row i = 0..M-1 is computed and written to C[i*ldc + j].
 *   rows != NULL: only rows[0..nrows-1] (each in [0, M)) are computed; output row r of C and
 *   Mag (r = 0..nrows-1) holds row rows[r].  This is how large shapes are sampled.
 *   Mag may be NULL.  Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* B, int64_t ldb,
                     double* C, double* Mag, int64_t ldc,
                     const int64_t* rows, int64_t nrows, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || ldc < N) return -1;
    if (K > 0 && (lda < K || ldb < K)) return -1;
    int64_t nout = rows ? nrows : M;
    if (nout <= 0 || N == 0) return 0;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;

    /* step 1: decode B once, and each needed row of A once */
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(nout * (K > 0 ? K : 1)));
    if (!Bd || !Ad) { free(Bd); free(Ad); return -1; }
    if (K > 0) {
        decode_matrix(B, N, K, ldb, Bd);
        for (int64_t r = 0; r < nout; ++r) {
            int64_t i = rows ? rows[r] : r;
            decode_matrix(A + i * lda, 1, K, lda, Ad + r * K);
        }
    }

    /* step 2: the triple loop, k ascending */
    if (nthreads < 1) nthreads = 1;
    #pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (int64_t r = 0; r < nout; ++r) {
        const double* a = Ad + r * K;
        for (int64_t j = 0; j < N; ++j) {
            const double* b = Bd + j * K;
            double s = 0.0, m = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = a[k] * b[k];
                s += p;
                m += fabs(p);
            }
            C[r * ldc + j] = s;
            if (Mag) Mag[r * ldc + j] = m;
        }
    }
    free(Bd);
    free(Ad);
    return 0;
}

/*
 * Round a binary64 value to the nearest bf16 (8 significant bits, binary32 exponent range),
 * ties to even, and return its bit pattern.  Overflow goes to +-inf, NaN to a quiet NaN.
 * This is a single rounding straight from binary64.
 */
uint16_t oracle_round_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int e;
    (void)frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                    /* quantum 2^q keeps 8 significant bits */
    if (q < -133) q = -133;           /* bf16 subnormal quantum (binary32's 2^-149 << 16) */
    double scaled = ldexp(a, -q);     /* exact: only the exponent changes */
    double n = nearbyint(scaled);     /* default rounding mode: nearest, ties to even */
    double v = ldexp(n, q);
    if (v > 0x1.FEp127) return (uint16_t)(sign | 0x7F80);  /* above the largest finite bf16 */
    float vf = (float)v;              /* exact: v has <= 8 significant bits in range */
    uint32_t w;
    memcpy(&w, &vf, sizeof w);
    return (uint16_t)(sign | ((w >> 16) & 0x7FFF));
}

/* Vector form of oracle_round_bf16 over n values. */
void oracle_round_bf16_array(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

/* Vector form of step 1, exported so the decode can be pinned on its own. */
void oracle_decode_bf16_array(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode_bf16(h[i]);
}
