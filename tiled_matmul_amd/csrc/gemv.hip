// Skinny-M GEMM (decode GEMV): C (M x N) = X (M x K) * W^T, W (N x K) bf16 K-contiguous,
// M <= 16.  Ladder step 6.
//
// The page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "Roofline", places a
// 1 x 4096 x 4096 decode at about one FLOP per byte, far below the ridge, so the kernel is
// bound by reading W once from HBM; the only goal is to stream W at full bandwidth.
//
// Design: workgroup = 8 waves, one per 16 rows of W (a 16-row block of C columns).  The 8
// waves interleave over the K axis in 32-wide steps (wave w takes steps w, w+8, ...), so the
// workgroup sweeps each W row front to back with all of its loads in flight at once: every
// wave issues UNROLL 16-byte loads per lane (UNROLL KB of W) before it consumes any.  The
// contraction of a step is one v_mfma_f32_16x16x32_bf16 with the W block as the first
// operand and X (rows m >= M read as zero) as the second, so the MFMA does the 16-row dot
// products; X is tiny and is served by the caches.  The 8 partial 16 x 16 results are summed
// through LDS.
//
// Preconditions checked by the planner: M <= 16, K % 8 == 0, ldb (W pitch) and lda (X pitch)
// multiples of 8, X and W 16-byte aligned, 16 * ldb * 2 and 16 * lda * 2 below 2^31.
#include "launch.hpp"

namespace tmm {

// Cache policy bits of the W loads: 2 = non-temporal (W is streamed once; measured 4-8%
// faster than the default policy on a cold 32 MiB W).
#ifndef TMM_GEMV_AUX
#define TMM_GEMV_AUX 2
#endif

template <int OUT, int UNROLL>
__global__ __launch_bounds__(512) void gemv_kernel(GemmArgs g) {
    constexpr int WAVES = 8;
    __shared__ f32x4 red[WAVES][64];
    const int lane = lane_id(), w = wave_id();
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t rows_w = min<int64_t>(16, g.N - n0);

    const auto rw = make_rsrc(g.B + n0 * g.ldb, static_cast<uint32_t>(((rows_w - 1) * g.ldb + g.K) * 2));
    const auto rx = make_rsrc(g.A, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));
    // Lane l supplies row (l % 16) and k chunk (l / 16) of each 16 x 32 step.
    const int r = lane & 15, c = lane >> 4;
    const uint32_t vw = r < rows_w ? static_cast<uint32_t>(r * g.ldb * 2 + c * 16) : OOB;
    const uint32_t vx = r < g.M ? static_cast<uint32_t>(r * g.lda * 2 + c * 16) : OOB;
    const uint32_t K = static_cast<uint32_t>(g.K);
    const int steps = static_cast<int>((g.K + 31) / 32);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = w; s0 < steps; s0 += WAVES * UNROLL) {
        u32x4 wv[UNROLL], xv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int s = s0 + u * WAVES;
            const uint32_t k = static_cast<uint32_t>(s) * 32u + 8u * c;   // this lane's chunk
            const bool ok = s < steps && k < K;
            wv[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? vw : OOB, 64u * s, TMM_GEMV_AUX);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int s = s0 + u * WAVES;
            const uint32_t k = static_cast<uint32_t>(s) * 32u + 8u * c;
            const bool ok = s < steps && k < K;
            xv[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? vx : OOB, 64u * s, 0);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            acc = mfma_16x16x32(__builtin_bit_cast(bf16x8, wv[u]), __builtin_bit_cast(bf16x8, xv[u]), acc);
    }

    // acc holds D[n][m] = sum over this wave's k steps; lane l, register i: m = l % 16,
    // n = 4 (l / 16) + i.  Reduce over the 8 waves.
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        f32x4 s = red[0][lane];
#pragma unroll
        for (int v = 1; v < WAVES; ++v) s += red[v][lane];
        const int64_t m = lane & 15;
        const int64_t n = n0 + 4 * (lane >> 4);
        if (m < g.M) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (n + i < g.N) {
                    if constexpr (OUT == OUT_F32)
                        static_cast<float*>(g.C)[m * g.ldc + n + i] = s[i];
                    else
                        static_cast<uint16_t*>(g.C)[m * g.ldc + n + i] = f32_to_bf16(s[i]);
                }
            }
        }
    }
}

#ifndef TMM_GEMV_UNROLL
#define TMM_GEMV_UNROLL 8
#endif

// ---------------------------------------------------------------------------------------
// Small M (M <= 8): a dot-product kernel whose every load is contiguous.  Wave w of
// workgroup b owns ROWS consecutive rows of W; in each 512-element chunk of K, lane l reads
// the 16 bytes at k = 512 j + 8 l of each of its rows (so one load instruction reads 1 KB
// of one row) and the matching 16 bytes of each row of X (served by the caches), and
// accumulates the 8 products with v_dot2c_f32_bf16 (exact bf16 products, fp32 sums).
// UNROLL chunks are in flight before any is consumed.  The 64 lane partial sums of each
// (row, m) are then added across the wave with lane shuffles.  No LDS, no barrier.
// ---------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Eight bf16 products of w and x added to acc.  (The vector elements are copied to scalars
// before the bit cast: clang's __builtin_bit_cast of a vector-element lvalue reads element 0.)
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wi = w[i], xi = x[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wi), __builtin_bit_cast(bf16x2, xi),
                                              acc, false);
    }
    return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int OUT, int MP, int ROWS, int UNROLL>
__global__ __launch_bounds__(256) void gemv_dot_kernel(GemmArgs g) {
    const int lane = lane_id(), w = wave_id();
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * 4 + w) * ROWS;
    if (n0 >= g.N) return;   // wave-uniform; the kernel has no barrier
    const int rows = static_cast<int>(min<int64_t>(ROWS, g.N - n0));
    const int M = static_cast<int>(g.M);
    const auto rw = make_rsrc(g.B + n0 * g.ldb, static_cast<uint32_t>(((rows - 1) * g.ldb + g.K) * 2));
    const auto rx = make_rsrc(g.A, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));
    const uint32_t K = static_cast<uint32_t>(g.K);
    const uint32_t ldb2 = static_cast<uint32_t>(g.ldb * 2), lda2 = static_cast<uint32_t>(g.lda * 2);

    float acc[ROWS][MP];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MP; ++m) acc[r][m] = 0.f;

    for (uint32_t c0 = 0; c0 < K; c0 += 512u * UNROLL) {
        u32x4 wv[UNROLL][ROWS], xv[UNROLL][MP];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint32_t k = c0 + 512u * u + 8u * lane;
            const bool ok = k < K;
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                wv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(
                    rw, ok && r < rows ? r * ldb2 + 2u * k : OOB, 0, TMM_GEMV_AUX);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint32_t k = c0 + 512u * u + 8u * lane;
            const bool ok = k < K;
#pragma unroll
            for (int m = 0; m < MP; ++m)
                xv[u][m] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok && m < M ? m * lda2 + 2u * k : OOB, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int m = 0; m < MP; ++m) acc[r][m] = dot8(wv[u][r], xv[u][m], acc[r][m]);
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MP; ++m) acc[r][m] = wave_sum(acc[r][m]);
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MP; ++m) {
            if (m >= M) break;
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                if (r >= rows) break;
                const int64_t off = m * g.ldc + n0 + r;
                if constexpr (OUT == OUT_F32)
                    static_cast<float*>(g.C)[off] = acc[r][m];
                else
                    static_cast<uint16_t*>(g.C)[off] = f32_to_bf16(acc[r][m]);
            }
        }
    }
}

// Rows of W per wave and 512-element K chunks in flight per wave (swept on MI355X at
// M=1, N=K=4096: 2 rows x 4 chunks was fastest, within 3% of 1-4 rows x 2-8 chunks).
#ifndef TMM_DOT_ROWS
#define TMM_DOT_ROWS 2
#endif
#ifndef TMM_DOT_UNROLL
#define TMM_DOT_UNROLL 4
#endif

template <int OUT, int MP>
static void launch_dot_mp(const GemmArgs& g, const Plan& p, hipStream_t s) {
    hipLaunchKernelGGL((gemv_dot_kernel<OUT, MP, TMM_DOT_ROWS, TMM_DOT_UNROLL>), dim3(p.grid_x), dim3(256), 0,
                       s, g);
}

template <int OUT>
static void launch_dot_out(const GemmArgs& g, const Plan& p, hipStream_t s) {
    if (g.M <= 1) launch_dot_mp<OUT, 1>(g, p, s);
    else if (g.M <= 2) launch_dot_mp<OUT, 2>(g, p, s);
    else if (g.M <= 4) launch_dot_mp<OUT, 4>(g, p, s);
    else launch_dot_mp<OUT, 8>(g, p, s);
}

hipError_t launch_gemv_dot(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    if (out == OUT_F32) launch_dot_out<OUT_F32>(g, p, s);
    else launch_dot_out<OUT_BF16>(g, p, s);
    return hipGetLastError();
}

int gemv_dot_rows_per_workgroup() { return 4 * TMM_DOT_ROWS; }

hipError_t launch_gemv(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    constexpr int U = TMM_GEMV_UNROLL;
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemv_kernel<OUT_F32, U>), dim3(p.grid_x), dim3(512), 0, s, g);
    else
        hipLaunchKernelGGL((gemv_kernel<OUT_BF16, U>), dim3(p.grid_x), dim3(512), 0, s, g);
    return hipGetLastError();
}

}  // namespace tmm
