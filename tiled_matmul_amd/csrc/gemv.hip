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

// Cache policy bits of the W loads (W is streamed once).
#ifndef TMM_GEMV_AUX
#define TMM_GEMV_AUX 0
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

hipError_t launch_gemv(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    constexpr int U = TMM_GEMV_UNROLL;
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemv_kernel<OUT_F32, U>), dim3(p.grid_x), dim3(512), 0, s, g);
    else
        hipLaunchKernelGGL((gemv_kernel<OUT_BF16, U>), dim3(p.grid_x), dim3(512), 0, s, g);
    return hipGetLastError();
}

}  // namespace tmm
