// The first rungs of the GEMM ladder, C = A * B^T with A (M x K) and B (N x K) bf16,
// K-contiguous, fp32 accumulation.  Both kernels load through plain per-lane global loads,
// handle any pitch and alignment (2-byte aligned operands), and mask every tail, so they
// also serve as the general fallback of the fast kernels; gemm_simple_kernel also takes
// MN-major operands (the general fallback for those layouts).
//
//   gemm_simple_kernel  -- the page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section
//                          "9 步优化", steps 1-3: one workgroup per 64 x 64 output tile of
//                          a 2-D grid, a loop over K blocks that reuses one LDS staging
//                          buffer, accumulation in place.  Arithmetic is fp32 FMA on VALU.
//   gemm_mfma_kernel    -- the same structure with the contraction on the matrix cores:
//                          v_mfma_f32_16x16x32_bf16 into a register-blocked accumulator
//                          (the page's accumulator next to the tensor core becomes VGPRs).
//                          128 x 128 tile, four waves of 64 x 64.  One LDS stage, loads
//                          are synchronous with compute (the page's step 3 state).
#include "launch.hpp"

namespace tmm {

// ---------------------------------------------------------------------------------------
// K == 0: the empty sum, C = 0.
// ---------------------------------------------------------------------------------------
template <int OUT>
__global__ __launch_bounds__(256) void zero_fill_kernel(GemmArgs g) {
    const int64_t per = g.M * g.N;
    const int64_t total = per * g.batch;
    for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += 256ll * gridDim.x) {
        int64_t b = e / per, r = e - b * per;
        int64_t m = r / g.N, n = r - m * g.N;
        int64_t off = b * g.sC + m * g.ldc + n;
        if constexpr (OUT == OUT_F32)
            static_cast<float*>(g.C)[off] = 0.0f;
        else
            static_cast<uint16_t*>(g.C)[off] = 0;
    }
}

// ---------------------------------------------------------------------------------------
// Ladder step 1: LDS-tiled, fp32 VALU.  Thread (tr, tc) owns rows tr + 16 i and columns
// tc + 16 j (i, j < 4) of the tile, so LDS reads of a k row are conflict-free broadcasts.
// ---------------------------------------------------------------------------------------
template <int OUT>
__global__ __launch_bounds__(256) void gemm_simple_kernel(GemmArgs g) {
    constexpr int T = 64, BK = 32;
    __shared__ float As[BK][T + 1];
    __shared__ float Bs[BK][T + 1];
    const int64_t b = blockIdx.z;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * T, n0 = static_cast<int64_t>(blockIdx.x) * T;
    const uint16_t* A = g.A + b * g.sA;
    const uint16_t* B = g.B + b * g.sB;
    const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
        // Consecutive threads walk the contiguous direction of each operand: k for a
        // K-major operand, m (n) for an MN-major one.
#pragma unroll
        for (int i = 0; i < (T * BK) / 256; ++i) {
            const int e = tid + 256 * i;
            {
                const int r = g.la == LAYOUT_K ? e / BK : e % T, kk = g.la == LAYOUT_K ? e % BK : e / T;
                const int64_t gk = k0 + kk, gm = m0 + r;
                const int64_t off = g.la == LAYOUT_K ? gm * g.lda + gk : gk * g.lda + gm;
                As[kk][r] = (gm < g.M && gk < g.K) ? bf16_to_f32(A[off]) : 0.0f;
            }
            {
                const int r = g.lb == LAYOUT_K ? e / BK : e % T, kk = g.lb == LAYOUT_K ? e % BK : e / T;
                const int64_t gk = k0 + kk, gn = n0 + r;
                const int64_t off = g.lb == LAYOUT_K ? gn * g.ldb + gk : gk * g.ldb + gn;
                Bs[kk][r] = (gn < g.N && gk < g.K) ? bf16_to_f32(B[off]) : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][tr + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tc + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + tr + 16 * i;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tc + 16 * j;
            if (n >= g.N) continue;
            const int64_t off = b * g.sC + m * g.ldc + n;
            if constexpr (OUT == OUT_F32)
                static_cast<float*>(g.C)[off] = acc[i][j];
            else
                static_cast<uint16_t*>(g.C)[off] = f32_to_bf16(acc[i][j]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Ladder step 3 (MFMA inner loop), single LDS stage.  LDS rows are padded to 80 bytes so
// that the 16-byte fragment reads of 8 consecutive rows land in 8 distinct bank groups.
// VEC: elements per global load (8, 4, 2 or 1); the planner picks the widest that the
// operands' alignment, pitches and K allow, so a VEC chunk is either wholly inside K or
// wholly outside it.
// ---------------------------------------------------------------------------------------
template <int VEC>
struct VecLoad;
template <> struct VecLoad<8> { typedef u32x4 T; };
template <> struct VecLoad<4> { typedef u32x2 T; };
template <> struct VecLoad<2> { typedef uint32_t T; };
template <> struct VecLoad<1> { typedef uint16_t T; };

template <int OUT, int VEC>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs g, int vec_store) {
    constexpr int T = 128, BK = 32, PITCH = BK + 8;   // elements per LDS row (80 bytes)
    constexpr int WT = 64, F = WT / 16;               // wave tile and fragments per side
    typedef typename VecLoad<VEC>::T VT;
    __shared__ __attribute__((aligned(16))) uint16_t As[T * PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[T * PITCH];

    const int64_t b = blockIdx.z;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * T, n0 = static_cast<int64_t>(blockIdx.x) * T;
    const uint16_t* A = g.A + b * g.sA;
    const uint16_t* B = g.B + b * g.sB;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int wm = w >> 1, wn = w & 1;

    f32x4 acc[F][F];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragment read offsets: row (lane % 16) of a 16-row block, k chunk (lane / 16).
    const int rd = (lane & 15) * PITCH + 8 * (lane >> 4);

    for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
        constexpr int CHUNKS = T * BK / VEC;          // per operand
#pragma unroll
        for (int i = 0; i < CHUNKS / 256; ++i) {
            const int e = (tid + 256 * i) * VEC, r = e / BK, kk = e % BK;
            const int64_t gk = k0 + kk;
            VT va{}, vb{};
            if (m0 + r < g.M && gk < g.K)
                va = *reinterpret_cast<const VT*>(A + (m0 + r) * g.lda + gk);
            if (n0 + r < g.N && gk < g.K)
                vb = *reinterpret_cast<const VT*>(B + (n0 + r) * g.ldb + gk);
            *reinterpret_cast<VT*>(As + r * PITCH + kk) = va;
            *reinterpret_cast<VT*>(Bs + r * PITCH + kk) = vb;
        }
        __syncthreads();
        bf16x8 fb[F], fa[F];
#pragma unroll
        for (int i = 0; i < F; ++i) {
            fb[i] = *reinterpret_cast<const bf16x8*>(Bs + (wn * WT + 16 * i) * PITCH + rd);
            fa[i] = *reinterpret_cast<const bf16x8*>(As + (wm * WT + 16 * i) * PITCH + rd);
        }
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
            for (int j = 0; j < F; ++j) acc[i][j] = mfma_16x16x32(fb[i], fa[j], acc[i][j]);
        __syncthreads();
    }
    void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + b * g.sC)
                              : static_cast<void*>(static_cast<uint16_t*>(g.C) + b * g.sC);
    store_acc<OUT, F, F>(Cb, g.ldc, g.M, g.N, m0 + wm * WT, n0 + wn * WT, acc, vec_store != 0);
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_zero_fill(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    if (out == OUT_F32)
        hipLaunchKernelGGL(zero_fill_kernel<OUT_F32>, dim3(p.grid_x), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL(zero_fill_kernel<OUT_BF16>, dim3(p.grid_x), dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_simple(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z);
    if (out == OUT_F32)
        hipLaunchKernelGGL(gemm_simple_kernel<OUT_F32>, grid, dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL(gemm_simple_kernel<OUT_BF16>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

template <int OUT>
static hipError_t launch_mfma_out(const GemmArgs& g, const Plan& p, hipStream_t s) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z);
    switch (p.vec) {
        case 8: hipLaunchKernelGGL((gemm_mfma_kernel<OUT, 8>), grid, dim3(256), 0, s, g, p.vec_store); break;
        case 4: hipLaunchKernelGGL((gemm_mfma_kernel<OUT, 4>), grid, dim3(256), 0, s, g, p.vec_store); break;
        case 2: hipLaunchKernelGGL((gemm_mfma_kernel<OUT, 2>), grid, dim3(256), 0, s, g, p.vec_store); break;
        default: hipLaunchKernelGGL((gemm_mfma_kernel<OUT, 1>), grid, dim3(256), 0, s, g, p.vec_store); break;
    }
    return hipGetLastError();
}

hipError_t launch_mfma(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    return out == OUT_F32 ? launch_mfma_out<OUT_F32>(g, p, s) : launch_mfma_out<OUT_BF16>(g, p, s);
}

}  // namespace tmm
