// Skinny-M GEMM (decode GEMV): C (M x N) = X (M x K) * W^T, W (N x K) bf16 K-contiguous,
// M <= 16.  Ladder step 6.
//
// The page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "Roofline", places a
// 1 x 4096 x 4096 decode at about one FLOP per byte, far below the ridge, so the kernel is
// bound by reading W once from HBM; the only goal is to stream W at full bandwidth.  Every
// workgroup needs all of X, so X is staged once per workgroup in LDS: read from global
// memory per step instead, it doubles the traffic through the load units (measured: a W
// stream that takes 7.8 us takes 11.8 us with X fragments loaded beside it).
//
// Two forms (the planner picks by M):
//   * MFMA form (gemv_kernel): workgroup = 8 waves, one 16-row block of W.  The waves
//     interleave over K in 32-wide steps (wave w takes steps w, w+8, ...) with all their W
//     loads in flight at once; each step is one v_mfma_f32_16x16x32_bf16 with the W block as
//     the first operand and the X fragment (from LDS) as the second.  The 8 partial 16 x 16
//     results are summed through LDS.
//   * dot-product form (gemv_lds_kernel): contiguous 1 KB loads of single W rows, products
//     on the VALU; fastest for the smallest M.
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

template <int OUT, int UNROLL, bool PAIRS>
__global__ __launch_bounds__(512) void gemv_kernel(GemmArgs g) {
    static_assert(!PAIRS || UNROLL % 2 == 0, "pairs of steps");
    constexpr int WAVES = 8, KX = 4096;
    constexpr int XST = KX * 2 + 16;   // LDS pitch of a row of X: 16 bytes of padding move
                                       // each row 4 banks, so a fragment read is conflict-free
    __shared__ __attribute__((aligned(1024))) uint8_t xs[16 * XST];
    __shared__ f32x4 red[WAVES][64];
    const int lane = lane_id(), w = wave_id();
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t rows_w = min<int64_t>(16, g.N - n0);
    const int M = static_cast<int>(g.M);

    const auto rw = make_rsrc(g.B + n0 * g.ldb, static_cast<uint32_t>(((rows_w - 1) * g.ldb + g.K) * 2));
    const auto rx = make_rsrc(g.A, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));
    // Lane l supplies row (l % 16) and k chunk (l / 16) of each 16 x 32 step.
    const int r = lane & 15, c = lane >> 4;
    const uint32_t vw = r < rows_w ? static_cast<uint32_t>(r * g.ldb * 2 + c * 16) : OOB;
    const uint32_t K = static_cast<uint32_t>(g.K), lda2 = static_cast<uint32_t>(g.lda * 2);
    const uint8_t* xfrag = xs + r * XST + c * 16;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    constexpr int CH = KX / 512;
    for (uint32_t k0 = 0; k0 < K; k0 += KX) {
        if (k0 > 0) barrier();   // every wave is done with the previous phase of X
        // X rows 0..15 of this phase, 1 KB per load; rows >= M and columns >= K land as zeros.
        static_assert((16 * CH) % WAVES == 0, "X loads split evenly over the waves");
#pragma unroll
        for (int i = 0; i < 16 * CH / WAVES; ++i) {
            const int q = w + i * WAVES, m = q / CH, j = q % CH;
            const uint32_t k = k0 + 512u * j + 8u * lane;
            load_lds_16(rx, xs + m * XST + j * 1024, m < M && k < K ? m * lda2 + 2u * k : OOB, 0);
        }
        asm volatile("" ::: "memory");   // the W loads below stay behind the X loads
        const int steps = static_cast<int>((min(K - k0, static_cast<uint32_t>(KX)) + 31) / 32);
        u32x4 wv[UNROLL];
        // k step of load u of the group starting at s0 (= w + i WAVES UNROLL): with PAIRS,
        // steps 2 j and 2 j + 1 (the two halves of each 128-byte line of a W row) go to one
        // wave back to back; otherwise the waves take steps in turn.
        auto step_of = [&](int s0, int u) {
            if constexpr (PAIRS) return (s0 - w) + 2 * (w + WAVES * (u / 2)) + (u % 2);
            return s0 + u * WAVES;
        };
        auto load_w = [&](int s0) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int s = step_of(s0, u);
                const uint32_t k = k0 + static_cast<uint32_t>(s) * 32u + 8u * c;   // this lane's chunk
                wv[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, s < steps && k < K ? vw : OOB, 2u * (k0 + 32u * s),
                                                              TMM_GEMV_AUX);
            }
        };
        // The first group of W loads goes out while X lands: loads complete in order, so
        // once at most UNROLL are outstanding this wave's X loads are done.
        load_w(w);
        wait_vmcnt<UNROLL>();
        barrier();
        for (int s0 = w; s0 < steps; s0 += WAVES * UNROLL) {
            if (s0 != w) load_w(s0);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int s = step_of(s0, u);
                if (s < steps) {   // wave-uniform
                    const bf16x8 xv = *reinterpret_cast<const bf16x8*>(xfrag + s * 64);
                    acc = mfma_16x16x32(__builtin_bit_cast(bf16x8, wv[u]), xv, acc);
                }
            }
        }
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

// Each wave loads both 64-byte halves of a W row's 128-byte lines back to back (1) or the
// waves take the 32-deep k steps in turn (0).
#ifndef TMM_GEMV_PAIRS
#define TMM_GEMV_PAIRS 1
#endif

// W loads in flight per wave (16 covers a whole phase of 4096 k at once).
#ifndef TMM_GEMV_UNROLL
#define TMM_GEMV_UNROLL 16
#endif

// ---------------------------------------------------------------------------------------
// Small M: the dot-product form.
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

// Wave w of workgroup b owns ROWS consecutive rows of W.  In each 512-element chunk of K,
// lane l takes the 16 bytes at k = 512 j + 8 l of each of its rows, so one load instruction
// reads 1 KB of one row of W, and UNROLL chunks are in flight before any is consumed.  X
// is staged once per workgroup in LDS, in phases of KX elements of K, by direct-to-LDS
// loads (rows m >= M and columns k >= K land as zeros, so the products past the ends are
// 0 * 0); the first W chunks are issued before the wait for X, so the two overlap.  One
// ds_read of X per (chunk, row of X) serves the ROWS rows of W the wave holds.  Products:
// v_dot2c_f32_bf16 (exact bf16 products, fp32 sums); the 64 lane partial sums of each
// output are added with lane shuffles at the end.  The VALU work grows with M (4 M dot
// instructions per 16 bytes of W), which is why larger M takes the MFMA form above.
template <int OUT, int MP, int ROWS, int UNROLL, int WAVES, int KX>
__global__ __launch_bounds__(64 * WAVES) void gemv_lds_kernel(GemmArgs g) {
    static_assert(KX % (512 * UNROLL) == 0, "a phase holds whole groups of chunks");
    __shared__ __attribute__((aligned(1024))) uint8_t xs[MP * KX * 2];
    const int lane = lane_id(), w = wave_id();
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * WAVES + w) * ROWS;
    const int rows = static_cast<int>(max<int64_t>(0, min<int64_t>(ROWS, g.N - n0)));
    const int M = static_cast<int>(g.M);
    const uint32_t K = static_cast<uint32_t>(g.K);
    const uint32_t ldb2 = static_cast<uint32_t>(g.ldb * 2), lda2 = static_cast<uint32_t>(g.lda * 2);
    // A wave past the last row of W still stages X and takes part in the barriers; its
    // resource covers nothing, so its W loads read zeros.
    const auto rw = make_rsrc(rows > 0 ? g.B + n0 * g.ldb : g.B,
                              rows > 0 ? static_cast<uint32_t>(((rows - 1) * g.ldb + g.K) * 2) : 0u);
    const auto rx = make_rsrc(g.A, static_cast<uint32_t>(((g.M - 1) * g.lda + g.K) * 2));

    float acc[ROWS][MP];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MP; ++m) acc[r][m] = 0.f;

    constexpr int CH = KX / 512;   // 1 KB chunks per row of X per phase
    for (uint32_t k0 = 0; k0 < K; k0 += KX) {
        if (k0 > 0) barrier();   // every wave is done with the previous phase of X
        static_assert((MP * CH) % WAVES == 0 || MP * CH < WAVES, "X loads split evenly over the waves");
#pragma unroll
        for (int i = 0; i < (MP * CH + WAVES - 1) / WAVES; ++i) {
            const int q = w + i * WAVES, m = q / CH, j = q % CH;
            if (q >= MP * CH) break;   // wave-uniform (only when MP * CH < WAVES)
            const uint32_t k = k0 + 512u * j + 8u * lane;
            load_lds_16(rx, xs + m * KX * 2 + j * 1024, m < M && k < K ? m * lda2 + 2u * k : OOB, 0);
        }
        asm volatile("" ::: "memory");   // the W loads below stay behind the X loads
        const uint32_t kend = min(K - k0, static_cast<uint32_t>(KX));
        u32x4 wv[UNROLL][ROWS];
        auto load_w = [&](uint32_t c0) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const uint32_t k = k0 + c0 + 512u * u + 8u * lane;
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    wv[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rw, k < K && r < rows ? r * ldb2 + 2u * k : OOB,
                                                                     0, TMM_GEMV_AUX);
            }
        };
        // The first W chunks go out while X lands (loads complete in order).
        load_w(0);
        wait_vmcnt<UNROLL * ROWS>();
        barrier();
        for (uint32_t c0 = 0; c0 < kend; c0 += 512u * UNROLL) {
            if (c0 != 0) load_w(c0);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int m = 0; m < MP; ++m) {
                    const u32x4 xv = *reinterpret_cast<const u32x4*>(xs + m * KX * 2 + (c0 + 512u * u) * 2 + lane * 16);
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) acc[r][m] = dot8(wv[u][r], xv, acc[r][m]);
                }
        }
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

#ifndef TMM_LDS_ROWS
#define TMM_LDS_ROWS 1
#endif
#ifndef TMM_LDS_UNROLL
#define TMM_LDS_UNROLL 4
#endif
#ifndef TMM_LDS_WAVES
#define TMM_LDS_WAVES 16
#endif
constexpr int LDS_KX = 4096;   // K elements of X per staged phase (MP x 8 KB of LDS)

template <int OUT, int MP>
static void launch_lds_mp(const GemmArgs& g, const Plan& p, hipStream_t s) {
    hipLaunchKernelGGL((gemv_lds_kernel<OUT, MP, TMM_LDS_ROWS, TMM_LDS_UNROLL, TMM_LDS_WAVES, LDS_KX>),
                       dim3(p.grid_x), dim3(64 * TMM_LDS_WAVES), 0, s, g);
}

template <int OUT>
static void launch_lds_out(const GemmArgs& g, const Plan& p, hipStream_t s) {
    if (g.M <= 1) launch_lds_mp<OUT, 1>(g, p, s);
    else if (g.M <= 2) launch_lds_mp<OUT, 2>(g, p, s);
    else if (g.M <= 4) launch_lds_mp<OUT, 4>(g, p, s);
    else if (g.M <= 8) launch_lds_mp<OUT, 8>(g, p, s);
    else launch_lds_mp<OUT, 16>(g, p, s);
}

hipError_t launch_gemv_lds(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    if (out == OUT_F32) launch_lds_out<OUT_F32>(g, p, s);
    else launch_lds_out<OUT_BF16>(g, p, s);
    return hipGetLastError();
}

int gemv_lds_rows_per_workgroup() { return TMM_LDS_WAVES * TMM_LDS_ROWS; }
int gemv_lds_threads() { return 64 * TMM_LDS_WAVES; }

hipError_t launch_gemv(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    constexpr int U = TMM_GEMV_UNROLL;
    constexpr bool PR = TMM_GEMV_PAIRS != 0;
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemv_kernel<OUT_F32, U, PR>), dim3(p.grid_x), dim3(512), 0, s, g);
    else
        hipLaunchKernelGGL((gemv_kernel<OUT_BF16, U, PR>), dim3(p.grid_x), dim3(512), 0, s, g);
    return hipGetLastError();
}

}  // namespace tmm
