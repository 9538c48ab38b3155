// Fixed-role waves, C = A * B^T (bf16 in, fp32 accumulate): ladder step 7 as the page builds
// it, kept as a selectable rung so that the choice made for the AUTO kernels can be measured.
//
// The page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "9 步优化", step 7, splits
// the warps of a block into roles: producers that only move tiles into shared memory, an MMA
// consumer, and a write-back role, handing stages over with barriers so that copy and math
// proceed in parallel.  Here: eight waves, two per SIMD (wave w and wave w + 4 share SIMD
// w mod 4).  Waves 0-3 are producers: they only issue the direct-to-LDS loads of a three-slot
// ring of 64-deep blocks.  Waves 4-7 are consumers: they only read fragments from LDS and issue
// MFMAs, and write their accumulators back at the end of each tile while the producers are
// already loading the next tile's blocks (the write-back role).  Producers and consumers run
// one flattened stream of (tile, block) pairs over the workgroup's tiles and meet at one
// workgroup barrier per block:
//
//   producers, iteration j:  load block j + 2 (into the slot of block j - 1); wait until this
//                            wave's loads of block j + 1 have landed; barrier
//   consumers, iteration j:  MFMAs on block j's first 32 k while reading its second 32 k;
//                            barrier; MFMAs on block j's second 32 k while reading block
//                            j + 1's first 32 k; at the last block of a tile, store C
//
// At the barrier every producer's share of block j + 1 is in LDS and every consumer is done
// with block j, whose slot the producers fill with block j + 3 in the next iteration.
//
// gfx950 gives every wave of a dispatch the same registers: with two waves per SIMD each
// has 256 (against 512 at one wave per SIMD), so a consumer holds a 128 x 64 accumulator
// block (128 registers) and the workgroup tile is 256 x 128, where the 4-wave ring kernels
// hold 128 x 128 per wave and a 256 x 256 tile.  That is the trade this rung measures.
//
// Preconditions (planner): both operands K-major, A and B 4-byte aligned with even pitches
// and strides, K a multiple of 8, 256 * ld * 2 below 2^31.
#include "launch.hpp"
#include "mfma_step.hpp"

namespace tmm {

#ifndef TMM_ROLES_TAIL
#define TMM_ROLES_TAIL 8
#endif

namespace rl {
constexpr int BM = 256, BN = 128, BK = 64, NS = 3;
constexpr int ROWB = BK * 2;                      // bytes per LDS row
constexpr int A_T = BM * ROWB, B_T = BN * ROWB;   // 32 KB + 16 KB per slot
constexpr int STAGE = A_T + B_T;
constexpr int NP = 4, NC = 4;                     // producer and consumer waves
constexpr int R = 8;                              // LDS rows per load instruction
constexpr int LA = BM / (NP * R), LB = BN / (NP * R), L = LA + LB;   // loads per producer per block
constexpr int WM = 128, WN = 64;                  // consumer wave tile (2 x 2 consumers)
constexpr int FM = WM / 16, FN = WN / 16;
static_assert(NS * STAGE <= 160 * 1024, "LDS capacity");
static_assert(2 * L <= 63, "vmcnt range");
__device__ __forceinline__ int swz(int r) { return r & 7; }
}  // namespace rl

template <int OUT>
__global__ __launch_bounds__(512, 1) void gemm_roles_kernel(GemmArgs g, TileGrid tg, int vec_store) {
    using namespace rl;
    using MM = Mma<16>;
    using Acc = MM::Acc;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];

    const int lane = lane_id(), w = wave_id();
    const int nk = static_cast<int>((g.K + BK - 1) / BK);
    const uint32_t K = static_cast<uint32_t>(g.K);
    // this workgroup's tiles: blockIdx.x, blockIdx.x + gridDim.x, ...; J (tile, block) pairs
    const int ntiles = blockIdx.x < tg.total ? (tg.total - 1 - static_cast<int>(blockIdx.x)) / gridDim.x + 1 : 0;
    const int J = ntiles * nk;

    if (w < NP) {
        // ---------------- producers ----------------
        const int p = w, lrow = lane / 8;
        const uint32_t chunk_k = 8u * static_cast<uint32_t>((lane % 8) ^ swz(lrow));
        // Loads of pair j into slot j mod NS (nothing past the last pair).
        auto issue = [&](int j) {
            if (j >= J) return;
            const int i = j / nk, kb = j - i * nk;
            int bt, tm, tn;
            tile_of(static_cast<int>(blockIdx.x) + i * static_cast<int>(gridDim.x), tg, bt, tm, tn);
            const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
            const int64_t rows_a = min<int64_t>(BM, g.M - m0), rows_b = min<int64_t>(BN, g.N - n0);
            const auto ra = make_rsrc(g.A + bt * g.sA + m0 * g.lda, static_cast<uint32_t>(((rows_a - 1) * g.lda + g.K) * 2));
            const auto rb = make_rsrc(g.B + bt * g.sB + n0 * g.ldb, static_cast<uint32_t>(((rows_b - 1) * g.ldb + g.K) * 2));
            const uint32_t k0 = static_cast<uint32_t>(kb) * BK;
            const bool ok = k0 + chunk_k < K;
            uint8_t* slot = lds + (j % NS) * STAGE;
#pragma unroll
            for (int q = 0; q < LA; ++q) {
                const int r = (q * NP + p) * R + lrow;
                const uint32_t v = ok && r < rows_a ? static_cast<uint32_t>(r * g.lda) * 2u + 2u * chunk_k : OOB;
                load_lds_16(ra, slot + (q * NP + p) * R * ROWB, v, 2u * k0);
            }
#pragma unroll
            for (int q = 0; q < LB; ++q) {
                const int r = (q * NP + p) * R + lrow;
                const uint32_t v = ok && r < rows_b ? static_cast<uint32_t>(r * g.ldb) * 2u + 2u * chunk_k : OOB;
                load_lds_16(rb, slot + A_T + (q * NP + p) * R * ROWB, v, 2u * k0);
            }
        };
        issue(0);
        issue(1);
        if (J > 1)
            wait_vmcnt<L>();   // pair 0 has landed (pair 1 may be in flight)
        else
            wait_vmcnt<0>();   // no pair 1 was issued
        barrier();
        for (int j = 0; j < J; ++j) {
            issue(j + 2);
            if (j + 2 < J)
                wait_vmcnt<L>();   // everything but pair j + 2: pair j + 1 has landed
            else
                wait_vmcnt<0>();
            barrier();
        }
        return;
    }

    // ---------------- consumers ----------------
    const int c = w - NP, cm = c / 2, cn = c % 2;
    int rd[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) rd[kk] = (lane % 16) * ROWB + (((4 * kk + lane / 16) ^ swz(lane % 16)) * 16);
    const int a_off = cm * WM * ROWB, b_off = A_T + cn * WN * ROWB;
    using F = Frags<FN, FM>;
    auto read_one = [&](F& f, int q, int j, int kk) {
        const uint8_t* slot = lds + (j % NS) * STAGE;
        if (q < FN)
            f.b[q] = *reinterpret_cast<const bf16x8*>(slot + b_off + 16 * q * ROWB + rd[kk]);
        else
            f.a[q - FN] = *reinterpret_cast<const bf16x8*>(slot + a_off + 16 * (q - FN) * ROWB + rd[kk]);
    };
    constexpr int NR = FN + FM;
    Acc acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int jj = 0; jj < FM; ++jj) acc[i][jj] = MM::zero();

    barrier();
    F f[2];
    if (J > 0) {
#pragma unroll
        for (int q = 0; q < NR; ++q) read_one(f[0], q, 0, 0);
    }
    wait_cnt<63, 0>();
    for (int j = 0; j < J; ++j) {
        step<FN, FM, NR, 0, true, MM, TMM_ROLES_TAIL>(acc, f[0], [&](int q) { read_one(f[1], q, j, 1); },
                                                       [&](int) {});
        __builtin_amdgcn_sched_barrier(0);
        wait_cnt<63, 0>();
        __builtin_amdgcn_sched_barrier(0);
        barrier();
        const int jn = j + 1 < J ? j + 1 : j;   // the last step re-reads its own block (unused)
        step<FN, FM, NR, 0, true, MM, TMM_ROLES_TAIL>(acc, f[1], [&](int q) { read_one(f[0], q, jn, 0); },
                                                       [&](int) {});
        __builtin_amdgcn_sched_barrier(0);
        wait_cnt<63, 0>();
        __builtin_amdgcn_sched_barrier(0);
        const int i = j / nk;
        if (j - i * nk == nk - 1) {   // last block of tile i: write it back, start the next
            int bt, tm, tn;
            tile_of(static_cast<int>(blockIdx.x) + i * static_cast<int>(gridDim.x), tg, bt, tm, tn);
            const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
            void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                      : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
            store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + cm * WM, n0 + cn * WN, acc, vec_store != 0);
#pragma unroll
            for (int a = 0; a < FN; ++a)
#pragma unroll
                for (int b = 0; b < FM; ++b) acc[a][b] = MM::zero();
        }
    }
}

hipError_t launch_roles(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    const dim3 grid(p.grid_x), block(512);
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_roles_kernel<OUT_F32>), grid, block, 0, s, g, p.grid, p.vec_store);
    else
        hipLaunchKernelGGL((gemm_roles_kernel<OUT_BF16>), grid, block, 0, s, g, p.grid, p.vec_store);
    return hipGetLastError();
}

}  // namespace tmm
