// The pipelined GEMM, C = A * B^T (bf16 in, fp32 accumulate): ladder steps 2 and 4.
//
// Prior art is the page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "9 步优化":
// step 4 moves whole tiles from global memory to shared memory with a copy engine and a
// completion barrier, step 5 rotates two staging buffers so that loading block i+1 overlaps
// computing block i, step 6 keeps about one workgroup per SM alive and hands it tiles in an
// L2-friendly order.  On gfx950 the same functions map to:
//
//   * copy engine  -> per-lane direct-to-LDS loads (buffer_load_dwordx4 ... lds): each lane
//     moves 16 bytes from global memory into LDS without touching VGPRs; a wave writes
//     1 KB of consecutive LDS bytes per instruction.
//   * completion barrier -> the issuing wave's s_waitcnt vmcnt, then s_barrier.
//   * staging ring -> STAGES slots of (BM + BN) x BK bf16 in LDS; slot k+STAGES-1 is filled
//     while slot k is consumed.
//   * swizzle (the page's section on layout, and the blog's section on TIRx tile layouts:
//     shuffle data in shared memory to avoid bank conflicts) -> LDS row r holds its 16-byte
//     k-chunks permuted by c' = c XOR f(r).  The direct-to-LDS write order is fixed by lane
//     order, so the permutation is applied on the global side: the lane that writes
//     physical slot s of row r fetches logical chunk s XOR f(r) of that row.  The 8 lanes of
//     one row still fetch one 128-byte segment, so the load stays fully coalesced.
//   * register-blocked accumulator -> each of the 4 waves owns a (BM/2) x (BN/2) block of
//     the tile as v_mfma_f32_16x16x32_bf16 accumulators.
//   * tile scheduler -> PERSIST: gridDim.x ~ number of CUs, workgroup w takes work items
//     w, w + grid, ... through tile_of(), the XCD-aware grouped order.  While a finished
//     tile is written back, the next tile's first stages are already loading.
//
// Preconditions checked by the planner: K % 8 == 0, lda, ldb, strideA, strideB multiples
// of 8 and A, B 16-byte aligned, BM * lda * 2 and BN * ldb * 2 below 2^31.  Rows beyond M
// (N) and k-chunks beyond K are turned into out-of-range buffer offsets, which read zeros.
#include "launch.hpp"

namespace tmm {

template <int BM, int BN, int BK, int STAGES, int SWZ>
struct PipeCfg {
    static constexpr int WM = BM / 2, WN = BN / 2;      // wave tile (2 x 2 waves)
    static constexpr int FM = WM / 16, FN = WN / 16;    // 16-wide fragments per wave
    static constexpr int KC = BK / 8;                   // 16-byte chunks per LDS row
    static constexpr int R = 64 / KC;                   // LDS rows per wave load instruction
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int IA = BM / (4 * R), IB = BN / (4 * R);   // loads per wave per stage
    static constexpr int LOADS = IA + IB;
    static_assert(IA * 4 * R == BM && IB * 4 * R == BN, "tile rows must split over 4 waves");
    static_assert(BK % 32 == 0 && KC <= 8, "BK must be 32 or 64");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert((STAGES - 1) * LOADS <= 63, "vmcnt holds at most 63 outstanding loads");

    // XOR pattern applied to the chunk index of LDS row r.
    static __device__ __forceinline__ int swz(int r) {
        if constexpr (SWZ == 0) return 0;
        else if constexpr (SWZ == 1) return r & (KC - 1);
        else return (r >> 1) & (KC - 1);
    }
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int BK, int STAGES, int SWZ, int OUT, bool XCD_ORDER>
__global__ __launch_bounds__(256, 1) void gemm_pipe_kernel(GemmArgs g, TileGrid tg, int vec_store) {
    typedef PipeCfg<BM, BN, BK, STAGES, SWZ> P;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * P::STAGE_BYTES];

    const int lane = lane_id(), w = wave_id();
    const int wm = w >> 1, wn = w & 1;
    const int nk = static_cast<int>((g.K + BK - 1) / BK);

    // Per-lane global offsets (bytes from the tile's first row, at k = 0) of the 16-byte
    // chunk this lane moves in each of its load instructions, and the matching LDS row
    // chunk it lands in.  Load i of wave w covers LDS rows [(4 i + w) R, (4 i + w + 1) R).
    const int lrow = lane / P::KC, lslot = lane % P::KC;
    uint32_t chunk_k[P::IA > P::IB ? P::IA : P::IB];    // element k offset of the chunk
#pragma unroll
    for (int i = 0; i < (P::IA > P::IB ? P::IA : P::IB); ++i) {
        const int r = (4 * i + w) * P::R + lrow;
        chunk_k[i] = 8u * static_cast<uint32_t>(lslot ^ P::swz(r));
    }
    // Fragment read offsets within a stage (bytes), for each 32-wide k step: row
    // (lane % 16) of a 16-row block (the swizzle depends on row % 16 only), chunk
    // 4 kk + lane / 16.
    int rd[BK / 32];
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
        const int r = lane & 15, c = 4 * kk + (lane >> 4);
        rd[kk] = r * BK * 2 + ((c ^ P::swz(r)) * 16);
    }

    for (int t = blockIdx.x; t < tg.total; t += gridDim.x) {
        int bt, tm, tn;
        if constexpr (XCD_ORDER) {
            tile_of(t, tg, bt, tm, tn);
        } else {
            const int tiles = tg.tiles_m * tg.tiles_n;
            bt = t / tiles;
            tm = (t % tiles) / tg.tiles_n;
            tn = t % tg.tiles_n;
        }
        const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
        const int64_t rows_a = min<int64_t>(BM, g.M - m0), rows_b = min<int64_t>(BN, g.N - n0);
        const uint16_t* Ab = g.A + bt * g.sA + m0 * g.lda;
        const uint16_t* Bb = g.B + bt * g.sB + n0 * g.ldb;
        const auto ra = make_rsrc(Ab, static_cast<uint32_t>(((rows_a - 1) * g.lda + g.K) * 2));
        const auto rb = make_rsrc(Bb, static_cast<uint32_t>(((rows_b - 1) * g.ldb + g.K) * 2));

        // Row part of each load's offset; out-of-range rows get an offset past the buffer.
        uint32_t va[P::IA], vb[P::IB];
#pragma unroll
        for (int i = 0; i < P::IA; ++i) {
            const int r = (4 * i + w) * P::R + lrow;
            va[i] = r < rows_a ? static_cast<uint32_t>(r * g.lda) * 2u + 2u * chunk_k[i] : OOB;
        }
#pragma unroll
        for (int i = 0; i < P::IB; ++i) {
            const int r = (4 * i + w) * P::R + lrow;
            vb[i] = r < rows_b ? static_cast<uint32_t>(r * g.ldb) * 2u + 2u * chunk_k[i] : OOB;
        }

        // Issue all loads of K block kb into ring slot `slot`.
        auto issue = [&](int kb, int slot) {
            uint8_t* sa = lds + slot * P::STAGE_BYTES;
            uint8_t* sb = sa + P::A_BYTES;
            const uint32_t k0 = static_cast<uint32_t>(kb) * BK;
            const uint32_t soff = 2u * k0;
            if (k0 + BK <= static_cast<uint32_t>(g.K)) {
#pragma unroll
                for (int i = 0; i < P::IA; ++i)
                    load_lds_16(ra, sa + (4 * i + w) * P::R * BK * 2, va[i], soff);
#pragma unroll
                for (int i = 0; i < P::IB; ++i)
                    load_lds_16(rb, sb + (4 * i + w) * P::R * BK * 2, vb[i], soff);
            } else {  // K tail: chunks at k >= K read zeros
#pragma unroll
                for (int i = 0; i < P::IA; ++i) {
                    const bool ok = k0 + chunk_k[i] < static_cast<uint32_t>(g.K);
                    load_lds_16(ra, sa + (4 * i + w) * P::R * BK * 2, ok ? va[i] : OOB, soff);
                }
#pragma unroll
                for (int i = 0; i < P::IB; ++i) {
                    const bool ok = k0 + chunk_k[i] < static_cast<uint32_t>(g.K);
                    load_lds_16(rb, sb + (4 * i + w) * P::R * BK * 2, ok ? vb[i] : OOB, soff);
                }
            }
        };

        f32x4 acc[P::FN][P::FM];
#pragma unroll
        for (int i = 0; i < P::FN; ++i)
#pragma unroll
            for (int j = 0; j < P::FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Prologue: the first STAGES-1 K blocks.  (Every wave has passed the previous
        // tile's final barrier, so the whole ring is free.)
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nk) issue(s, s);

        for (int kb = 0; kb < nk; ++kb) {
            // Block kb has landed once at most (STAGES-2) later blocks are outstanding.
            if (kb + STAGES - 2 < nk) wait_vmcnt<(STAGES - 2) * P::LOADS>();
            else wait_vmcnt<0>();
            barrier();  // every wave's share of block kb is in LDS; block kb-1 is consumed
            if (kb + STAGES - 1 < nk) issue(kb + STAGES - 1, (kb + STAGES - 1) % STAGES);

            const uint8_t* sa = lds + (kb % STAGES) * P::STAGE_BYTES;
            const uint8_t* sb = sa + P::A_BYTES;
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
                bf16x8 fb[P::FN], fa[P::FM];
#pragma unroll
                for (int i = 0; i < P::FN; ++i)
                    fb[i] = *reinterpret_cast<const bf16x8*>(sb + (wn * P::WN + 16 * i) * BK * 2 + rd[kk]);
#pragma unroll
                for (int j = 0; j < P::FM; ++j)
                    fa[j] = *reinterpret_cast<const bf16x8*>(sa + (wm * P::WM + 16 * j) * BK * 2 + rd[kk]);
#pragma unroll
                for (int i = 0; i < P::FN; ++i)
#pragma unroll
                    for (int j = 0; j < P::FM; ++j) acc[i][j] = mfma_16x16x32(fb[i], fa[j], acc[i][j]);
            }
        }
        barrier();  // all fragment reads of this tile are done before the ring is refilled

        void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                  : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
        store_acc<OUT, P::FN, P::FM>(Cb, g.ldc, g.M, g.N, m0 + wm * P::WM, n0 + wn * P::WN, acc,
                                     vec_store != 0);
    }
}

template <int BM, int BN, int BK, int STAGES, int SWZ, bool XCD>
static hipError_t launch_pipe_cfg(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_pipe_kernel<BM, BN, BK, STAGES, SWZ, OUT_F32, XCD>), dim3(p.grid_x),
                           dim3(256), 0, s, g, p.grid, p.vec_store);
    else
        hipLaunchKernelGGL((gemm_pipe_kernel<BM, BN, BK, STAGES, SWZ, OUT_BF16, XCD>), dim3(p.grid_x),
                           dim3(256), 0, s, g, p.grid, p.vec_store);
    return hipGetLastError();
}

hipError_t launch_pipe(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    switch (p.kernel) {
        case K_PIPE_256: return launch_pipe_cfg<256, 256, 64, 2, 1, false>(g, out, p, s);
        case K_PIPE_128: return launch_pipe_cfg<128, 128, 64, 3, 1, false>(g, out, p, s);
        case K_PERSIST_256: return launch_pipe_cfg<256, 256, 64, 2, 1, true>(g, out, p, s);
        case K_PERSIST_128: return launch_pipe_cfg<128, 128, 64, 3, 1, true>(g, out, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tmm
