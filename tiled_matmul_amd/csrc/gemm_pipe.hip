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
// Preconditions checked by the planner: A, B 4-byte aligned, lda, ldb, strideA, strideB
// even (every row starts on a 4-byte boundary; the 16-byte loads do not need more),
// BM * lda * 2 and BN * ldb * 2 below 2^31.  Rows beyond M (N) and k-chunks beyond K8 = K
// rounded down to a multiple of 8 are turned into out-of-range buffer offsets, which read
// zeros; the remaining K - K8 < 8 columns enter through one extra k step after the loop.
#include "launch.hpp"
#include "mfma_step.hpp"

namespace tmm {

template <int BM, int BN, int BK, int STAGES, int SWZ, int WAVES_M = 2, int WAVES_N = 2>
struct PipeCfg {
    static constexpr int NW = WAVES_M * WAVES_N;        // waves per workgroup
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // wave tile
    static constexpr int KC = BK / 8;                   // 16-byte chunks per LDS row
    static constexpr int R = 64 / KC;                   // LDS rows per wave load instruction
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int IA = BM / (NW * R), IB = BN / (NW * R);   // loads per wave per stage
    static constexpr int LOADS = IA + IB;
    static_assert(IA * NW * R == BM && IB * NW * R == BN, "tile rows must split over the waves");
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

// RAGGED: K is not a multiple of 8 (a separate instance, so that the common case carries
// none of the tail code and none of the registers it holds).
template <int BM, int BN, int BK, int STAGES, int SWZ, int MF, int OUT, bool XCD_ORDER, int WAVES_M,
          int WAVES_N, bool RAGGED>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, WAVES_M * WAVES_N / 4) void gemm_pipe_kernel(
    GemmArgs g, TileGrid tg, int vec_store) {
    typedef PipeCfg<BM, BN, BK, STAGES, SWZ, WAVES_M, WAVES_N> P;
    typedef Mma<MF> T;
    constexpr int KSTEPS = BK / T::KS;
    constexpr bool FINE = WAVES_M * WAVES_N >= 8;   // see step()
    constexpr int FN = P::WN / T::ROWS, FM = P::WM / T::ROWS;   // fragments per wave
    // Loads issued after the last load of block kb + 1 when block kb + 1 must have landed.
    constexpr int WAIT_N = (STAGES - 2) * P::LOADS;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * P::STAGE_BYTES];

    const int lane = lane_id(), w = wave_id();
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const int nk = static_cast<int>((g.K + BK - 1) / BK);
    const uint32_t K = static_cast<uint32_t>(g.K);
    // The 16-byte loads cover k < K8; a ragged tail K8 <= k < K (K not a multiple of 8) is
    // added by one more MFMA step after the loop.
    const uint32_t K8 = RAGGED ? K & ~7u : K;
    constexpr int NW = P::NW;

    // Per-lane element k offset of the 16-byte chunk this lane moves in each of its load
    // instructions.  Load i of wave w covers LDS rows [(NW i + w) R, (NW i + w + 1) R); lane
    // writes physical slot (lane % KC) of row (lane / KC), which holds logical chunk
    // slot ^ swz(row).
    const int lrow = lane / P::KC, lslot = lane % P::KC;
    constexpr int IMAX = P::IA > P::IB ? P::IA : P::IB;
    uint32_t chunk_k[IMAX];
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
        const int r = (NW * i + w) * P::R + lrow;
        chunk_k[i] = 8u * static_cast<uint32_t>(lslot ^ P::swz(r));
    }
    // Fragment read offsets within a stage (bytes), for each k step: row (lane % ROWS) of
    // a ROWS-row block (the swizzle depends on row % 8 only), chunk
    // (KS / 8) kk + lane / ROWS.
    int rd[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
        const int r = lane % T::ROWS, c = (T::KS / 8) * kk + lane / T::ROWS;
        rd[kk] = r * BK * 2 + ((c ^ P::swz(r)) * 16);
    }
    const int a_frag0 = wm * P::WM * BK * 2, b_frag0 = P::A_BYTES + wn * P::WN * BK * 2;

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
            const int r = (NW * i + w) * P::R + lrow;
            va[i] = r < rows_a ? static_cast<uint32_t>(r * g.lda) * 2u + 2u * chunk_k[i] : OOB;
        }
#pragma unroll
        for (int i = 0; i < P::IB; ++i) {
            const int r = (NW * i + w) * P::R + lrow;
            vb[i] = r < rows_b ? static_cast<uint32_t>(r * g.ldb) * 2u + 2u * chunk_k[i] : OOB;
        }

        // Issue every load of K block kb into ring slot `slot`.  Chunks at k >= K (the K
        // tail, or a block past the end) get out-of-range offsets and write zeros.
        auto issue = [&](int kb, int slot) {
            uint8_t* sa = lds + slot * P::STAGE_BYTES;
            uint8_t* sb = sa + P::A_BYTES;
            const uint32_t k0 = static_cast<uint32_t>(kb) * BK;
            const uint32_t soff = 2u * k0;
#pragma unroll
            for (int i = 0; i < P::IA; ++i)
                load_lds_16(ra, sa + (NW * i + w) * P::R * BK * 2, k0 + chunk_k[i] < K8 ? va[i] : OOB, soff);
#pragma unroll
            for (int i = 0; i < P::IB; ++i)
                load_lds_16(rb, sb + (NW * i + w) * P::R * BK * 2, k0 + chunk_k[i] < K8 ? vb[i] : OOB, soff);
        };
        auto read_frags = [&](Frags<FN, FM>& f, int slot, int kk) {
            const uint8_t* base = lds + slot * P::STAGE_BYTES + rd[kk];
#pragma unroll
            for (int i = 0; i < FN; ++i)
                f.b[i] = *reinterpret_cast<const bf16x8*>(base + b_frag0 + T::ROWS * i * BK * 2);
#pragma unroll
            for (int j = 0; j < FM; ++j)
                f.a[j] = *reinterpret_cast<const bf16x8*>(base + a_frag0 + T::ROWS * j * BK * 2);
        };

        // One load instruction of block kb (i < IA: A rows, else B rows) into slot `slot`.
        auto issue_one = [&](int i, int kb, int slot) {
            uint8_t* sa = lds + slot * P::STAGE_BYTES;
            const uint32_t k0 = static_cast<uint32_t>(kb) * BK;
            if (i < P::IA)
                load_lds_16(ra, sa + (NW * i + w) * P::R * BK * 2, k0 + chunk_k[i] < K8 ? va[i] : OOB, 2u * k0);
            else
                load_lds_16(rb, sa + P::A_BYTES + (NW * (i - P::IA) + w) * P::R * BK * 2,
                            k0 + chunk_k[i - P::IA] < K8 ? vb[i - P::IA] : OOB, 2u * k0);
        };
        // One fragment (q < FN: B fragment q, else A fragment q - FN) of k step kk of `slot`.
        auto read_one = [&](Frags<FN, FM>& f, int q, int slot, int kk) {
            const uint8_t* base = lds + slot * P::STAGE_BYTES + rd[kk];
            if (q < FN)
                f.b[q] = *reinterpret_cast<const bf16x8*>(base + b_frag0 + T::ROWS * q * BK * 2);
            else
                f.a[q - FN] = *reinterpret_cast<const bf16x8*>(base + a_frag0 + T::ROWS * (q - FN) * BK * 2);
        };

        typename T::Acc acc[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = T::zero();

        // Prologue: blocks 0 .. STAGES-2, wait for block 0, then block STAGES-1, and the
        // fragments of block 0's first k step.  (Every wave has passed the previous tile's
        // final barrier, so the whole ring is free.)
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s) issue(s, s);
        wait_vmcnt<WAIT_N>();
        barrier();
        issue(STAGES - 1, STAGES - 1);
        Frags<FN, FM> f[2];
        read_frags(f[0], 0, 0);
        wait_cnt<63, 0>();

        // Block kb: k steps 0 .. KSTEPS-2 read the next step's fragments, then run their own
        // MFMAs.  The last step first waits for this wave's loads of block kb+1 and for its
        // own fragment reads, passes the barrier (every wave's share of kb+1 is in LDS and
        // every wave is done reading block kb), starts reading block kb+1's first fragments,
        // refills block kb's slot with block kb+STAGES, and only then runs its MFMAs, so the
        // reads and loads overlap them.  Blocks past the end are issued too (their chunks
        // are all beyond K and read as zeros): the count of outstanding loads is then the same
        // in every iteration and the loop body has no branch.
        int slot = 0;
        for (int kb = 0; kb < nk; ++kb) {
#pragma unroll
            for (int kk = 0; kk + 1 < KSTEPS; ++kk)
                step<FN, FM, FN + FM, 0, FINE>(acc, f[kk & 1], [&](int q) { read_one(f[(kk + 1) & 1], q, slot, kk + 1); },
                                         [&](int) {});
            constexpr int LAST = (KSTEPS - 1) & 1;
            const int next_slot = slot + 1 == STAGES ? 0 : slot + 1;
            wait_cnt<WAIT_N, 0>();
            barrier();
            step<FN, FM, FN + FM, P::LOADS, FINE>(acc, f[LAST], [&](int q) { read_one(f[LAST ^ 1], q, next_slot, 0); },
                                            [&](int q) { issue_one(q, kb + STAGES, slot); });
            // The reads of block kb+1's first fragments were interleaved with the MFMAs just
            // issued and have long completed; saying so here keeps the compiler from stalling
            // the next iteration's first MFMA on a conservative lgkmcnt.
            __builtin_amdgcn_sched_barrier(0);
            wait_cnt<63, 0>();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (LAST == 1) {
                // KSTEPS even: the next block's first fragments went to f[0]; nothing to move.
            } else {
                f[0] = f[1];
            }
            slot = next_slot;
        }
        wait_vmcnt<0>();   // the trailing zero-fill loads have landed
        barrier();  // all fragment reads of this tile are done before the ring is refilled

        if constexpr (RAGGED) {
            // Ragged K tail: one more k step over k = K8 .. K8 + KS - 1 whose first 16-byte
            // chunk holds elements K8 .. K - 1 of each row and everything else is zero.
            // Each thread stages whole rows into ring slot 0 (free since the barrier above),
            // element by element so nothing at or beyond K is read; then every wave reads
            // its fragments as in the loop.
            const uint16_t* Ag = g.A + bt * g.sA + m0 * g.lda;
            const uint16_t* Bg = g.B + bt * g.sB + n0 * g.ldb;
            for (int r = threadIdx.x; r < BM + BN; r += 64 * NW) {
                const bool is_a = r < BM;
                const int rr = is_a ? r : r - BM;
                uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (rr < (is_a ? rows_a : rows_b)) {
                    const uint16_t* row = is_a ? Ag + rr * g.lda : Bg + rr * g.ldb;
#pragma unroll
                    for (int e = 0; e < 7; ++e)
                        if (K8 + e < K) h[e] = row[K8 + e];
                }
                uint8_t* dst = lds + (is_a ? 0 : P::A_BYTES) + rr * BK * 2;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 v = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
#pragma unroll
                for (int c = 0; c < T::KS / 8; ++c)
                    *reinterpret_cast<u32x4*>(dst + ((c ^ P::swz(rr)) * 16)) = c == 0 ? v : z;
            }
            barrier();
            read_frags(f[0], 0, 0);
            wait_cnt<63, 0>();
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = T::run(f[0].b[i], f[0].a[j], acc[i][j]);
            barrier();   // the ring is read before the next tile refills it
        }

        void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                  : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
        if constexpr (MF == 16)
            store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * P::WM, n0 + wn * P::WN, acc,
                                   vec_store != 0);
        else
            store_acc32<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * P::WM, n0 + wn * P::WN, acc,
                                     vec_store != 0);
    }
}

// MFMA shape of the 4-wave and of the 8-wave kernels (16 = v_mfma_f32_16x16x32_bf16,
// 32 = v_mfma_f32_32x32x16_bf16); 16 measured faster for both on MI355X.
#ifndef TMM_MFMA
#define TMM_MFMA 16
#endif

#ifndef TMM_SPEC_MFMA
#define TMM_SPEC_MFMA 16
#endif

template <int BM, int BN, int BK, int STAGES, int SWZ, bool XCD, int MF = TMM_MFMA, int WM = 2, int WN = 2>
static hipError_t launch_pipe_cfg(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    constexpr int THREADS = 64 * WM * WN;
    const bool ragged = (g.K & 7) != 0;
#define TMM_LAUNCH(O, R)                                                                          \
    hipLaunchKernelGGL((gemm_pipe_kernel<BM, BN, BK, STAGES, SWZ, MF, O, XCD, WM, WN, R>), dim3(p.grid_x), \
                       dim3(THREADS), 0, s, g, p.grid, p.vec_store)
    if (out == OUT_F32 && ragged) {
        TMM_LAUNCH(OUT_F32, true);
    } else if (out == OUT_F32) {
        TMM_LAUNCH(OUT_F32, false);
    } else if (ragged) {
        TMM_LAUNCH(OUT_BF16, true);
    } else {
        TMM_LAUNCH(OUT_BF16, false);
    }
#undef TMM_LAUNCH
    return hipGetLastError();
}

// Ring shape of the two tile sizes: K block, ring depth, swizzle pattern.
#ifndef TMM_BIG_BK
#define TMM_BIG_BK 64
#endif
#ifndef TMM_BIG_STAGES
#define TMM_BIG_STAGES 2
#endif
#ifndef TMM_SMALL_BK
#define TMM_SMALL_BK 64
#endif
#ifndef TMM_SMALL_STAGES
#define TMM_SMALL_STAGES 3
#endif
#ifndef TMM_SWZ
#define TMM_SWZ 1
#endif

hipError_t launch_pipe(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    constexpr int BBK = TMM_BIG_BK, BST = TMM_BIG_STAGES, SBK = TMM_SMALL_BK, SST = TMM_SMALL_STAGES;
    constexpr int SWZ = TMM_SWZ;
    switch (p.kernel) {
        case K_PIPE_256: return launch_pipe_cfg<256, 256, BBK, BST, SWZ, false>(g, out, p, s);
        case K_PIPE_128: return launch_pipe_cfg<128, 128, SBK, SST, SWZ, false>(g, out, p, s);
        case K_PERSIST_256: return launch_pipe_cfg<256, 256, BBK, BST, SWZ, true>(g, out, p, s);
        case K_PERSIST_128: return launch_pipe_cfg<128, 128, SBK, SST, SWZ, true>(g, out, p, s);
        // Two consumer groups of four waves (rows 0-127 and 128-255) share each B stage.
        case K_SPEC_256:
            return launch_pipe_cfg<256, 256, BBK, BST, SWZ, true, TMM_SPEC_MFMA, 2, 4>(g, out, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tmm
