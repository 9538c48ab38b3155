// Persistent 256 x 256 GEMM, C = A * B^T (bf16 in, fp32 accumulate), with separate LDS rings
// for the A and B tiles: ladder steps 4-6 with the loads spread evenly over the K loop.
//
// Prior art is the page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "9 步优化"
// (steps 4-6: asynchronous tile copies into a staging ring, overlap of the next block's copy
// with the current block's math, a persistent workgroup per SM).  The kernels of
// gemm_pipe.hip issue a whole 64-deep block of direct-to-LDS loads (64 KB) in the half of the
// block that follows its barrier, because only then is a slot free.  Here the A tile has a
// three-slot ring and the B tile a two-slot ring (3 x 32 KB + 2 x 32 KB = the whole 160 KB of
// LDS), and each of a block's two k steps issues one half of a later block's loads:
//
//   iteration b (A(j), B(j): the A and B tiles of 64-deep block j; A(j) in slot j mod 3,
//   B(j) in slot j mod 2):
//     step 0: MFMAs on block b's first 32 k, read the fragments of its second 32 k,
//             load A(b+2) (into the slot of A(b-1))
//     wait until this wave's loads of A(b+1) and B(b+1) have landed; barrier
//     step 1: MFMAs on block b's second 32 k, read block b+1's first fragments,
//             load B(b+2) (into the slot of B(b))
//
// At the barrier every wave has finished reading block b and every wave's share of block b+1
// is in LDS.  A(b-1)'s slot has been free since the previous barrier; B(b)'s is free from
// this one.  Rows stay 128 bytes (64 k), so every load instruction fetches 8 whole cache
// lines.
//
// Two wave layouts: eight waves (2 x 4, 128 x 64 each, two waves per SIMD, builtin MFMAs)
// and four waves (2 x 2, 128 x 128 each, one wave per SIMD, a third less LDS read traffic
// per MFMA; the MFMAs are inline assembly with AGPR accumulators so that LLVM interleaves
// the reads and loads without register copies).  16-byte chunk c of LDS row r sits in slot
// c XOR (r mod 8).
//
// Preconditions (planner): A, B 4-byte aligned with even pitches and strides, 256 * ld * 2
// below 2^31.  A ragged K tail (K mod 8 != 0) is staged through LDS as one extra k step.
#include "launch.hpp"
#include "mfma_step.hpp"

namespace tmm {

// MFMAs after each k step's last fragment read (see step()); measured on MI355X: 16 for the
// 4-wave layout (1-2% faster than reads spread to the end of the step; 24-40 no better), 0
// for the 8-wave layout.
#ifndef TMM_RING4_TAIL
#define TMM_RING4_TAIL 16
#endif
#ifndef TMM_RING8_TAIL
#define TMM_RING8_TAIL 0
#endif

namespace rg {
constexpr int BM = 256, BN = 256, BK = 64, NA = 3, NB = 2;
constexpr int ROWB = BK * 2;                        // bytes per LDS row
constexpr int TILE = 256 * ROWB;                    // one A or B tile of one block: 32 KB
constexpr int B_BASE = NA * TILE;                   // B slots follow the A slots
constexpr int R = 8;                                // LDS rows per wave load instruction
static_assert((NA + NB) * TILE <= 160 * 1024, "LDS capacity");
__device__ __forceinline__ int swz(int r) { return r & 7; }
}  // namespace rg

// MF: MFMA shape (16: v_mfma_f32_16x16x32_bf16, one per 32-deep k step and accumulator;
// 32: v_mfma_f32_32x32x16_bf16, two per k step).
template <int OUT, bool RAGGED, int WAVES_M, int WAVES_N, bool ASM, int MF>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, WAVES_M * WAVES_N / 4) void gemm_ring_kernel(
    GemmArgs g, TileGrid tg, int vec_store) {
    using namespace rg;
    using MM = std::conditional_t<MF == 16, std::conditional_t<ASM, MmaAsm16, Mma<16>>,
                                  std::conditional_t<ASM, MmaAsm32, Mma<32>>>;
    using Acc = typename MM::Acc;
    constexpr int KH = 32 / MM::KS;             // MFMAs per accumulator per 32-deep k step
    constexpr int CPM = MM::KS / 8;             // 16-byte k chunks per MFMA operand row
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, FM = WM / MF, FN = WN / MF;
    // MFMAs at the end of each k step that follow the step's last fragment read.
    constexpr int RTAIL = NW == 4 ? TMM_RING4_TAIL : TMM_RING8_TAIL;
    constexpr int L = 256 / (NW * R);   // load instructions per wave for one A (or B) tile
    static_assert(L * NW * R == 256, "rows split over the waves");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[(NA + NB) * TILE];

    const int lane = lane_id(), w = wave_id();
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const uint32_t K = static_cast<uint32_t>(g.K);
    const uint32_t K8 = RAGGED ? K & ~7u : K;
    const int nk = static_cast<int>((g.K + BK - 1) / BK);

    // Load i of wave w: tile rows (NW i + w) R + lane / 8; the lane writes physical chunk
    // lane % 8, i.e. fetches logical chunk (lane % 8) ^ swz(row).  R = 8, so swz(row) =
    // lane / 8 for every i.
    const int lrow = lane / 8;
    const uint32_t chunk_k = 8u * static_cast<uint32_t>((lane % 8) ^ swz(lrow));
    // Fragment reads of sub-step h of k step kk: row lane % MF of an MF-row block, logical
    // chunk 4 kk + CPM h + lane / MF.
    int rd[2][KH];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < KH; ++h)
            rd[kk][h] = (lane % MF) * ROWB + (((4 * kk + CPM * h + lane / MF) ^ swz(lane % MF)) * 16);
    const int a_off = wm * WM * ROWB, b_off = wn * WN * ROWB;

    for (int t = blockIdx.x; t < tg.total; t += gridDim.x) {
        int bt, tm, tn;
        tile_of(t, tg, bt, tm, tn);
        const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
        const int64_t rows_a = min<int64_t>(BM, g.M - m0), rows_b = min<int64_t>(BN, g.N - n0);
        const uint16_t* Ab = g.A + bt * g.sA + m0 * g.lda;
        const uint16_t* Bb = g.B + bt * g.sB + n0 * g.ldb;
        const auto ra = make_rsrc(Ab, static_cast<uint32_t>(((rows_a - 1) * g.lda + g.K) * 2));
        const auto rb = make_rsrc(Bb, static_cast<uint32_t>(((rows_b - 1) * g.ldb + g.K) * 2));
        uint32_t va[L], vb[L];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int r = (NW * i + w) * R + lrow;
            va[i] = r < rows_a ? static_cast<uint32_t>(r * g.lda) * 2u + 2u * chunk_k : OOB;
            vb[i] = r < rows_b ? static_cast<uint32_t>(r * g.ldb) * 2u + 2u * chunk_k : OOB;
        }

        // Load instruction q of the A (IS_A) or B tile of block j into the tile at LDS byte
        // offset `dst` (chunks at k >= K8 read zeros; blocks past the end read zeros).
        auto load_one = [&](bool is_a, int q, int j, int dst) {
            const uint32_t k0 = static_cast<uint32_t>(j) * BK;
            const bool ok = k0 + chunk_k < K8;
            load_lds_16(is_a ? ra : rb, lds + dst + (NW * q + w) * R * ROWB, ok ? (is_a ? va[q] : vb[q]) : OOB,
                        2u * k0);
        };
        // Fragment q of k step kk from the A tile at `at` and the B tile at `bt_`: q < KH FN:
        // B fragment q % FN of sub-step q / FN, else A fragment (q - KH FN) % FM of sub-step
        // (q - KH FN) / FM.
        using F = Frags<KH * FN, KH * FM>;
        auto read_one = [&](F& f, int q, int at, int bt_, int kk) {
            if (q < KH * FN) {
                const int h = q / FN, i = q % FN;
                f.b[q] = *reinterpret_cast<const bf16x8*>(lds + bt_ + b_off + MF * i * ROWB + rd[kk][h]);
            } else {
                const int r = q - KH * FN, h = r / FM, j = r % FM;
                f.a[r] = *reinterpret_cast<const bf16x8*>(lds + at + a_off + MF * j * ROWB + rd[kk][h]);
            }
        };
        constexpr int NR = KH * (FN + FM);

        Acc acc[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = MM::zero();
        if constexpr (ASM) agpr_fence(acc);

        // Prologue: A(0), B(0), A(1), B(1); block 0 complete (this wave), barrier (every
        // wave's), then block 0's first fragments.  (Every wave has passed the previous
        // tile's final barrier, so both rings are free.)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int q = 0; q < L; ++q) load_one(true, q, j, j * TILE);
#pragma unroll
            for (int q = 0; q < L; ++q) load_one(false, q, j, B_BASE + j * TILE);
        }
        wait_vmcnt<2 * L>();
        barrier();
        F f[2];
#pragma unroll
        for (int q = 0; q < NR; ++q) read_one(f[0], q, 0, B_BASE, 0);
        wait_cnt<63, 0>();

        // a0, a1, a2: A slots of blocks b, b+1, b+2; b0, b1: B slots of blocks b, b+1.
        int a0 = 0, a1 = TILE, a2 = 2 * TILE, b0 = B_BASE, b1 = B_BASE + TILE;
        for (int b = 0; b < nk; ++b) {
            step<FN, FM, NR, L, true, MM, RTAIL>(acc, f[0], [&](int q) { read_one(f[1], q, a0, b0, 1); },
                                               [&](int q) { load_one(true, q, b + 2, a2); });
            wait_cnt<L, 0>();   // everything but this step's A(b+2) loads has landed
            barrier();
            step<FN, FM, NR, L, true, MM, RTAIL>(acc, f[1], [&](int q) { read_one(f[0], q, a1, b1, 0); },
                                               [&](int q) { load_one(false, q, b + 2, b0); });
            __builtin_amdgcn_sched_barrier(0);
            wait_cnt<63, 0>();
            __builtin_amdgcn_sched_barrier(0);
            const int at = a0;
            a0 = a1, a1 = a2, a2 = at;
            const int bt_ = b0;
            b0 = b1, b1 = bt_;
        }
        wait_vmcnt<0>();   // the trailing zero-fill loads have landed
        barrier();         // every fragment read of this tile is done: the rings are free

        if constexpr (RAGGED) {
            // Elements K8 .. K - 1 of every row, element by element (nothing at or beyond K is
            // read), as chunk 0 of one more 32-deep step (A in A slot 0, B in B slot 0);
            // chunks 1-3 are zero.
            for (int r = threadIdx.x; r < BM + BN; r += 64 * NW) {
                const bool is_a = r < BM;
                const int rr = is_a ? r : r - BM;
                uint32_t hv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (rr < (is_a ? rows_a : rows_b)) {
                    const uint16_t* row = is_a ? Ab + rr * g.lda : Bb + rr * g.ldb;
#pragma unroll
                    for (int e = 0; e < 7; ++e)
                        if (K8 + e < K) hv[e] = row[K8 + e];
                }
                uint8_t* dst = lds + (is_a ? 0 : B_BASE) + rr * ROWB;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 v = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                 hv[6] | (hv[7] << 16)};
#pragma unroll
                for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(dst + ((c ^ swz(rr)) * 16)) = c == 0 ? v : z;
            }
            barrier();
#pragma unroll
            for (int q = 0; q < NR; ++q) read_one(f[0], q, 0, B_BASE, 0);
            wait_cnt<63, 0>();
#pragma unroll
            for (int h = 0; h < KH; ++h)
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j) acc[i][j] = MM::run(f[0].b[h * FN + i], f[0].a[h * FM + j], acc[i][j]);
            barrier();   // read before the next tile refills the rings
        }
        if constexpr (ASM) agpr_fence(acc);

        void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                  : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
        if constexpr (MF == 16)
            store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, vec_store != 0);
        else
            store_acc32<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, vec_store != 0);
    }
}

template <int WM, int WN, bool ASM, int MF>
static hipError_t launch_ring_cfg(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    const bool ragged = (g.K & 7) != 0;
    const dim3 grid(p.grid_x), block(64 * WM * WN);
    if (out == OUT_F32 && ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_F32, true, WM, WN, ASM, MF>), grid, block, 0, s, g, p.grid, p.vec_store);
    else if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_F32, false, WM, WN, ASM, MF>), grid, block, 0, s, g, p.grid, p.vec_store);
    else if (ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_BF16, true, WM, WN, ASM, MF>), grid, block, 0, s, g, p.grid, p.vec_store);
    else
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_BF16, false, WM, WN, ASM, MF>), grid, block, 0, s, g, p.grid, p.vec_store);
    return hipGetLastError();
}

// MFMA shape of the ring kernels (16 or 32; v_mfma_f32_32x32x16_bf16 measured 5-7% slower on
// MI355X for both layouts).
#ifndef TMM_RING4_MFMA
#define TMM_RING4_MFMA 16
#endif
#ifndef TMM_RING8_MFMA
#define TMM_RING8_MFMA 16
#endif

hipError_t launch_ring(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    switch (p.kernel) {
        case K_RING8_256: return launch_ring_cfg<2, 4, false, TMM_RING8_MFMA>(g, out, p, s);
        case K_RING4_256: return launch_ring_cfg<2, 2, true, TMM_RING4_MFMA>(g, out, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tmm
