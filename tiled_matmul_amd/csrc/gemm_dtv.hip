// Persistent 256 x 256 GEMM, C = A * B^T (bf16 in, fp32 accumulate), whose A operand goes
// from global memory straight into the MFMA fragment registers; only the B tile is staged in
// LDS.
//
// Prior art is the page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "9 步优化"
// (steps 4-6: asynchronous tile copies into a staging ring overlapped with the math, a
// persistent workgroup per SM) and section "Roofline" (the fix for a starved math unit is
// fewer bytes moved per product).  In the ring kernels both tiles pass through LDS: per
// 64-deep block a CU writes 64 KB into LDS and its four waves read 128 KB of fragments back,
// against 2048 MFMA cycles, and LDS traffic is what holds those kernels below the MFMA rate.
// Here each wave of the 2 x 2 layout (128 x 128 per wave) loads its own A fragments with
// 16-byte buffer loads in the MFMA operand layout (lane l: row l % 16 of a 16-row fragment,
// elements 8 (l / 16) .. + 7 of a 32-deep k step), so per block the LDS carries 32 KB of
// B writes and 64 KB of B fragment reads: half of both.  The two waves that share A rows
// each load them (the L2 serves the second read).
//
//   k step s (block b = s / 2, half kk = s mod 2) of a tile:
//     MFMAs on the B fragments read in step s - 1 and the A fragments of register set s mod 4;
//     between them: the B fragments of step s + 1 (LDS), the A fragments of step s + 3 into
//     register set (s + 3) mod 4 (the set step s - 1 used), and half of the B tile of block
//     b + 3 into LDS slot (b + 3) mod 4 (the slot of block b - 1, whose last fragment reads
//     preceded the barrier of block b - 1).
//     Before each step: every load issued up to step s - 3 has landed; in the middle of each
//     block (between its two steps): a barrier, after which block b + 1's B tile is complete.
//
// 12 loads per step (8 A fragments, 4 B load instructions), so "landed up to step s - 3"
// is s_waitcnt vmcnt(24).  The K loop runs over an even number of blocks; a block past the
// end of K reads zeros (buffer loads out of range) and adds nothing.
//
// Preconditions (planner): both operands K-major, 16-byte aligned, pitches, batch strides and
// K multiples of 8, 256 * ld * 2 below 2^31.
#include <type_traits>

#include "launch.hpp"
#include "mfma_step.hpp"

namespace tmm {

// MFMAs of each k step after its last B fragment read (they cover that read's latency).
#ifndef TMM_DTV_TAIL
#define TMM_DTV_TAIL 16
#endif

namespace dv {
constexpr int BK = 64, NB = 4, ROWB = BK * 2, TILE = 256 * ROWB, R = 8;
constexpr int FN = 8, FM = 8;            // 16-row fragments per wave and k step: B (n), A (m)
constexpr int LB = 256 / (4 * R);        // B load instructions per wave for one block
constexpr int NLD = FM + LB / 2;         // loads per k step
constexpr int WAIT = 2 * NLD;            // loads that may be in flight at the start of a step
static_assert(NB * TILE <= 160 * 1024, "LDS capacity");
}  // namespace dv

template <int OUT>
__global__ __launch_bounds__(256, 1) void gemm_dtv_kernel(GemmArgs g, TileGrid tg, int vec_store) {
    using namespace dv;
    using MM = MmaAsm16;
    using Acc = MM::Acc;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NB * TILE];

    const int lane = lane_id(), w = wave_id();
    const int wm = w >> 1, wn = w & 1;
    const uint32_t K = static_cast<uint32_t>(g.K);
    const int nk = static_cast<int>((g.K + BK - 1) / BK);
    const int nk2 = (nk + 1) & ~1;

    // B load i of wave w fills LDS rows (4 i + w) R + lane / 8 of a slot; 16-byte chunk c of
    // row r sits at physical chunk c ^ (r mod 8), so the lane (physical chunk lane % 8)
    // fetches logical chunk (lane % 8) ^ (lane / 8).
    const uint32_t bchunk = 8u * static_cast<uint32_t>((lane & 7) ^ (lane >> 3));
    // B fragment of k step kk: row lane % 16 of a 16-row block, logical chunk 4 kk + lane / 16.
    int rdo[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) rdo[kk] = (lane & 15) * ROWB + (((4 * kk + (lane >> 4)) ^ (lane & 7)) * 16);
    const int b_off = wn * 128 * ROWB;
    // A fragment j of k step kk: row 16 j + lane % 16 of the wave's 128 rows, elements
    // 32 kk + acol .. + 7 of the block.
    const uint32_t acol = 8u * static_cast<uint32_t>(lane >> 4);

    for (int t = blockIdx.x; t < tg.total; t += gridDim.x) {
        int bt, tm, tn;
        tile_of(t, tg, bt, tm, tn);
        const int64_t m0 = static_cast<int64_t>(tm) * 256, n0 = static_cast<int64_t>(tn) * 256;
        const int64_t rows_a = min<int64_t>(256, g.M - m0), rows_b = min<int64_t>(256, g.N - n0);
        const uint16_t* Ab = g.A + bt * g.sA + m0 * g.lda;
        const uint16_t* Bb = g.B + bt * g.sB + n0 * g.ldb;
        const auto ra = make_rsrc(Ab, static_cast<uint32_t>(((rows_a - 1) * g.lda + g.K) * 2));
        const auto rb = make_rsrc(Bb, static_cast<uint32_t>(((rows_b - 1) * g.ldb + g.K) * 2));
        uint32_t va[FM], vb[LB];   // per-lane byte offsets (rows outside the tile: OOB)
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int r = wm * 128 + 16 * j + (lane & 15);
            va[j] = r < rows_a ? static_cast<uint32_t>(r * g.lda) * 2u + 2u * acol : OOB;
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            const int r = (4 * i + w) * R + (lane >> 3);
            vb[i] = r < rows_b ? static_cast<uint32_t>(r * g.ldb) * 2u + 2u * bchunk : OOB;
        }

        // A fragment j of k step s into x (elements at or beyond K read zeros).
        auto load_a = [&](bf16x8& x, int j, int s) {
            const uint32_t k0 = static_cast<uint32_t>(s >> 1) * BK, kk = static_cast<uint32_t>(s & 1);
            const bool ok = k0 + 32u * kk + acol < K;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? va[j] + 64u * kk : OOB, 2u * k0, 0);
            x = __builtin_bit_cast(bf16x8, v);
        };
        // B load instruction q of block b into its LDS slot.
        auto load_b = [&](int q, int b) {
            const uint32_t k0 = static_cast<uint32_t>(b) * BK;
            const bool ok = k0 + bchunk < K;
            load_lds_16(rb, lds + (b & (NB - 1)) * TILE + (4 * q + w) * R * ROWB, ok ? vb[q] : OOB, 2u * k0);
        };
        // B fragment i of k step s.
        auto read_b = [&](int i, int s) {
            return *reinterpret_cast<const bf16x8*>(lds + ((s >> 1) & (NB - 1)) * TILE + b_off + 16 * i * ROWB +
                                                    rdo[s & 1]);
        };

        Acc acc[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = MM::zero();
        agpr_fence(acc);

        bf16x8 X[4][FM];    // A fragments of k steps s with s mod 4 = 0 .. 3
        bf16x8 Fb[2][FN];   // B fragments of k steps s with s mod 2 = 0, 1

        // Prologue: B(0), A of steps 0 and 1, B(1), A of step 2, B(2) (48 loads); then B(0)
        // and step 0's A have landed (32 in flight), barrier, step 0's B fragments.
#pragma unroll
        for (int q = 0; q < LB; ++q) load_b(q, 0);
#pragma unroll
        for (int j = 0; j < FM; ++j) load_a(X[0][j], j, 0);
#pragma unroll
        for (int j = 0; j < FM; ++j) load_a(X[1][j], j, 1);
#pragma unroll
        for (int q = 0; q < LB; ++q) load_b(q, 1);
#pragma unroll
        for (int j = 0; j < FM; ++j) load_a(X[2][j], j, 2);
#pragma unroll
        for (int q = 0; q < LB; ++q) load_b(q, 2);
        wait_vmcnt<32>();
        barrier();
#pragma unroll
        for (int i = 0; i < FN; ++i) Fb[0][i] = read_b(i, 0);
        wait_cnt<63, 0>();

        // One k step with A register set P = s mod 4 (see the header for the schedule).
        auto kstep = [&](auto Pc, int s) {
            constexpr int P = decltype(Pc)::value, PF = P & 1, PL = (P + 3) & 3;
            constexpr int NM = FN * FM, TAIL = TMM_DTV_TAIL, D = NM - TAIL;
            static_assert(TAIL >= 0 && TAIL < NM, "reads need MFMAs to hide behind");
            const int bl = (s >> 1) + 3, qb = LB / 2 * (s & 1);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int r0 = m < D ? (m * FN + D - 1) / D : FN, r1 = m < D ? ((m + 1) * FN + D - 1) / D : FN;
                const int g0 = (m * NLD + NM - 1) / NM, g1 = ((m + 1) * NLD + NM - 1) / NM;
#pragma unroll
                for (int q = r0; q < (r1 < FN ? r1 : FN); ++q) Fb[PF ^ 1][q] = read_b(q, s + 1);
#pragma unroll
                for (int q = g0; q < (g1 < NLD ? g1 : NLD); ++q) {
                    if (q < FM)
                        load_a(X[PL][q], q, s + 3);
                    else
                        load_b(qb + q - FM, bl);
                }
                __builtin_amdgcn_sched_barrier(0);
                acc[m / FM][m % FM] = MM::run(Fb[PF][m / FM], X[P][m % FM], acc[m / FM][m % FM]);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_cnt<63, 0>();   // step s + 1's B fragments are in registers
            __builtin_amdgcn_sched_barrier(0);
        };

        for (int b = 0; b < nk2; b += 2) {
            const int s = 2 * b;
            wait_vmcnt<WAIT>();
            kstep(std::integral_constant<int, 0>{}, s);
            wait_vmcnt<WAIT>();
            barrier();
            kstep(std::integral_constant<int, 1>{}, s + 1);
            wait_vmcnt<WAIT>();
            kstep(std::integral_constant<int, 2>{}, s + 2);
            wait_vmcnt<WAIT>();
            barrier();
            kstep(std::integral_constant<int, 3>{}, s + 3);
        }
        wait_vmcnt<0>();   // the loads that ran past the end have landed
        barrier();         // every fragment read of this tile is done: the ring is free
        agpr_fence(acc);

        void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                  : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
        store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * 128, n0 + wn * 128, acc, vec_store != 0);
    }
}

hipError_t launch_dtv(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    const dim3 grid(p.grid_x), block(256);
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_dtv_kernel<OUT_F32>), grid, block, 0, s, g, p.grid, p.vec_store);
    else
        hipLaunchKernelGGL((gemm_dtv_kernel<OUT_BF16>), grid, block, 0, s, g, p.grid, p.vec_store);
    return hipGetLastError();
}

}  // namespace tmm
