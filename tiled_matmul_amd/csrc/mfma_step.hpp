// MFMA building blocks shared by the pipelined GEMM kernels: the two bf16 MFMA shapes of
// gfx950 (as builtins, and the 16x16x32 shape as inline assembly with AGPR accumulators),
// register fragments, and one k step of MFMAs interleaved with fragment reads and tile
// loads.  Internal to libgemm_bf16.so.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace tmm {

// The two bf16 MFMA shapes of gfx950.  ROWS x ROWS output block per instruction, KS = k
// depth per instruction; lane l supplies row (l % ROWS) and the 8-element k chunk
// (l / ROWS) of each operand.
template <int MF>
struct Mma;
template <>
struct Mma<16> {
    static constexpr int ROWS = 16, KS = 32;
    typedef f32x4 Acc;
    static __device__ __forceinline__ Acc run(bf16x8 a, bf16x8 b, Acc c) { return mfma_16x16x32(a, b, c); }
    static __device__ __forceinline__ Acc zero() { return Acc{0.f, 0.f, 0.f, 0.f}; }
};
template <>
struct Mma<32> {
    static constexpr int ROWS = 32, KS = 16;
    typedef f32x16 Acc;
    static __device__ __forceinline__ Acc run(bf16x8 a, bf16x8 b, Acc c) { return mfma_32x32x16(a, b, c); }
    static __device__ __forceinline__ Acc zero() {
        Acc z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0.f;
        return z;
    }
};

// One k step of MFMAs on fragments `f`, with NR fragment reads (rd(q)) and NG load issues
// (ld(q)) for later steps placed between the MFMAs.  sched_barrier fences fix this order:
// LDS reads issued in one burst fill the LDS command FIFO and, since a wave issues in order,
// stall the MFMAs queued behind them.  With FINE, read q goes before MFMA
// q (NM - TAIL) / NR, so the last TAIL MFMAs of the step cover the latency of the last reads
// (the next step waits for all of them), and load q goes before MFMA q NM / NG.
// FINE = false keeps the reads and loads in one group ahead of the MFMAs (the 4-wave kernel
// of gemm_pipe.hip, whose 256 builtin accumulators leave LLVM too few registers to
// interleave without copies).
// MM: the MFMA policy (default: the builtin shape that matches Acc).
template <int FN, int FM, int NR, int NG, bool FINE, typename MM = void, int TAIL = -1, typename Acc, typename F,
          typename RD, typename LD>
__device__ __forceinline__ void step(Acc (&acc)[FN][FM], const F& f, RD rd, LD ld) {
    using M = std::conditional_t<std::is_void_v<MM>, Mma<(sizeof(Acc) == 16 ? 16 : 32)>, MM>;
    constexpr int NM = FN * FM;
    if constexpr (!FINE) {
#pragma unroll
        for (int q = 0; q < NR; ++q) rd(q);
#pragma unroll
        for (int q = 0; q < NG; ++q) ld(q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m / FM][m % FM] = M::run(f.b[m / FM], f.a[m % FM], acc[m / FM][m % FM]);
        __builtin_amdgcn_sched_barrier(0);
        return;
    } else if constexpr (TAIL < 0) {
        // Slots: max(NR, NG) groups of MFMAs, read q and load q at the head of group q.
        constexpr int SLOTS = NR > NG ? NR : NG;
        static_assert(NM >= SLOTS, "needs at least one MFMA per slot");
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) {
            if (q < NR) rd(q);
            if (q < NG) ld(q);
            __builtin_amdgcn_sched_barrier(0);
            constexpr int base = NM / SLOTS, extra = NM % SLOTS;
            const int m0 = q * base + (q < extra ? q : extra);
            const int m1 = m0 + base + (q < extra ? 1 : 0);
#pragma unroll
            for (int m = m0; m < m1; ++m) {
                const int i = m / FM, j = m % FM;
                acc[i][j] = M::run(f.b[i], f.a[j], acc[i][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // f may hold KH sub-steps of fragments (b[KH FN], a[KH FM]): MFMA m uses sub-step
        // m / (FN FM).
        constexpr int KH = static_cast<int>(sizeof(f.b) / sizeof(f.b[0])) / FN;
        constexpr int NMK = NM * KH;
        static_assert(TAIL < NMK, "reads need MFMAs to hide behind");
        constexpr int D = NMK - TAIL;
#pragma unroll
        for (int m = 0; m < NMK; ++m) {
            // reads q with q D / NR == m, loads q with q NMK / NG == m
            const int r0 = m < D ? (m * NR + D - 1) / D : NR, r1 = m < D ? ((m + 1) * NR + D - 1) / D : NR;
            const int g0 = (m * NG + NMK - 1) / NMK, g1 = ((m + 1) * NG + NMK - 1) / NMK;
#pragma unroll
            for (int q = r0; q < (r1 < NR ? r1 : NR); ++q) rd(q);
#pragma unroll
            for (int q = g0; q < (g1 < NG ? g1 : NG); ++q) ld(q);
            __builtin_amdgcn_sched_barrier(0);
            const int h = m / NM, i = (m % NM) / FM, j = m % FM;
            acc[i][j] = M::run(f.b[h * FN + i], f.a[h * FM + j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Register fragments of one k step of a wave: FN fragments of the B tile (the MFMA's first
// operand) and FM of the A tile (its second).
template <int FN, int FM>
struct Frags {
    bf16x8 b[FN];
    bf16x8 a[FM];
};

// v_mfma_f32_16x16x32_bf16 as inline assembly with the accumulator pinned to AGPRs ("+a").
// With 256 accumulators per lane (a 128 x 128 wave tile), LLVM then keeps every accumulator
// in AGPRs and the fragments in VGPRs and interleaves reads and loads with the MFMAs without
// copies between the two files.  The compiler's hazard checks do not see into the assembly:
// agpr_fence() must separate these MFMAs from any ordinary instruction that writes or reads
// their accumulators.
struct MmaAsm16 {
    static constexpr int ROWS = 16, KS = 32;
    typedef f32x4 Acc;
    static __device__ __forceinline__ Acc run(bf16x8 a, bf16x8 b, Acc c) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
        return c;
    }
    static __device__ __forceinline__ Acc zero() { return Acc{0.f, 0.f, 0.f, 0.f}; }
};

// v_mfma_f32_32x32x16_bf16 the same way (16 AGPRs per accumulator).
struct MmaAsm32 {
    static constexpr int ROWS = 32, KS = 16;
    typedef f32x16 Acc;
    static __device__ __forceinline__ Acc run(bf16x8 a, bf16x8 b, Acc c) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
        return c;
    }
    static __device__ __forceinline__ Acc zero() { return Mma<32>::zero(); }
};

// Every accumulator passes through an empty assembly statement before and after 24 wait
// states (more than the longest MFMA-result hazard on gfx950).  Volatile assembly keeps its
// order, so whatever produced an accumulator precedes the wait states and whatever consumes
// it follows them.
template <int FN, int FM, typename Acc>
__device__ __forceinline__ void agpr_fence(Acc (&acc)[FN][FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) asm volatile("" : "+a"(acc[i][j]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) asm volatile("" : "+a"(acc[i][j]));
}

}  // namespace tmm
