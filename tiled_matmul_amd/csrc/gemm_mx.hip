// Block-scaled low-precision GEMM: C = A * B^T with A (M x K) and B (N x K) in an 8-bit
// floating-point format (E4M3 or E5M2) and one power-of-two scale (E8M0) per 32 consecutive
// k of a row, fp32 accumulate, fp32 or bf16 out.
//
// The page "Modern GPU Programming for MLSys：深度解读", section "背景", names low-precision
// block-scaled GEMM among the kernel families that decide training and serving speed; the
// format taken here is the OCP microscaling one (blocks of 32, E8M0 scales), which gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 computes natively.
//
// mx_ring_kernel is the 4-wave ring kernel of gemm_ring.hip with bytes for elements: a
// 256 x 128-byte LDS row holds 128 k, so the ring geometry (A: 3 slots, B: 2 slots of 32 KB)
// and the direct-to-LDS loads are unchanged (the swizzle differs: a fragment read here spans
// 32 rows, not 16); a 128-deep block is two 64-deep k steps of 32 x 32 x 64 MFMAs.  Operand layout of that MFMA, measured on MI355X with an
// in-bounds probe: lane l supplies row l % 32; with g = l / 32, bytes 0-15 of its 32 are
// k = 16 g .. 16 g + 15 and bytes 16-31 are k = 32 + 16 g .. 32 + 16 g + 15 of the 64-deep
// step, and the scale operand of lane group h applies to k = 32 h .. 32 h + 31.  So a lane
// reads 16-byte chunks 4 kk + g and 4 kk + 2 + g of its row and passes the scale of 32-block
// 2 kk + g of the 128-deep block.  The scales are not in LDS (the rings fill it): every lane
// needs, per fragment and block, the dword that holds its row's four 32-block scales, and
// shifts the byte it needs into place when it reads the fragment.  The two halves of the wave
// cover the same 32 rows, so one load fetches two blocks' dwords (the low half block j, the
// high half block j + 1) and a permlane32 swap gives every lane both.
//
// mx_simple_kernel: any K (multiple of 32), pitch and alignment; 64 x 64 tile per workgroup,
// each thread 4 x 4 outputs, operands decoded with the gfx950 conversion instructions and
// scaled with ldexp, fp32 FMA.
#include "launch.hpp"
#include "mfma_step.hpp"

namespace tmm {

// Scale dwords of two consecutive blocks per load (the halves of the wave load one block each,
// a permlane32 swap shares them): half the scale load instructions.
#ifndef TMM_MX_SCALE_PAIRS
#define TMM_MX_SCALE_PAIRS 1
#endif

// MFMAs at the end of each k step that follow its last fragment read (see step()).
#ifndef TMM_MX_TAIL
#define TMM_MX_TAIL 8
#endif

namespace mx {
constexpr int BM = 256, BN = 256, BKB = 128, NA = 3, NB = 2;   // BKB: bytes (= k) per block
constexpr int ROWB = BKB;
constexpr int TILE = 256 * ROWB;
constexpr int B_BASE = NA * TILE;
constexpr int R = 8;   // LDS rows per wave load instruction
static_assert((NA + NB) * TILE <= 160 * 1024, "LDS capacity");
// LDS position of 16-byte chunk c of tile row r: c ^ swz(r).  A fragment read takes one chunk
// of 32 consecutive rows (two rows per 256-byte bank row); swz sends the rows that share a
// bank position to lanes 8, 34 or 42 apart, which the LDS serves without a conflict
// (measured: SQ_LDS_BANK_CONFLICT 0).  swz depends on bits 1, 2 and 4 of r only.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
}  // namespace mx

typedef __attribute__((ext_vector_type(8))) int i32x8;

// One MFMA operand: 32 bytes of one row and the scale (E8M0 in bits 0-7) of its 32-block.
struct MxFrag {
    i32x8 v;
    int s;
};
template <int FN, int FM>
struct MxFrags {
    MxFrag b[FN];
    MxFrag a[FM];
};

// The scaled 32 x 32 x 64 MFMA; the first operand is the B fragment (format FB), the second
// the A fragment (format FA).  Inline assembly with the accumulator pinned to AGPRs, as
// MmaAsm16: with the builtin and 256 accumulators per lane LLVM moves accumulators between
// the register files and spills.  agpr_fence() separates these MFMAs from ordinary
// instructions on the accumulators.  The scale operands are written by a VALU shift at least
// one k step's tail of MFMAs before the MFMA that reads them.
template <int FB, int FA>
struct MmaMx32 {
    static constexpr int ROWS = 32;
    typedef f32x16 Acc;
    static __device__ __forceinline__ Acc run(const MxFrag& b, const MxFrag& a, Acc c) {
        if constexpr (FB == MX_E4M3 && FA == MX_E4M3)
            asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                         : "+a"(c) : "v"(b.v), "v"(a.v), "v"(b.s), "v"(a.s));
        else if constexpr (FB == MX_E5M2 && FA == MX_E4M3)
            asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:1"
                         : "+a"(c) : "v"(b.v), "v"(a.v), "v"(b.s), "v"(a.s));
        else if constexpr (FB == MX_E4M3 && FA == MX_E5M2)
            asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] blgp:1"
                         : "+a"(c) : "v"(b.v), "v"(a.v), "v"(b.s), "v"(a.s));
        else
            asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:1 blgp:1"
                         : "+a"(c) : "v"(b.v), "v"(a.v), "v"(b.s), "v"(a.s));
        return c;
    }
};

template <int OUT, int FA, int FB>
__global__ __launch_bounds__(256, 1) void mx_ring_kernel(MxArgs g, TileGrid tg, int vec_store) {
    using namespace mx;
    using MM = MmaMx32<FB, FA>;
    using Acc = f32x16;
    constexpr int NW = 4, WAVES_N = 2;
    constexpr int WM = 128, WN = 128, FM = WM / 32, FN = WN / 32;
    constexpr int L = TILE / (NW * 1024);   // load instructions per wave per tile: 8
    constexpr int NR = 2 * (FN + FM);       // fragment reads per k step (two per fragment)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[(NA + NB) * TILE];

    const int lane = lane_id(), w = wave_id();
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const int nk = static_cast<int>(g.K / BKB);
    const int lg = lane >> 5;                 // lane group: 32-block 2 kk + lg of a k step
    const int lrow = lane / 8;
    // Every load of this lane writes a tile row congruent to 8 w + lrow modulo 32.
    const uint32_t chunk_b = 16u * static_cast<uint32_t>((lane % 8) ^ swz(8 * w + lrow));
    // Fragment read e (0, 1) of k step kk: row lane % 32 of the fragment, chunk 4 kk + 2 e + lg.
    int rd[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            rd[kk][e] = (lane % 32) * ROWB + (((4 * kk + 2 * e + lg) ^ swz(lane % 32)) * 16);
    const int a_off = wm * WM * ROWB, b_off = wn * WN * ROWB;

    for (int t = blockIdx.x; t < tg.total; t += gridDim.x) {
        int bt, tm, tn;
        tile_of(t, tg, bt, tm, tn);
        (void)bt;
        const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
        const int64_t rows_a = min<int64_t>(BM, g.M - m0), rows_b = min<int64_t>(BN, g.N - n0);
        const uint8_t* Ab = g.A + m0 * g.lda;
        const uint8_t* Bb = g.B + n0 * g.ldb;
        const auto ra = make_rsrc(Ab, static_cast<uint32_t>((rows_a - 1) * g.lda + g.K));
        const auto rb = make_rsrc(Bb, static_cast<uint32_t>((rows_b - 1) * g.ldb + g.K));
        const auto rsa = make_rsrc(g.SA + m0 * g.ldsa, static_cast<uint32_t>((rows_a - 1) * g.ldsa + g.K / 32));
        const auto rsb = make_rsrc(g.SB + n0 * g.ldsb, static_cast<uint32_t>((rows_b - 1) * g.ldsb + g.K / 32));
        // Byte offsets: load q of this lane reads tile row (NW q + w) R + lrow, i.e. va0 + q
        // strideA; fragment j's scale row wm WM + 32 j + lane % 32, i.e. sa0 + j sstrideA.
        // Rows at or beyond the tile's end fall outside the buffer resources (pitch >= K and
        // >= K / 32) and read zeros, so the offsets need no row test; the offsets stay below
        // 2^31 (256 rows times a pitch below 2^23).
        const uint32_t va0 = static_cast<uint32_t>((w * R + lrow) * g.lda) + chunk_b;
        const uint32_t vb0 = static_cast<uint32_t>((w * R + lrow) * g.ldb) + chunk_b;
        const uint32_t strideA = static_cast<uint32_t>(NW * R * g.lda), strideB = static_cast<uint32_t>(NW * R * g.ldb);
        const uint32_t sa0 = static_cast<uint32_t>((wm * WM + lane % 32) * g.ldsa);
        const uint32_t sb0 = static_cast<uint32_t>((wn * WN + lane % 32) * g.ldsb);
        const uint32_t sstrideA = static_cast<uint32_t>(32 * g.ldsa), sstrideB = static_cast<uint32_t>(32 * g.ldsb);

        // (The block index is wave-uniform; readfirstlane keeps the soffset operands in SGPRs,
        // which LLVM otherwise loses track of and serves with a per-lane loop.)
        auto load_one = [&](bool is_a, int q, int j, int dst) {
            j = __builtin_amdgcn_readfirstlane(j);
            const uint32_t k0 = static_cast<uint32_t>(j) * BKB;   // blocks past the end read zeros
            const bool ok = k0 < static_cast<uint32_t>(g.K);
            const uint32_t off = is_a ? va0 + q * strideA : vb0 + q * strideB;
            load_lds_16(is_a ? ra : rb, lds + dst + (NW * q + w) * R * ROWB, ok ? off : OOB, ok ? k0 : 0u);
        };
        // Scale dwords of block j for every fragment (FN of B, then FM of A).
        auto load_scales = [&](int q, int j, int (&sb)[FN], int (&sa)[FM]) {
            j = __builtin_amdgcn_readfirstlane(j);
            const uint32_t soff = j < nk ? static_cast<uint32_t>(j) * 4u : 0u;
            if (q < FN)
                sb[q] = __builtin_amdgcn_raw_buffer_load_b32(rsb, j < nk ? sb0 + q * sstrideB : OOB, soff, 0);
            else
                sa[q - FN] = __builtin_amdgcn_raw_buffer_load_b32(rsa, j < nk ? sa0 + (q - FN) * sstrideA : OOB, soff, 0);
        };
        // With TMM_MX_SCALE_PAIRS: scale dwords of blocks j (lanes 0-31) and j + 1 (lanes 32-63)
        // in one load per fragment; swap_scales then gives every lane both (the low half's
        // values in the first set, the high half's in the second).
        auto load_scale_pair = [&](int q, int j, int (&sb)[FN], int (&sa)[FM]) {
            j = __builtin_amdgcn_readfirstlane(j);
            const int jl = j + (lane >> 5);
            const uint32_t soff = j < nk ? static_cast<uint32_t>(j) * 4u : 0u;
            const uint32_t hi = static_cast<uint32_t>(lane >> 5) * 4u;
            if (q < FN)
                sb[q] = __builtin_amdgcn_raw_buffer_load_b32(rsb, jl < nk ? sb0 + q * sstrideB + hi : OOB, soff, 0);
            else
                sa[q - FN] = __builtin_amdgcn_raw_buffer_load_b32(rsa, jl < nk ? sa0 + (q - FN) * sstrideA + hi : OOB,
                                                                  soff, 0);
        };
        auto swap_scales = [&](int (&sb0_)[FN], int (&sa0_)[FM], int (&sb1_)[FN], int (&sa1_)[FM]) {
#pragma unroll
            for (int q = 0; q < FN; ++q) {
                const auto r = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(sb0_[q]),
                                                                static_cast<uint32_t>(sb0_[q]), false, false);
                sb0_[q] = static_cast<int>(r[0]), sb1_[q] = static_cast<int>(r[1]);
            }
#pragma unroll
            for (int q = 0; q < FM; ++q) {
                const auto r = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(sa0_[q]),
                                                                static_cast<uint32_t>(sa0_[q]), false, false);
                sa0_[q] = static_cast<int>(r[0]), sa1_[q] = static_cast<int>(r[1]);
            }
        };
        using F = MxFrags<FN, FM>;
        // Read q of k step kk (q / 2: fragment, B first; q % 2: which 16 bytes); with the first
        // read the fragment takes scale byte 2 kk + lg of its set entry.
        auto read_one = [&](F& f, int q, int at, int bt_, int kk, const int (&sb)[FN], const int (&sa)[FM]) {
            const int fr = q / 2, e = q % 2;
            MxFrag& x = fr < FN ? f.b[fr] : f.a[fr - FN];
            const int base = fr < FN ? bt_ + b_off + 32 * fr * ROWB : at + a_off + 32 * (fr - FN) * ROWB;
            const u32x4 v = *reinterpret_cast<const u32x4*>(lds + base + rd[kk][e]);
#pragma unroll
            for (int c = 0; c < 4; ++c) x.v[4 * e + c] = static_cast<int>(v[c]);
            if (e == 0) {
                const int s = fr < FN ? sb[fr] : sa[fr - FN];
                x.s = static_cast<int>(static_cast<uint32_t>(s) >> (8 * (2 * kk + lg)));
            }
        };
        Acc acc[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = Mma<32>::zero();
        agpr_fence(acc);

        // Scale sets: X holds block b's, Y block b+1's at the start of iteration b (b even;
        // the roles alternate).  Block b+2's are loaded into block b's set in step 1 of
        // iteration b, after its last use.
        int sbX[FN], saX[FM], sbY[FN], saY[FM];
        // Prologue: scales(0), A(0), B(0), scales(1), A(1), B(1), in this order (fenced: the
        // wait counts on it); all but A(1), B(1) complete.
#pragma unroll
        for (int q = 0; q < FN + FM; ++q) {
            if (TMM_MX_SCALE_PAIRS)
                load_scale_pair(q, 0, sbX, saX);
            else
                load_scales(q, 0, sbX, saX);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < L; ++q) load_one(true, q, 0, 0);
#pragma unroll
        for (int q = 0; q < L; ++q) load_one(false, q, 0, B_BASE);
        __builtin_amdgcn_sched_barrier(0);
        if (!TMM_MX_SCALE_PAIRS) {
#pragma unroll
            for (int q = 0; q < FN + FM; ++q) load_scales(q, 1, sbY, saY);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < L; ++q) load_one(true, q, 1, TILE);
#pragma unroll
        for (int q = 0; q < L; ++q) load_one(false, q, 1, B_BASE + TILE);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<2 * L>();
        barrier();
        if (TMM_MX_SCALE_PAIRS) swap_scales(sbX, saX, sbY, saY);
        F f[2];
#pragma unroll
        for (int q = 0; q < NR; ++q) read_one(f[0], q, 0, B_BASE, 0, sbX, saX);
        wait_cnt<63, 0>();

        int a0 = 0, a1 = TILE, a2 = 2 * TILE, b0 = B_BASE, b1 = B_BASE + TILE;
        // One iteration on block b with its scales in (sbC, saC) and block b+1's in (sbN, saN).
        // With scale pairs, an even iteration loads the pair (b+2, b+3) into block b's set and
        // the next (odd) one swaps it into the sets of blocks b+2 and b+3 once both are free.
        auto iteration = [&](auto odd, int b, int (&sbC)[FN], int (&saC)[FM], int (&sbN)[FN], int (&saN)[FM]) {
            constexpr bool ODD = decltype(odd)::value;
            step<FN, FM, NR, L, true, MM, TMM_MX_TAIL>(acc, f[0], [&](int q) { read_one(f[1], q, a0, b0, 1, sbC, saC); },
                                             [&](int q) { load_one(true, q, b + 2, a2); });
            wait_cnt<L, 0>();   // all but this step's A(b+2) loads: B(b+1), scales(b+1) landed
            barrier();
            constexpr bool PAIRS = TMM_MX_SCALE_PAIRS != 0;
            if constexpr (PAIRS && ODD) swap_scales(sbN, saN, sbC, saC);
            constexpr int NS = PAIRS && ODD ? 0 : FN + FM;   // scale loads in this step
            step<FN, FM, NR, L + NS, true, MM, TMM_MX_TAIL>(
                acc, f[1], [&](int q) { read_one(f[0], q, a1, b1, 0, sbN, saN); },
                [&](int q) {
                    // scales first: a wait LLVM places for them then leaves the B loads in flight
                    if (q < NS) {
                        if constexpr (PAIRS)
                            load_scale_pair(q, b + 2, sbC, saC);
                        else
                            load_scales(q, b + 2, sbC, saC);
                    } else {
                        load_one(false, q - NS, b + 2, b0);
                    }
                });
            __builtin_amdgcn_sched_barrier(0);
            wait_cnt<63, 0>();
            __builtin_amdgcn_sched_barrier(0);
            const int at = a0;
            a0 = a1, a1 = a2, a2 = at;
            const int bt_ = b0;
            b0 = b1, b1 = bt_;
        };
        // Two iterations per trip, leaving after either: the only way back to the top is
        // through an odd iteration, whose wait covers the scale loads of the even one (with a
        // path from one even iteration straight to the next, LLVM waits for loads in flight
        // before every scale read of step 0).  nk >= 1.
        for (int b = 0;; b += 2) {
            iteration(std::integral_constant<bool, false>{}, b, sbX, saX, sbY, saY);
            if (b + 1 >= nk) break;
            iteration(std::integral_constant<bool, true>{}, b + 1, sbY, saY, sbX, saX);
            if (b + 2 >= nk) break;
        }
        wait_vmcnt<0>();   // the trailing zero-fill loads have landed
        barrier();         // every fragment read of this tile is done: the rings are free
        agpr_fence(acc);
        store_acc32<OUT, FN, FM>(g.C, g.ldc, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, vec_store != 0);
    }
}

// 8-bit float -> fp32 with the gfx950 conversion instructions (OCP E4M3 / E5M2).
template <int FMT>
__device__ __forceinline__ float mx_decode(uint32_t byte) {
    if constexpr (FMT == MX_E4M3)
        return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(byte), 0);
    else
        return __builtin_amdgcn_cvt_f32_bf8(static_cast<int>(byte), 0);
}

// E8M0 scale -> its power of two as an exponent (e - 127).
__device__ __forceinline__ int mx_scale_exp(uint32_t e) { return static_cast<int>(e) - 127; }

template <int OUT, int FA, int FB>
__global__ __launch_bounds__(256) void mx_simple_kernel(MxArgs g) {
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 64 + 4 * ty, n0 = static_cast<int64_t>(blockIdx.x) * 64 + 4 * tx;
    float acc[4][4] = {};
    for (int64_t k = 0; k < g.K; ++k) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + i, n = n0 + i;
            a[i] = m < g.M ? ldexpf(mx_decode<FA>(g.A[m * g.lda + k]), mx_scale_exp(g.SA[m * g.ldsa + k / 32])) : 0.f;
            b[i] = n < g.N ? ldexpf(mx_decode<FB>(g.B[n * g.ldb + k]), mx_scale_exp(g.SB[n * g.ldsb + k / 32])) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + i;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + j;
            if (n >= g.N) continue;
            if constexpr (OUT == OUT_F32)
                static_cast<float*>(g.C)[m * g.ldc + n] = acc[i][j];
            else
                static_cast<uint16_t*>(g.C)[m * g.ldc + n] = f32_to_bf16(acc[i][j]);
        }
    }
}

template <int OUT, int FA, int FB>
static hipError_t launch_mx_fmt(const MxArgs& g, const Plan& p, hipStream_t s) {
    if (p.kernel == K_MX_RING_256)
        hipLaunchKernelGGL((mx_ring_kernel<OUT, FA, FB>), dim3(p.grid_x), dim3(256), 0, s, g, p.grid, p.vec_store);
    else
        hipLaunchKernelGGL((mx_simple_kernel<OUT, FA, FB>), dim3(p.grid_x, p.grid_y), dim3(256), 0, s, g);
    return hipGetLastError();
}

template <int OUT>
static hipError_t launch_mx_out(const MxArgs& g, const Plan& p, hipStream_t s) {
    if (g.fa == MX_E4M3 && g.fb == MX_E4M3) return launch_mx_fmt<OUT, MX_E4M3, MX_E4M3>(g, p, s);
    if (g.fa == MX_E4M3) return launch_mx_fmt<OUT, MX_E4M3, MX_E5M2>(g, p, s);
    if (g.fb == MX_E4M3) return launch_mx_fmt<OUT, MX_E5M2, MX_E4M3>(g, p, s);
    return launch_mx_fmt<OUT, MX_E5M2, MX_E5M2>(g, p, s);
}

hipError_t launch_mx(const MxArgs& g, int out, const Plan& p, hipStream_t s) {
    return out == OUT_F32 ? launch_mx_out<OUT_F32>(g, p, s) : launch_mx_out<OUT_BF16>(g, p, s);
}

}  // namespace tmm
