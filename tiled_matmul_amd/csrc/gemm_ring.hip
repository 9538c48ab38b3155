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
#include <algorithm>

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
// MF: MFMA shape (16: v_mfma_f32_16x16x32_bf16, one per 32-deep k step and accumulator;
// 32: v_mfma_f32_32x32x16_bf16, two per k step).  AMN / BMN: the A / B operand is MN-major
// (element (i, k) at k * ld + i; MF = 16 only).  An MN-major tile sits in LDS as 64 k-rows
// of 256 elements (512 bytes), 16-byte chunk c of k-row r at chunk c ^ 2 sigma(r) with
// sigma(r) = ((r >> 3) mod 4) ^ 2 (r mod 4) ^ ((r >> 2) mod 2) (bits 0-4 of r only); its
// fragments are read with ds_read_b64_tr_b16, which
// within each group of 16 lanes returns to lane i, element e, element (i mod 4) of the
// 8 bytes addressed by lane 4 e + i / 4 (measured on MI355X).  So lane j of group g
// addresses k-row 8 g + 4 e2 + j / 4, columns 4 (j mod 4) .. + 3 of the fragment, and lane
// i receives the 4 consecutive k of column i: two such reads (e2 = 0, 1) make the MFMA
// operand.  Each transpose read of 64 lanes touches 16 k-rows, 8 per half-wave; sigma gives
// the 8 k-rows of each half-wave 8 different 32-byte positions of a 256-byte bank row, so
// the read is free of bank conflicts (measured: SQ_LDS_BANK_CONFLICT 0).
// OUT: OUT_F32 or OUT_BF16 into C, or OUT_PARTIAL: split K, the fp32 partial sum of each work
// item's K range into the workspace (its own instance, so that the other instances keep one
// range per tile as a compile-time constant and their registers).
constexpr int OUT_PARTIAL = 2;

// Stream-K with atomic work claiming (gemm_bf16_streamk).  Work units: units 0 .. T_dp - 1 are
// whole tiles (data-parallel); units T_dp .. T_dp + G_sk - 1 are stream-K slots: slot s is the
// iterations [s L, min((s + 1) L, I)) of the I = T_sk * nk (tile, K block) iterations of the
// last T_sk tiles, taken tile by tile, with L = ceil(I / G): its segments are the pieces of
// the tiles it touches; only its first and last can be parts of a tile (any between are whole
// tiles).  Workgroup g starts with unit g and claims each further unit with
// an atomic add on ctr[0] (returning gridDim.x + old); the claim is made by one lane after the
// first barrier of a unit and handed to the other waves through ctr[2 + g], read after the
// unit's last barrier (so no wave reads a claim that is not yet made or already replaced).  A
// tile split over several slots is finished by whichever of its segments arrives last, per
// wave (each wave owns a 128 x 128 quarter), on the word ctr[2 + gridDim.x + 4 u + wave]: each
// segment counts its arrival there (low 16 bits); every segment but the last then stores its
// fp32 partial quarter to part[(2 s + (0 for the slot's first segment, 1 for its last)) * 4 +
// wave] in register order (part: SK_PART_OFFSET bytes after ctr) and counts it as written
// (high bits); the last waits for those counts, adds the partials and its own accumulators in
// slot order (a fixed order, so the result does not depend on which workgroup arrives last),
// writes C and resets the word.  ctr[1] counts exiting workgroups; each clears its ctr[2 + g]
// on the way out and the last one resets ctr[0] and ctr[1], so every word of the counter
// region is zero again after the call.  The only wait is the last segment's, for segments that
// have arrived (they are running and have only their stores left), so it always ends.
// Only what cannot be derived is passed (the kernel keeps these live across its K loop): the
// counters (the partials follow them at SK_PART_OFFSET bytes), the whole tiles, the cut tiles
// and the slot length L.
struct SkArgs {
    int* ctr;
    int T_dp, T_sk, L;
};
constexpr int SK_PART_OFFSET = 16384;
// Cache policy of the partials' stores and loads: sc0 | sc1, system coherence (memory, not a
// cache of one XCD).
constexpr int SK_COHERENT = 1 | 16;
// Polls of a cut tile's counter before the last piece gives up waiting (about 2^22 x 128
// cycles, far beyond any real wait: the pieces it waits for have only their stores left).
constexpr int kSkSpinLimit = 1 << 22;

// x / d for x < 2^22 and d >= 1: the float estimate (reciprocal within an ulp or two) is within
// one of the quotient, then corrected.
__device__ __forceinline__ uint32_t sk_div(uint32_t x, uint32_t d) {
    uint32_t q = static_cast<uint32_t>(static_cast<float>(x) * __builtin_amdgcn_rcpf(static_cast<float>(d)));
    if (q * d > x) --q;
    else if ((q + 1) * d <= x) ++q;
    return q;
}

// Keeps the accumulators in AGPRs at this point (a register-allocation constraint only: no
// instruction, no wait states), so that code after a branch does not have them copied out
// before it.
template <int FN, int FM, typename Acc>
__device__ __forceinline__ void agpr_pin(Acc (&acc)[FN][FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) asm volatile("" : "+a"(acc[i][j]));
}

struct SkSeg {
    int t, kb0, nk;     // tile, first K block, K blocks
    int u, s, part;     // stream-K tile (t - T_dp), slot, partial of the slot (0: its first segment, 1: its last)
    int s_lo, s_hi;     // the slots that hold this tile's segments
    bool direct;        // the whole tile: write C
    bool has_next;      // the slot continues into the next tile
};

__device__ __forceinline__ SkSeg sk_segment(const SkArgs& a, int unit, int seg, uint32_t nk) {
    SkSeg r{};
    if (unit < a.T_dp) {
        r.t = unit, r.kb0 = 0, r.nk = static_cast<int>(nk), r.direct = true, r.has_next = false;
        return r;
    }
    const uint32_t L = static_cast<uint32_t>(a.L);
    const uint32_t I = static_cast<uint32_t>(a.T_sk) * nk;
    // slots in XCD order (the workgroups one XCD starts with take neighbouring slots)
    const int G_sk = static_cast<int>((I + L - 1) / L);
    const uint32_t s = static_cast<uint32_t>(xcd_order(unit - a.T_dp, G_sk));
    const uint32_t lo = s * L, hi = min(lo + L, I);
    const uint32_t u = sk_div(lo, nk) + static_cast<uint32_t>(seg);
    const uint32_t tb = u * nk;
    const uint32_t a0 = max(lo, tb), a1 = min(hi, tb + nk);
    r.t = a.T_dp + static_cast<int>(u), r.u = static_cast<int>(u), r.s = static_cast<int>(s), r.part = seg > 0;
    r.kb0 = static_cast<int>(a0 - tb), r.nk = static_cast<int>(a1 - a0);
    r.has_next = hi > tb + nk;
    r.s_lo = static_cast<int>(sk_div(tb, L));
    r.s_hi = static_cast<int>(sk_div(tb + nk - 1, L));
    // The divisions run on the vector unit; the results are the same in every lane, and saying
    // so keeps the branches on them uniform (and the loop's bookkeeping in scalar registers).
    r.t = __builtin_amdgcn_readfirstlane(r.t), r.u = __builtin_amdgcn_readfirstlane(r.u);
    r.kb0 = __builtin_amdgcn_readfirstlane(r.kb0), r.nk = __builtin_amdgcn_readfirstlane(r.nk);
    r.s_lo = __builtin_amdgcn_readfirstlane(r.s_lo), r.s_hi = __builtin_amdgcn_readfirstlane(r.s_hi);
    r.has_next = __builtin_amdgcn_readfirstlane(r.has_next ? 1 : 0) != 0;
    r.direct = r.s_lo == r.s_hi;
    return r;
}

template <int OUT, bool RAGGED, int WAVES_M, int WAVES_N, bool ASM, int MF, bool AMN, bool BMN, bool SK = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, WAVES_M * WAVES_N / 4) void gemm_ring_kernel(
    GemmArgs g, TileGrid tg, int vec_store, SkArgs sk) {
    using namespace rg;
    using MM = std::conditional_t<MF == 16, std::conditional_t<ASM, MmaAsm16, Mma<16>>,
                                  std::conditional_t<ASM, MmaAsm32, Mma<32>>>;
    using Acc = typename MM::Acc;
    static_assert(MF == 16 || !(AMN || BMN), "MN-major operands take the 16x16x32 shape");
    constexpr int KH = 32 / MM::KS;             // MFMAs per accumulator per 32-deep k step
    constexpr int CPM = MM::KS / 8;             // 16-byte k chunks per MFMA operand row
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, FM = WM / MF, FN = WN / MF;
    // MFMAs at the end of each k step that follow the step's last fragment read.
    constexpr int RTAIL = NW == 4 ? TMM_RING4_TAIL : TMM_RING8_TAIL;
    constexpr int L = 256 / (NW * R);   // load instructions per wave for one A (or B) tile
    static_assert(L * NW * R == 256, "rows split over the waves");
    static_assert(64 / (NW * 2) == L, "an MN-major tile takes as many loads as a K-major one");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[(NA + NB) * TILE];

    const int lane = lane_id(), w = wave_id();
    const int wm = w / WAVES_N, wn = w % WAVES_N;
    const uint32_t K = static_cast<uint32_t>(g.K);
    const uint32_t K8 = RAGGED ? K & ~7u : K;
    const int nk_all = static_cast<int>((g.K + BK - 1) / BK);
    const int S = OUT == OUT_PARTIAL ? g.splits : 1;   // K ranges per tile

    // K-major tiles.  Load i of wave w: tile rows (NW i + w) R + lane / 8; the lane writes
    // physical chunk lane % 8, i.e. fetches logical chunk (lane % 8) ^ swz(row).  R = 8, so
    // swz(row) = lane / 8 for every i.  Fragment reads of sub-step h of k step kk: row
    // lane % MF of an MF-row block, logical chunk 4 kk + CPM h + lane / MF.
    auto lane_consts = [&](int ln, int& lrow_, uint32_t& chunk_k_, int (&rd_)[2][KH]) {
        lrow_ = ln / 8;
        chunk_k_ = 8u * static_cast<uint32_t>((ln % 8) ^ swz(lrow_));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int h = 0; h < KH; ++h)
                rd_[kk][h] = (ln % MF) * ROWB + (((4 * kk + CPM * h + ln / MF) ^ swz(ln % MF)) * 16);
    };
    int lrow0, rd0[2][KH];
    uint32_t chunk_k0;
    lane_consts(lane, lrow0, chunk_k0, rd0);
    const int a_off = wm * WM * ROWB, b_off = wn * WN * ROWB;

    // MN-major tiles.  Load i of wave w: k-rows (NW i + w) 2 + lane / 32, physical chunk
    // lane % 32, logical chunk (lane % 32) ^ 2 sigma(k-row).
    auto sigma = [](int r) { return ((r >> 3) & 3) ^ ((r & 3) << 1) ^ ((r >> 2) & 1); };
    int mn_col[L];   // element column (within the tile) this lane fetches in load i
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int r = (NW * i + w) * 2 + (lane >> 5);
        mn_col[i] = 8 * ((lane & 31) ^ (2 * sigma(r)));
    }
    // Transpose reads: lane j of group gq addresses k-row 8 gq + 4 e2 + j / 4 (+ 32 kk) and
    // columns col0 + 16 i + 4 (j mod 4); with col0 a multiple of 128 the physical chunk is
    // col0 / 8 + 2 (i ^ sigma) + (j / 2) mod 2.
    const int gq = lane >> 4, jl = lane & 15;
    int tr_base[2], tr_sig[2];
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
        const int r = 8 * gq + 4 * e2 + (jl >> 2);
        tr_sig[e2] = sigma(r);
        tr_base[e2] = r * 512 + ((jl >> 1) & 1) * 16 + (jl & 1) * 8;
    }
    const int a_col0 = wm * WM, b_col0 = wn * WN;   // first fragment column of this wave

    static_assert(!SK || (OUT != OUT_PARTIAL && WAVES_M == 2 && WAVES_N == 2 && MF == 16), "stream-K layout");
    int unit = blockIdx.x, seg = 0;   // stream-K: the current unit and segment
    // stream-K units: the whole tiles and ceil(I / L) slots
    const int sk_units = SK ? sk.T_dp + static_cast<int>((static_cast<uint32_t>(sk.T_sk) * nk_all + sk.L - 1) /
                                                         static_cast<uint32_t>(sk.L))
                            : 0;
    for (int item = blockIdx.x; SK ? unit < sk_units : item < tg.total * S; item += gridDim.x) {
        // Work item = (tile, K range); range s covers blocks [s nk / S, (s + 1) nk / S).
        int t = item / S, s_rng = item - (item / S) * S;
        int kb0 = static_cast<int>(static_cast<int64_t>(s_rng) * nk_all / S);
        int nk = static_cast<int>(static_cast<int64_t>(s_rng + 1) * nk_all / S) - kb0;
        if constexpr (SK) {
            const SkSeg sg = sk_segment(sk, unit, seg, static_cast<uint32_t>(nk_all));
            t = sg.t, kb0 = sg.kb0, nk = sg.nk, s_rng = 0;
        }
        // The per-lane constants.  Stream-K recomputes them per work item from an opaque copy of
        // the lane id, so that the compiler does not keep them live across the work loop, where
        // the longer epilogue needs the registers.
        int lrow = lrow0, rd[2][KH];
        uint32_t chunk_k = chunk_k0;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int h = 0; h < KH; ++h) rd[kk][h] = rd0[kk][h];
        if constexpr (SK) {
            int lane_k = lane;
            asm volatile("" : "+v"(lane_k));
            lane_consts(lane_k, lrow, chunk_k, rd);
        }

        int bt, tm, tn;
        if constexpr (SK) {
            // whole tiles: the XCD order over the first T_dp tiles of the raster; cut tiles: the
            // rest of the raster, in order
            if (t < sk.T_dp) raster_of(xcd_order(t, sk.T_dp), tg, bt, tm, tn);
            else raster_of(t, tg, bt, tm, tn);
        } else {
            tile_of(t, tg, bt, tm, tn);
        }
        const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
        const int64_t rows_a = min<int64_t>(BM, g.M - m0), rows_b = min<int64_t>(BN, g.N - n0);
        const uint16_t* Ab = g.A + bt * g.sA + (AMN ? m0 : m0 * g.lda);
        const uint16_t* Bb = g.B + bt * g.sB + (BMN ? n0 : n0 * g.ldb);
        const auto ra = make_rsrc(Ab, static_cast<uint32_t>(AMN ? ((g.K - 1) * g.lda + rows_a) * 2
                                                                : ((rows_a - 1) * g.lda + g.K) * 2));
        const auto rb = make_rsrc(Bb, static_cast<uint32_t>(BMN ? ((g.K - 1) * g.ldb + rows_b) * 2
                                                                : ((rows_b - 1) * g.ldb + g.K) * 2));
        // Per-lane offsets of each load (out-of-range rows or columns: OOB).
        uint32_t va[L], vb[L];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if constexpr (AMN) {
                const int r = (NW * i + w) * 2 + (lane >> 5);
                va[i] = mn_col[i] < rows_a ? static_cast<uint32_t>(r * g.lda + mn_col[i]) * 2u : OOB;
            } else {
                const int r = (NW * i + w) * R + lrow;
                va[i] = r < rows_a ? static_cast<uint32_t>(r * g.lda) * 2u + 2u * chunk_k : OOB;
            }
            if constexpr (BMN) {
                const int r = (NW * i + w) * 2 + (lane >> 5);
                vb[i] = mn_col[i] < rows_b ? static_cast<uint32_t>(r * g.ldb + mn_col[i]) * 2u : OOB;
            } else {
                const int r = (NW * i + w) * R + lrow;
                vb[i] = r < rows_b ? static_cast<uint32_t>(r * g.ldb) * 2u + 2u * chunk_k : OOB;
            }
        }

        // Load instruction q of the A (is_a) or B tile of block j into the tile at LDS byte
        // offset `dst` (k >= K8 reads zeros; blocks past the end read zeros).
        // Blocks j >= nk of this range are loaded too (the last iterations run ahead); they
        // are never read, whatever they hold.
        auto load_one = [&](bool is_a, int q, int j, int dst) {
            const uint32_t k0 = static_cast<uint32_t>(kb0 + j) * BK;
            const bool mn = is_a ? AMN : BMN;
            if (mn) {
                const int64_t ld = is_a ? g.lda : g.ldb;
                const uint32_t kr = static_cast<uint32_t>((NW * q + w) * 2 + (lane >> 5));
                const bool ok = k0 + kr < K8;
                // Blocks past the end get no row offset, so OOB + soffset cannot wrap into range.
                const uint32_t soff = k0 < K ? static_cast<uint32_t>(k0 * ld) * 2u : 0u;
                load_lds_16(is_a ? ra : rb, lds + dst + (NW * q + w) * 2 * 512, ok ? (is_a ? va[q] : vb[q]) : OOB,
                            soff);
            } else {
                const bool ok = k0 + chunk_k < K8;
                load_lds_16(is_a ? ra : rb, lds + dst + (NW * q + w) * R * ROWB, ok ? (is_a ? va[q] : vb[q]) : OOB,
                            2u * k0);
            }
        };
        // MN-major fragment i (16 columns from col0 + 16 i) of k step kk of the tile at `tile`.
        // The transpose reads are inline assembly: issued through the builtin, LLVM waits for
        // every outstanding direct-to-LDS load before each of them (it cannot tell that they
        // read other slots).  Their completion is covered by the explicit lgkmcnt(0) that
        // ends every k step (fenced by sched_barrier) before the fragments are used.
        auto read_tr = [&](int tile, int col0, int i, int kk) {
            u32x2 h[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const int off = tile + kk * 32 * 512 + tr_base[e2] + (col0 / 8) * 16 + 32 * (i ^ tr_sig[e2]);
                const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(lds + off)));
                asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(h[e2]) : "v"(addr) : "memory");
            }
            const u32x4 v = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3);
            return __builtin_bit_cast(bf16x8, v);
        };
        // Fragment q of k step kk from the A tile at `at` and the B tile at `bt_`: q < KH FN:
        // B fragment q % FN of sub-step q / FN, else A fragment (q - KH FN) % FM of sub-step
        // (q - KH FN) / FM.
        using F = Frags<KH * FN, KH * FM>;
        auto read_one = [&](F& f, int q, int at, int bt_, int kk) {
            if (q < KH * FN) {
                const int h = q / FN, i = q % FN;
                if constexpr (BMN)
                    f.b[q] = read_tr(bt_, b_col0, i, kk);
                else
                    f.b[q] = *reinterpret_cast<const bf16x8*>(lds + bt_ + b_off + MF * i * ROWB + rd[kk][h]);
            } else {
                const int r = q - KH * FN, h = r / FM, j = r % FM;
                if constexpr (AMN)
                    f.a[r] = read_tr(at, a_col0, j, kk);
                else
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
        if constexpr (SK) {
            // Claim the unit after this one.  Past this barrier every wave has read the previous
            // claim (at the end of the previous unit), so its slot can be overwritten.
            if (seg == 0 && w == 0 && lane == 0) {
                const int next = static_cast<int>(gridDim.x) +
                                 __hip_atomic_fetch_add(sk.ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sk.ctr + 2 + blockIdx.x, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
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

        // the last range (stream-K: the segment that ends the tile) holds the end of K
        if (RAGGED && (SK ? kb0 + nk == nk_all : s_rng == S - 1)) {
            // Elements K8 .. K - 1 of every row, element by element (nothing at or beyond K is
            // read), as the first 8 k of one more 32-deep step (A in A slot 0, B in B slot 0),
            // each tile in its own layout; the rest of the step is zero.
            auto stage = [&](bool is_a, bool mn, const uint16_t* Xb, int64_t ld, int64_t rows, int dst) {
                if (mn) {
                    // k-rows 0 .. 31 of the MN-major tile; row e < 8 holds k = K8 + e.
                    for (int c = threadIdx.x; c < 32 * 32; c += 64 * NW) {
                        const int r = c >> 5, lc = c & 31, col = 8 * lc;
                        uint32_t hv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                        if (r < 8 && K8 + r < K) {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                if (col + e < rows) hv[e] = Xb[(K8 + r) * ld + col + e];
                        }
                        const u32x4 v = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                         hv[6] | (hv[7] << 16)};
                        *reinterpret_cast<u32x4*>(lds + dst + r * 512 + ((lc ^ (2 * sigma(r))) * 16)) = v;
                    }
                } else {
                    for (int rr = threadIdx.x; rr < 256; rr += 64 * NW) {
                        uint32_t hv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                        if (rr < rows) {
                            const uint16_t* row = Xb + rr * ld;
#pragma unroll
                            for (int e = 0; e < 7; ++e)
                                if (K8 + e < K) hv[e] = row[K8 + e];
                        }
                        uint8_t* d = lds + dst + rr * ROWB;
                        const u32x4 z = {0u, 0u, 0u, 0u};
                        const u32x4 v = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                         hv[6] | (hv[7] << 16)};
#pragma unroll
                        for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(d + ((c ^ swz(rr)) * 16)) = c == 0 ? v : z;
                    }
                }
                (void)is_a;
            };
            stage(true, AMN, Ab, g.lda, rows_a, 0);
            stage(false, BMN, Bb, g.ldb, rows_b, B_BASE);
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

        if constexpr (SK) {
            const SkSeg sg = sk_segment(sk, unit, seg, static_cast<uint32_t>(nk_all));   // again: fewer live registers
            void* const part = reinterpret_cast<char*>(sk.ctr) + SK_PART_OFFSET;
            if (sg.direct) {
                // The accumulators stay in AGPRs up to the stores: without this pin the
                // compiler copies them out before the branch for both paths, and spills.
                agpr_pin(acc);
                void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                          : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
                store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, vec_store != 0);
            } else {
                // A cut tile, per wave (each wave owns a 128 x 128 quarter).  The tile's counter
                // word counts arrivals in its low 16 bits and written partials in its high bits.
                // Every piece counts its arrival first.  A piece that is not the last to arrive
                // writes its partial quarter, in register order, through to memory
                // (system-coherent stores bypass the caches, so no cache maintenance is needed
                // for another XCD to read them; a release fence would write back this XCD's
                // whole L2), and then counts it as written.  The last piece to arrive writes no
                // partial: it waits until the others' partials are counted (each of those
                // pieces has arrived, so it is running and only has stores left: the wait ends),
                // adds them and its own accumulators in slot order (a fixed order, so the result
                // does not depend on which piece arrives last), writes C and clears the word.
                const uint32_t n_slots = (static_cast<uint32_t>(sk.T_sk) * nk_all + sk.L - 1) / sk.L;
                const auto rp = make_rsrc(part, n_slots * (2u * 4u * 65536u));   // slots x 2 segments x 4 quarters x 64 KB
                const int others = sg.s_hi - sg.s_lo;   // pieces besides this one
                int* cnt = sk.ctr + 2 + gridDim.x + 4 * sg.u + w;
                int old = 0;
                if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                old = __builtin_amdgcn_readfirstlane(old);
                if ((old & 0xffff) != others) {
                    const uint32_t quarter = (2u * sg.s + sg.part) * 4u + w;   // 64 KB each
#pragma unroll
                    for (int f = 0; f < FN * FM; ++f) {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[f / FM][f % FM]), rp,
                                                               (quarter * (FN * FM) + f) * 1024u + 16u * lane, 0,
                                                               SK_COHERENT);
                        if (f % 8 == 7) __builtin_amdgcn_sched_barrier(0);
                    }
                    wait_vmcnt<0>();   // the partial is in memory before it is counted
                    if (lane == 0) __hip_atomic_fetch_add(cnt, 1 << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    // Wait for the others' partials (polled with an atomic, which sees the
                    // other XCDs' counts; bounded: past the limit the quarter is written as NaN).
                    int v = 0;
                    if (lane == 0) {
                        v = __hip_atomic_fetch_add(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        for (int it = 0; (v >> 16) != others && it < kSkSpinLimit; ++it) {
                            __builtin_amdgcn_s_sleep(2);
                            v = __hip_atomic_fetch_add(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                    const bool ready = (__builtin_amdgcn_readfirstlane(v) >> 16) == others;
                    const uint32_t tb = static_cast<uint32_t>(sg.u) * static_cast<uint32_t>(nk_all);
                    void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                              : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
                    const bool full = vec_store != 0 && m0 + wm * WM + WM <= g.M && n0 + wn * WN + WN <= g.N;
                    // 8 fragments at a time: each slot's 8 loads in flight together
                    constexpr int FG = 8;
#pragma unroll
                    for (int f0 = 0; f0 < FN * FM; f0 += FG) {
                        f32x4 v8[FG];
#pragma unroll 1
                        for (int s2 = sg.s_lo; s2 <= sg.s_hi; ++s2) {
                            f32x4 x[FG];
                            if (s2 == sg.s) {   // this piece: its accumulators
#pragma unroll
                                for (int i = 0; i < FG; ++i) x[i] = acc[(f0 + i) / FM][(f0 + i) % FM];
                            } else {
                                // the slot's first segment if it starts in this tile, else its last
                                const uint32_t p2 =
                                    static_cast<uint32_t>(s2) * static_cast<uint32_t>(sk.L) >= tb ? 0u : 1u;
                                const uint32_t q2 = (2u * s2 + p2) * 4u + w;
#pragma unroll
                                for (int i = 0; i < FG; ++i)
                                    x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                         rp, (q2 * (FN * FM) + f0 + i) * 1024u + 16u * lane,
                                                                         0, SK_COHERENT));
                            }
#pragma unroll
                            for (int i = 0; i < FG; ++i) v8[i] = s2 == sg.s_lo ? x[i] : v8[i] + x[i];
                        }
#pragma unroll
                        for (int i = 0; i < FG; ++i) {
                            if (!ready) v8[i] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                      __builtin_nanf("")};
                            const int fi = (f0 + i) / FM, fj = (f0 + i) % FM;
                            store_frag<OUT>(Cb, g.ldc, g.M, g.N, m0 + wm * WM + 16 * fj + (lane & 15),
                                            n0 + wn * WN + 16 * fi + 4 * (lane >> 4), v8[i], full);
                        }
                    }
                    if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            // Next: the slot's second segment, or the unit claimed at the start of this one
            // (written before its barriers).  Selects rather than branches keep unit and seg in
            // scalar registers.
            const int claimed = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(sk.ctr + 2 + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            unit = sg.has_next ? unit : claimed;
            seg = sg.has_next ? seg + 1 : 0;
        } else if constexpr (OUT == OUT_PARTIAL) {   // range s_rng's partial (pitch N; 16-byte stores when N % 4 == 0)
            float* P = g.ws + (static_cast<int64_t>(s_rng) * g.batch + bt) * g.M * g.N;
            if constexpr (MF == 16)
                store_acc<OUT_F32, FN, FM>(P, g.N, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, g.N % 4 == 0);
            else
                store_acc32<OUT_F32, FN, FM>(P, g.N, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, g.N % 4 == 0);
        } else {
            void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                      : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
            if constexpr (MF == 16)
                store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, vec_store != 0);
            else
                store_acc32<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + wm * WM, n0 + wn * WN, acc, vec_store != 0);
        }
    }
    if constexpr (SK) {
        // Every wave has read this workgroup's last claim (at the end of its last unit): clear
        // it, then count the workgroup out; the last one to leave resets the claim and exit
        // counters.  So every word of the counter region is zero again when the call ends,
        // whatever the layout of the next call on the same workspace.
        barrier();
        if (w == 0 && lane == 0) {
            __hip_atomic_store(sk.ctr + 2 + blockIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int e = __hip_atomic_fetch_add(sk.ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (e == static_cast<int>(gridDim.x) - 1) {
                __hip_atomic_store(sk.ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sk.ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// Split-K reduction: C[b][m][n] = sum over s = 0 .. S-1, in that order, of ws[s][b][m][n]
// (fp32 sums; deterministic), converted to the output type.  V = 4: four consecutive
// elements of one row per thread (N % 4 == 0), 16-byte workspace loads, the S loads of a
// thread issued before they are summed; VC: C takes 16-byte (fp32) or 8-byte (bf16) stores.
template <int OUT, int V, bool VC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
    const int64_t mn = g.M * g.N, total = g.batch * mn, nv = total / V;
    for (int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; v < nv;
         v += static_cast<int64_t>(gridDim.x) * 256) {
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
        constexpr int U = 8;   // loads in flight per thread
        for (int s0 = 0; s0 < g.splits; s0 += U) {
            float x[U][V];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s0 + u < g.splits) {
                    const float* src = g.ws + (s0 + u) * total + v * V;
                    if constexpr (V == 4) {
                        const f32x4 t = *reinterpret_cast<const f32x4*>(src);
                        x[u][0] = t[0], x[u][1] = t[1], x[u][2] = t[2], x[u][3] = t[3];
                    } else {
                        x[u][0] = *src;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (s0 + u < g.splits)
#pragma unroll
                    for (int i = 0; i < V; ++i) acc[i] += x[u][i];
        }
        const int64_t e = v * V, b = e / mn, r = e - b * mn, m = r / g.N, n = r - m * g.N;
        const int64_t off = b * g.sC + m * g.ldc + n;
        if constexpr (OUT == OUT_F32) {
            float* c = static_cast<float*>(g.C) + off;
            if constexpr (VC) {
                *reinterpret_cast<f32x4*>(c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) c[i] = acc[i];
            }
        } else {
            uint16_t* c = static_cast<uint16_t*>(g.C) + off;
            if constexpr (VC) {
                const uint32_t lo = f32_to_bf16(acc[0]) | (uint32_t(f32_to_bf16(acc[1])) << 16);
                const uint32_t hi = f32_to_bf16(acc[2]) | (uint32_t(f32_to_bf16(acc[3])) << 16);
                *reinterpret_cast<u32x2*>(c) = u32x2{lo, hi};
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) c[i] = f32_to_bf16(acc[i]);
            }
        }
    }
}

template <int OUT>
static void launch_reduce_out(const GemmArgs& g, bool v4, bool vc, int blocks, hipStream_t s) {
    if (v4 && vc)
        hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 4, true>), dim3(blocks), dim3(256), 0, s, g);
    else if (v4)
        hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 4, false>), dim3(blocks), dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 1, false>), dim3(blocks), dim3(256), 0, s, g);
}

hipError_t launch_splitk_reduce(const GemmArgs& g, int out, hipStream_t s) {
    const int64_t total = g.batch * g.M * g.N;
    const bool v4 = g.N % 4 == 0;   // the workspace is 16-byte aligned with pitch N
    const uintptr_t ca = out == OUT_F32 ? 16 : 8;
    const bool vc = v4 && reinterpret_cast<uintptr_t>(g.C) % ca == 0 && g.ldc % 4 == 0 &&
                    (g.batch == 1 || g.sC % 4 == 0);
    const int64_t threads = v4 ? total / 4 : total;
    const int blocks = static_cast<int>(std::min<int64_t>((threads + 255) / 256, 65536));
    if (out == OUT_F32)
        launch_reduce_out<OUT_F32>(g, v4, vc, blocks, s);
    else
        launch_reduce_out<OUT_BF16>(g, v4, vc, blocks, s);
    return hipGetLastError();
}

template <int WM, int WN, bool ASM, int MF, bool AMN, bool BMN>
static hipError_t launch_ring_lay(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    const bool ragged = (g.K & 7) != 0;
    const dim3 grid(p.grid_x), block(64 * WM * WN);
    if (g.splits > 1 && ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_PARTIAL, true, WM, WN, ASM, MF, AMN, BMN>), grid, block, 0, s, g,
                           p.grid, p.vec_store, SkArgs{});
    else if (g.splits > 1)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_PARTIAL, false, WM, WN, ASM, MF, AMN, BMN>), grid, block, 0, s, g,
                           p.grid, p.vec_store, SkArgs{});
    else if (out == OUT_F32 && ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_F32, true, WM, WN, ASM, MF, AMN, BMN>), grid, block, 0, s, g, p.grid,
                           p.vec_store, SkArgs{});
    else if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_F32, false, WM, WN, ASM, MF, AMN, BMN>), grid, block, 0, s, g, p.grid,
                           p.vec_store, SkArgs{});
    else if (ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_BF16, true, WM, WN, ASM, MF, AMN, BMN>), grid, block, 0, s, g, p.grid,
                           p.vec_store, SkArgs{});
    else
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_BF16, false, WM, WN, ASM, MF, AMN, BMN>), grid, block, 0, s, g, p.grid,
                           p.vec_store, SkArgs{});
    return hipGetLastError();
}

// K-major operands: any ring configuration; MN-major ones: the 4-wave, 16x16x32 kernel.
template <int WM, int WN, bool ASM, int MF>
static hipError_t launch_ring_cfg(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    if (g.la == LAYOUT_K && g.lb == LAYOUT_K) return launch_ring_lay<WM, WN, ASM, MF, false, false>(g, out, p, s);
    if constexpr (WM == 2 && WN == 2) {
        if (g.la == LAYOUT_K) return launch_ring_lay<2, 2, true, 16, false, true>(g, out, p, s);
        if (g.lb == LAYOUT_K) return launch_ring_lay<2, 2, true, 16, true, false>(g, out, p, s);
        return launch_ring_lay<2, 2, true, 16, true, true>(g, out, p, s);
    }
    return hipErrorInvalidValue;
}

// MFMA shape of the ring kernels (16 or 32; v_mfma_f32_32x32x16_bf16 measured 5-7% slower on
// MI355X for both layouts).
#ifndef TMM_RING4_MFMA
#define TMM_RING4_MFMA 16
#endif
#ifndef TMM_RING8_MFMA
#define TMM_RING8_MFMA 16
#endif

// Stream-K with atomic work claiming: the 4-wave kernel, K-major operands.
hipError_t launch_ring_streamk(const GemmArgs& g, int out, const Plan& p, int* ctr, float* part, int T_dp,
                               int T_sk, int G_sk, int L, hipStream_t s) {
    const bool ragged = (g.K & 7) != 0;
    (void)G_sk;   // = ceil(T_sk nk / L), derived in the kernel
    if (reinterpret_cast<char*>(part) != reinterpret_cast<char*>(ctr) + SK_PART_OFFSET) return hipErrorInvalidValue;
    const SkArgs sk{ctr, T_dp, T_sk, L > 0 ? L : 1};
    const dim3 grid(p.grid_x), block(256);
    if (out == OUT_F32 && ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_F32, true, 2, 2, true, 16, false, false, true>), grid, block, 0, s, g,
                           p.grid, p.vec_store, sk);
    else if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_F32, false, 2, 2, true, 16, false, false, true>), grid, block, 0, s, g,
                           p.grid, p.vec_store, sk);
    else if (ragged)
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_BF16, true, 2, 2, true, 16, false, false, true>), grid, block, 0, s, g,
                           p.grid, p.vec_store, sk);
    else
        hipLaunchKernelGGL((gemm_ring_kernel<OUT_BF16, false, 2, 2, true, 16, false, false, true>), grid, block, 0, s,
                           g, p.grid, p.vec_store, sk);
    return hipGetLastError();
}

hipError_t launch_ring(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    switch (p.kernel) {
        case K_RING8_256: return launch_ring_cfg<2, 4, false, TMM_RING8_MFMA>(g, out, p, s);
        case K_RING4_256: return launch_ring_cfg<2, 2, true, TMM_RING4_MFMA>(g, out, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tmm
