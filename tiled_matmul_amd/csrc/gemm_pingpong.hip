// Ping-pong GEMM, C = A * B^T (bf16 in, fp32 accumulate): the last rungs of the ladder.
//
// The page "读书笔记-《面向机器学习系统的现代 GPU 编程》", section "9 步优化", ends with
// role specialisation (step 7: producers load, consumers multiply, handing data over through
// barriers) and two consumers sharing one B tile, each computing half the output rows
// (step 9).  On gfx950 the roles alternate in time instead of being fixed to warps:
//
//   * a 256 x 256 tile, 8 waves (2 per SIMD), two groups of 4: group g computes rows
//     128 g .. 128 g + 127 against the whole shared B stage; wave (g, wn) owns a 128 x 64
//     block as v_mfma_f32_16x16x32_bf16 accumulators (128 VGPRs);
//   * every K block of 32 passes through a memory phase (read the 12 fragments of the block
//     from LDS, issue this wave's 4 direct-to-LDS loads of a block three ahead, wait for its
//     own loads of the next block) and a compute phase (32 MFMAs), each closed by a
//     workgroup barrier;
//   * group 1 runs one phase behind group 0 (one extra barrier at the start; group 0 takes
//     one at the end), so while the wave of one group on a SIMD multiplies, the wave of the
//     other group on the same SIMD loads: the matrix pipe never waits behind a wave's own
//     LDS or load instructions;
//   * a 4-slot ring of K blocks (4 x 32 KB of LDS) gives each block's loads three phases
//     pairs of lead before its first read.
//
// Phase t (between two barriers): group 0 runs the memory phase of block t/2 when t is even
// and the compute phase of block (t-1)/2 when t is odd; group 1 is one phase later.  Block j
// is read at t = 2j (group 0) and 2j+1 (group 1), so its slot is free from t = 2j+2; the
// memory phase of block j+1 (t = 2j+2, 2j+3) refills it with block j+4.  Before the barrier
// that closes its memory phase of block j, a wave waits until at most 8 of its loads are
// outstanding, i.e. its share of block j+1 has landed: block j+1 is complete in LDS before
// either group reads it.  Both groups execute 2 nk + 2 barriers per tile.
//
// Preconditions as the other direct-to-LDS kernels (planner): K % 8 == 0, lda, ldb and batch
// strides multiples of 8, A and B 16-byte aligned, 256 * ld * 2 < 2^31.
#include "launch.hpp"

namespace tmm {

namespace pp {
constexpr int BM = 256, BN = 256, BK = 32, SLOTS = 4, NW = 8;
constexpr int KC = BK / 8;                 // 16-byte chunks per LDS row (64-byte rows)
constexpr int R = 64 / KC;                 // LDS rows per wave load instruction (16)
constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, SLOT_BYTES = A_BYTES + B_BYTES;
constexpr int IA = BM / (NW * R), IB = BN / (NW * R);   // 2 + 2 loads per wave per block
constexpr int LOADS = IA + IB;
constexpr int WM = 128, WN = 64, FM = WM / 16, FN = WN / 16;   // 8 A and 4 B fragments
static_assert(IA * NW * R == BM && IB * NW * R == BN, "rows split over the waves");
static_assert(SLOTS * SLOT_BYTES <= 160 * 1024, "LDS capacity");

// 64-byte rows: rows 2m and 2m+1 share one 128-byte bank line, so the XOR pattern pairs
// them: row r holds logical chunk c in physical slot c ^ ((r >> 1) & 3).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & (KC - 1); }
}  // namespace pp

// Workgroup barrier that also fences the instruction scheduler, so that no MFMA moves into
// a memory phase or memory instruction into a compute phase.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void pp_wait() {   // vmcnt(N), lgkmcnt(0)
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    constexpr int enc = (N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14);
    __builtin_amdgcn_s_waitcnt(enc);
}

template <int OUT, bool XCD_ORDER>
__global__ __launch_bounds__(512, 2) void gemm_pingpong_kernel(GemmArgs g, TileGrid tg, int vec_store) {
    using namespace pp;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[SLOTS * SLOT_BYTES];

    const int lane = lane_id(), w = wave_id();
    const int grp = w >> 2, wn = w & 3;
    const int nk = static_cast<int>((g.K + BK - 1) / BK);
    const uint32_t K = static_cast<uint32_t>(g.K);

    // Load i of wave w: rows (NW i + w) R .. +R of the A tile (i < IA) or the B tile; the lane
    // writes physical chunk (lane % KC) of row (lane / KC), i.e. fetches logical chunk
    // (lane % KC) ^ swz(row).  With R = 16 the row's swizzle depends on lane / KC only.
    const int lrow = lane / KC;
    const uint32_t chunk_k = 8u * static_cast<uint32_t>((lane % KC) ^ swz(lrow));
    // Fragment reads: row (lane % 16) of a 16-row block, logical chunk lane / 16.
    const int rd = (lane & 15) * BK * 2 + ((((lane >> 4)) ^ swz(lane & 15)) * 16);
    const int a_frag0 = grp * WM * BK * 2 + rd, b_frag0 = A_BYTES + wn * WN * BK * 2 + rd;

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
        const auto ra = make_rsrc(g.A + bt * g.sA + m0 * g.lda, static_cast<uint32_t>(((rows_a - 1) * g.lda + g.K) * 2));
        const auto rb = make_rsrc(g.B + bt * g.sB + n0 * g.ldb, static_cast<uint32_t>(((rows_b - 1) * g.ldb + g.K) * 2));
        uint32_t voff[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const bool is_a = i < IA;
            const int r = (NW * (is_a ? i : i - IA) + w) * R + lrow;
            const int64_t rows = is_a ? rows_a : rows_b;
            const int64_t ld = is_a ? g.lda : g.ldb;
            voff[i] = r < rows ? static_cast<uint32_t>(r * ld) * 2u + 2u * chunk_k : OOB;
        }
        // This wave's loads of K block kb (blocks past the end read zeros).
        auto issue = [&](int kb) {
            uint8_t* s = lds + (kb % SLOTS) * SLOT_BYTES;
            const uint32_t k0 = static_cast<uint32_t>(kb) * BK;
            const bool ok = k0 + chunk_k < K;
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const bool is_a = i < IA;
                uint8_t* dst = s + (is_a ? 0 : A_BYTES) + (NW * (is_a ? i : i - IA) + w) * R * BK * 2;
                load_lds_16(is_a ? ra : rb, dst, ok ? voff[i] : OOB, 2u * k0);
            }
        };

        f32x4 acc[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Prologue: all four slots; block 0 complete (this wave) + barrier = block 0 in LDS.
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) issue(s);
        pp_wait<(SLOTS - 1) * LOADS>();
        phase_barrier();
        if (grp == 1) phase_barrier();   // group 1 runs one phase behind

        for (int kb = 0; kb < nk; ++kb) {
            // Memory phase of block kb.
            bf16x8 fb[FN], fa[FM];
            const uint8_t* s = lds + (kb % SLOTS) * SLOT_BYTES;
#pragma unroll
            for (int i = 0; i < FN; ++i) fb[i] = *reinterpret_cast<const bf16x8*>(s + b_frag0 + 16 * i * BK * 2);
#pragma unroll
            for (int j = 0; j < FM; ++j) fa[j] = *reinterpret_cast<const bf16x8*>(s + a_frag0 + 16 * j * BK * 2);
            if (kb >= 1) issue(kb + SLOTS - 1);   // into the slot of block kb-1
            // This wave's share of block kb+1 has landed once at most two later blocks'
            // loads (kb+2, kb+3) are outstanding; and this wave's reads are done.
            pp_wait<(SLOTS - 2) * LOADS>();
            phase_barrier();
            // Compute phase of block kb.
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = mfma_16x16x32(fb[i], fa[j], acc[i][j]);
            phase_barrier();
        }
        if (grp == 0) phase_barrier();   // matches group 1's extra barrier
        pp_wait<0>();              // trailing zero-fill loads landed before the ring is reused

        void* Cb = OUT == OUT_F32 ? static_cast<void*>(static_cast<float*>(g.C) + bt * g.sC)
                                  : static_cast<void*>(static_cast<uint16_t*>(g.C) + bt * g.sC);
        store_acc<OUT, FN, FM>(Cb, g.ldc, g.M, g.N, m0 + grp * WM, n0 + wn * WN, acc, vec_store != 0);
        phase_barrier();           // no wave refills the ring while another still reads it
    }
}

hipError_t launch_pingpong(const GemmArgs& g, int out, const Plan& p, hipStream_t s) {
    if (out == OUT_F32)
        hipLaunchKernelGGL((gemm_pingpong_kernel<OUT_F32, true>), dim3(p.grid_x), dim3(512), 0, s, g, p.grid,
                           p.vec_store);
    else
        hipLaunchKernelGGL((gemm_pingpong_kernel<OUT_BF16, true>), dim3(p.grid_x), dim3(512), 0, s, g, p.grid,
                           p.vec_store);
    return hipGetLastError();
}

}  // namespace tmm
