// Fused attention forward: O = softmax(scale Q K^T, causal mask) V with grouped-query heads.
//
// The page "Modern GPU Programming for MLSys：深度解读" (outline of Part IV, Flash Attention
// 4) lists what the kernel is made of: a softmax between two matrix products, online-softmax
// rescaling (the keys are visited block by block; the running maximum m and sum l of each
// row are updated and the partial output rescaled by exp(m_old - m_new)), causal masking and
// grouped-query attention (query head h reads key/value head h / (Hq / Hkv)).
//
// attn_simple_kernel: one wave per query row, 64 keys per step: lane t scores key j0 + t
// (dot product over d from the row of Q staged in LDS), the wave takes the step's maximum and
// sum, and each lane accumulates d / 64 output columns over the step's keys.  Any d <= 256
// (d % 8 == 0); the general path and the reference the faster kernel is tested beside.
//
// attn_mfma_kernel (d = 64 or 128): a workgroup of 4 waves takes 128 query rows of one head
// (32 per wave) and visits the keys in blocks of 64, K and V tiles staged in LDS by
// direct-to-LDS loads (two buffers: block b+1 loads while block b is used).  Per block and
// wave, with v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T: the key tile is the first operand and the wave's Q rows (held in registers
//     for the whole loop) the second, so each lane ends with one query (lane mod 16) and 4
//     keys (4 (lane / 16) + r) of each 16-key tile: the online-softmax maximum and sum of a
//     query are an in-lane reduction over 16 values and two exchanges across lane groups.
//   P = exp(S - m), rounded to bf16, is the second operand of O^T = V^T P^T as it stands in
//     the accumulators: for a 32-key step (tiles t0, t1) lane group g holds keys 16 t0 + 4 g
//     + (0..3) and 16 t1 + 4 g + (0..3), which is taken as the step's k order; the V^T operand
//     follows the same order: two ds_read_b64_tr_b16 per fragment, each giving a lane 4
//     consecutive keys of one head-dim column (the transposing read's lane layout: within 16
//     lanes, lane i element e is element i mod 4 of the 8 bytes addressed by lane 4 e + i / 4).
//   O^T accumulates in registers; each lane ends with 4 consecutive head-dim values of one
//     query (vector stores).  Rescaling is selective: the reference maximum m of a query moves
//     (and O^T and the sum are multiplied by exp(m_old - m_new)) only when a new score exceeds
//     it by more than a factor 2^8, so most blocks skip the rescale.
// LDS rows are d * 2 bytes, their 16-byte chunks permuted by an XOR swizzle per row so that
// the K fragment reads and the transposing V reads are free of bank conflicts.
// Scores and the exponent are in base 2 (scale log2(e) folded into the scores).
#include <math.h>

#include "launch.hpp"

namespace tmm {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// Last key (exclusive) row i may see.
__device__ __forceinline__ int64_t attn_key_end(const AttnArgs& g, int64_t i) {
    if (!g.causal) return g.Lk;
    const int64_t e = i + (g.Lk - g.Lq) + 1;
    return e < 0 ? 0 : (e < g.Lk ? e : g.Lk);
}

template <int OUT>
__global__ __launch_bounds__(256) void attn_simple_kernel(AttnArgs g) {
    __shared__ float qs[4][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + w;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const bool active = i < g.Lq;
    const int64_t gk = h / (g.Hq / g.Hkv);
    const int d = static_cast<int>(g.d);
    if (active) {
        const uint16_t* q = g.Q + ((b * g.Hq + h) * g.Lq + i) * g.d;
        for (int c = lane; c < d; c += 64) qs[w][c] = bf16_to_f32(q[c]);
    }
    __syncthreads();
    if (!active) return;   // no barrier follows
    const uint16_t* Kb = g.K + (b * g.Hkv + gk) * g.Lk * g.d;
    const uint16_t* Vb = g.V + (b * g.Hkv + gk) * g.Lk * g.d;
    const int64_t jend = attn_key_end(g, i);
    float m = -INFINITY, l = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t j0 = 0; j0 < jend; j0 += 64) {
        const int64_t j = j0 + lane;
        float s = -INFINITY;
        if (j < jend) {
            const uint16_t* kr = Kb + j * g.d;
            float acc = 0.f;
            for (int c = 0; c < d; ++c) acc = fmaf(qs[w][c], bf16_to_f32(kr[c]), acc);
            s = acc * g.scale;
        }
        const float mn = fmaxf(m, wave_max(s));   // finite: key j0 is allowed
        const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
        const float p = j < jend ? expf(s - mn) : 0.f;
        l = l * alpha + wave_sum(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] *= alpha;
        const int64_t nkeys = jend - j0 < 64 ? jend - j0 : 64;
        for (int jj = 0; jj < nkeys; ++jj) {
            const float pj = __shfl(p, jj, 64);
            const uint16_t* vr = Vb + (j0 + jj) * g.d;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = lane + 64 * t;
                if (c < d) o[t] = fmaf(pj, bf16_to_f32(vr[c]), o[t]);
            }
        }
        m = mn;
    }
    const int64_t orow = ((b * g.Hq + h) * g.Lq + i) * g.d;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int c = lane + 64 * t;
        if (c >= d) continue;
        if constexpr (OUT == OUT_F32)
            static_cast<float*>(g.O)[orow + c] = o[t] * inv;
        else
            static_cast<uint16_t*>(g.O)[orow + c] = f32_to_bf16(o[t] * inv);
    }
    if (g.LSE && lane == 0) g.LSE[(b * g.Hq + h) * g.Lq + i] = l > 0.f ? m + logf(l) : -INFINITY;
}

namespace at {
constexpr int BKV = 64;
}

// 16-query tiles per wave of attn_mfma_kernel at d = 128 and d = 64 (a workgroup of 4 waves
// takes 64 QT queries).  QT = 2 runs two workgroups per CU; QT = 4 halves the LDS fragment
// reads per MFMA (every K and V^T fragment a wave reads serves twice as many queries) with
// one workgroup (one wave per SIMD, accumulators in AGPRs).
#ifndef TMM_ATTN_QT128
#define TMM_ATTN_QT128 2
#endif
#ifndef TMM_ATTN_QT64
#define TMM_ATTN_QT64 2
#endif

// attn_mfma_kernel's key loop: one barrier per block, block j+1's loads issued after it (1),
// or two, block j+1's loads issued before the first (0).
#ifndef TMM_ATTN_ONE_BARRIER
#define TMM_ATTN_ONE_BARRIER 1
#endif

// Wave priority raised over each block's two MFMA phases (1) or left alone (0).
#ifndef TMM_ATTN_SETPRIO
#define TMM_ATTN_SETPRIO 1
#endif

// Vector instructions the pipelined attention kernel places after each score MFMA.
#ifndef TMM_ATTN_PIPE_VALU
#define TMM_ATTN_PIPE_VALU 6
#endif

// Query rows per workgroup of each MFMA attention kernel (attn_pipe_kernel: 2 query tiles of 16
// per wave, always).
int attn_rows_per_workgroup(int kernel, int d) {
    if (kernel == K_ATTN_PIPE) return 128;
    return 64 * (d == 128 ? TMM_ATTN_QT128 : TMM_ATTN_QT64);
}

// Max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups that hold one query's
// scores) with gfx950's row swaps, in the VALU: permlane16_swap(x, x) leaves rows (0, 0, 2, 2)
// in one result and (1, 1, 3, 3) in the other, permlane32_swap(x, x) the low and the high
// half; every lane combines the two in the same order, so the four copies agree bitwise.
__device__ __forceinline__ float group4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Work item (batch b, query head h, query block qb) of the MFMA attention workgroup with grid
// (query blocks, Hq, B).  Workgroups are dispatched in linear order (x fastest) and handed to
// the 8 XCDs round-robin; the linear id is mapped so that each XCD gets a contiguous range of
// the order (b, K/V head, query block, query head of the group): the query blocks of one K/V
// head then run on one XCD, whose L2 serves their repeated reads of that head's K and V, and
// within an XCD the query blocks are started in launch-priority order (causal: the blocks
// with the most keys first) across the heads of the group.
#ifndef TMM_ATTN_XCD_MAP
#define TMM_ATTN_XCD_MAP 1   // 0: the plain order (b = z, h = y, query block from x)
#endif
__device__ __forceinline__ void attn_block_of(const AttnArgs& g, int64_t& b, int64_t& h, int64_t& qb) {
    if (!TMM_ATTN_XCD_MAP) {
        b = blockIdx.z, h = blockIdx.y;
        qb = g.causal ? static_cast<int64_t>(gridDim.x) - 1 - blockIdx.x : blockIdx.x;
        return;
    }
    constexpr int64_t XCD = 8;
    const int64_t nqb = gridDim.x, total = nqb * gridDim.y * gridDim.z;
    const int64_t t = blockIdx.x + nqb * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
    const int64_t per = total / XCD, extra = total % XCD, x = t % XCD, local = t / XCD;
    const int64_t L = x < extra ? x * (per + 1) + local : extra * (per + 1) + (x - extra) * per + local;
    const int64_t G = g.Hq / g.Hkv;
    const int64_t gi = L % G, rest = L / G, qi = rest % nqb, rest2 = rest / nqb;
    const int64_t kvh = rest2 % g.Hkv;
    b = rest2 / g.Hkv;
    h = kvh * G + gi;
    qb = g.causal ? nqb - 1 - qi : qi;
}

template <int D, int OUT, int QT>
__global__ __launch_bounds__(256, QT == 2 ? 2 : 1) void attn_mfma_kernel(AttnArgs g) {
    using namespace at;
    constexpr int WQ = 16 * QT, BQ = 4 * WQ;   // queries per wave, per workgroup
    constexpr int ROWB = D * 2;            // bytes per LDS row
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int TILE = BKV * ROWB;       // one K or V tile
    constexpr int RPI = 1024 / ROWB;       // rows per 1 KB load instruction
    constexpr int LPT = TILE / 1024 / 4;   // load instructions per wave per tile
    constexpr int KS = D / 32;             // k steps of S^T
    constexpr int DT = D / 16;             // 16-wide head-dim tiles of O^T
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][TILE];   // [buffer][K, V]
    // LDS position of 16-byte chunk c of K row r: c ^ kswz(r); of V row r: c ^ vswz(r).  The
    // LDS has 64 banks of 4 bytes (a 256-byte bank row, RP rows of a tile).  A K fragment read
    // (16 rows, one chunk each) then meets 16 different chunk positions at d = 128 and 8
    // positions in each of the two row halves at d = 64; a transposing V read (8 rows of 32
    // bytes per 256 bytes delivered) meets 8 different 32-byte positions of a bank row.  Both
    // are free of bank conflicts (measured: SQ_LDS_BANK_CONFLICT 0).
    constexpr int RP = 256 / ROWB;
    auto kswz = [](int r) { return r & (CPR - 1); };
    auto vswz = [](int r) { return 2 * ((r / RP) & (CPR / 2 - 1)); };

    const int lane = lane_id(), w = wave_id();
    const int lg = lane >> 4, lq = lane & 15;
    int64_t b, h, qb;
    attn_block_of(g, b, h, qb);
    const int64_t gk = h / (g.Hq / g.Hkv);
    const int64_t q0 = qb * BQ, qw = q0 + WQ * w;
    const int64_t shift = g.Lk - g.Lq;                 // causal: key j <= query i + shift
    const float sl2 = g.scale * 1.4426950408889634f;    // scores in base 2
    const uint16_t* Kb = g.K + (b * g.Hkv + gk) * g.Lk * D;
    const uint16_t* Vb = g.V + (b * g.Hkv + gk) * g.Lk * D;

    // Keys this workgroup visits: up to the last allowed key of its last query row.
    const int64_t q_last = min<int64_t>(q0 + BQ, g.Lq) - 1;
    int64_t kend = g.Lk;
    if (g.causal) kend = max<int64_t>(0, min<int64_t>(g.Lk, q_last + shift + 1));
    const int nblk = static_cast<int>((kend + BKV - 1) / BKV);

    // Q fragments (second operand of S^T): query qw + 16 qt + lq, head-dim 32 kk + 8 lg .. + 7.
    bf16x8 qf[QT][KS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int64_t qi = qw + 16 * qt + lq;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (qi < g.Lq) v = *reinterpret_cast<const u32x4*>(g.Q + ((b * g.Hq + h) * g.Lq + qi) * D + 32 * kk + 8 * lg);
            qf[qt][kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // Direct-to-LDS loads of key block j into buffer `buf` (rows past Lk read zeros).
    const int lrow = lane / CPR, lchunk = lane % CPR;
    auto load_block = [&](int j, int buf) {
        const int64_t kv0 = static_cast<int64_t>(j) * BKV;
        const int64_t rows = min<int64_t>(BKV, g.Lk - kv0);
        const uint32_t bytes = static_cast<uint32_t>(rows * ROWB);
        const auto rk = make_rsrc(Kb + kv0 * D, bytes), rv = make_rsrc(Vb + kv0 * D, bytes);
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int r = (4 * i + w) * RPI + lrow;   // row of this lane (< BKV)
            const uint32_t ok = static_cast<uint32_t>(r * ROWB);
            load_lds_16(rk, &lds[buf][0][(4 * i + w) * 1024], ok + 16u * static_cast<uint32_t>(lchunk ^ kswz(r)), 0u);
            load_lds_16(rv, &lds[buf][1][(4 * i + w) * 1024], ok + 16u * static_cast<uint32_t>(lchunk ^ vswz(r)), 0u);
        }
    };

    f32x4 oacc[DT][QT];
    float m[QT], l[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[qt] = -INFINITY, l[qt] = 0.f;
    }
    // Causal: key blocks that start past the last key this wave's last query may see add
    // nothing to its rows; the wave skips their products and softmax (not the barriers).
    const int64_t wave_kend = g.causal ? qw + WQ - 1 + shift : g.Lk - 1;

    if (nblk > 0) load_block(0, 0);
    for (int j = 0; j < nblk; ++j) {
        const int buf = j & 1;
        if (TMM_ATTN_ONE_BARRIER) {
            // One barrier per block: after it every wave's loads of block j have landed and
            // every wave is done with block j-1, whose buffer then takes block j+1.
            wait_vmcnt<0>();
            barrier();
            if (j + 1 < nblk) load_block(j + 1, buf ^ 1);
        } else {
            if (j + 1 < nblk) {
                load_block(j + 1, buf ^ 1);
                wait_vmcnt<2 * LPT>();   // block j's loads (this wave) have landed
            } else {
                wait_vmcnt<0>();
            }
            barrier();                   // ... and every wave's
        }
        const uint8_t* Kt = lds[buf][0];
        const uint8_t* Vt = lds[buf][1];
        const int64_t kv0 = static_cast<int64_t>(j) * BKV;
        if (kv0 <= wave_kend) {   // wave-uniform

        if (TMM_ATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
        // S^T = K Q^T: 4 key tiles x 2 query tiles.  Every K fragment of the block is read
        // first, then the MFMAs run in the same order, each waiting only for its own read.
        f32x4 s[4][QT];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) s[t][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kf[KS][4];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * t + lq;
                kf[kk][t] = *reinterpret_cast<const bf16x8*>(Kt + r * ROWB + 16 * ((4 * kk + lg) ^ kswz(r)));
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) s[t][qt] = mfma_16x16x32(kf[kk][t], qf[qt][kk], s[t][qt]);

        if (TMM_ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
        // Online softmax per query (lane's query: qw + 16 qt + lq; keys kv0 + 16 t + 4 lg + r).
        // scale > 0 (planner), so the maximum is taken over the raw scores and scaled once, and
        // each probability is one FMA and one exp2: exp2(s sl2 - m); masked scores are -inf,
        // for which exp2 gives 0 (an all-masked row uses 0 as its reference instead of -inf).
        const bool edge = kv0 + BKV > g.Lk || (g.causal && kv0 + BKV - 1 > qw + shift);
        u32x2 pb[QT][4];   // P in bf16: [query tile][key tile], 4 keys each
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            if (edge) {
                const int64_t qi = qw + 16 * qt + lq;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t kj = kv0 + 16 * t + 4 * lg + r;
                        if (kj >= g.Lk || (g.causal && kj > qi + shift)) s[t][qt][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[t][qt][r]);
            mx = group4_max(mx) * sl2;
            // Selective rescaling: the reference maximum moves only when a score exceeds it by
            // more than 2^8 (so probabilities stay <= 256, exact in fp32 sums and within bf16's
            // range); otherwise alpha is 1 and the accumulators are left as they are.
            const bool need = m[qt] == -INFINITY || mx > m[qt] + 8.f;
            const float mn = need ? mx : m[qt];
            const float alpha = !need ? 1.f : (m[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[qt] - mn));
            const float nref = mn == -INFINITY ? 0.f : -mn;
            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(fmaf(s[t][qt][r], sl2, nref));
                    sum += p[r];
                }
                pb[qt][t] = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
            }
            sum = group4_sum(sum);
            l[qt] = l[qt] * alpha + sum;
            m[qt] = mn;
            if (__builtin_amdgcn_ballot_w64(need) != 0) {   // wave-uniform
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[dt][qt][r] *= alpha;
            }
        }

        if (TMM_ATTN_SETPRIO) __builtin_amdgcn_s_setprio(1);
        // O^T += V^T P^T over two 32-key steps (key tiles 2 st, 2 st + 1).  The V^T fragments
        // of both steps are read first (two transposing reads each); the first step's MFMAs
        // wait only for the first step's reads, so the second step's reads overlap them.
        u32x2 hv[2][DT][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    // rows 16 (2 st + e2) + lane / 4, columns 16 dt + 4 (lane mod 4) .. + 3
                    const int r = 16 * (2 * st + e2) + lane / 4;
                    const int c = 2 * dt + ((lane & 3) >> 1);
                    const int off = r * ROWB + 16 * (c ^ vswz(r)) + 8 * (lane & 1);
                    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(Vt + off)));
                    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hv[st][dt][e2]) : "v"(addr) : "memory");
                }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8 pf[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                pf[qt] = __builtin_bit_cast(bf16x8, u32x4{pb[qt][2 * st][0], pb[qt][2 * st][1], pb[qt][2 * st + 1][0],
                                                          pb[qt][2 * st + 1][1]});
            // The transposing reads are assembly, whose results LLVM takes as ready at once:
            // wait for them here, fenced so that no use is scheduled above the wait.  LDS
            // reads complete in order; at most 2 DT - 1 <= 15 of the second step's reads may
            // still be outstanding once the first step's have landed.
            __builtin_amdgcn_sched_barrier(0);
            if (st == 0)
                wait_cnt<63, 2 * DT - 1>();
            else
                wait_cnt<63, 0>();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[st][dt][0], hv[st][dt][1], 0, 1, 2, 3));
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = mfma_16x16x32(vf, pf[qt], oacc[dt][qt]);
            }
        }
        if (TMM_ATTN_SETPRIO) __builtin_amdgcn_s_setprio(0);
        }          // kv0 <= wave_kend
        if (!TMM_ATTN_ONE_BARRIER)
            barrier();   // every wave is done with buffer `buf` before block j + 2 is loaded into it
    }

    // O = O^T / l: lane holds query qw + 16 qt + lq, head-dim 16 dt + 4 lg .. + 3.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int64_t qi = qw + 16 * qt + lq;
        if (qi >= g.Lq) continue;
        const float inv = l[qt] > 0.f ? 1.f / l[qt] : 0.f;
        const int64_t orow = ((b * g.Hq + h) * g.Lq + qi) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 v = {oacc[dt][qt][0] * inv, oacc[dt][qt][1] * inv, oacc[dt][qt][2] * inv, oacc[dt][qt][3] * inv};
            const int64_t c = 16 * dt + 4 * lg;
            if constexpr (OUT == OUT_F32)
                *reinterpret_cast<f32x4*>(static_cast<float*>(g.O) + orow + c) = v;
            else
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.O) + orow + c) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        if (g.LSE && lg == 0)
            g.LSE[(b * g.Hq + h) * g.Lq + qi] = l[qt] > 0.f ? (m[qt] + log2f(l[qt])) * 0.6931471805599453f : -INFINITY;
    }
}

// attn_pipe_kernel (d = 64 or 128): the tiles, LDS layouts and arithmetic of attn_mfma_kernel
// (32 queries per wave, 64-key blocks, S^T = K Q^T, base-2 online softmax with selective
// rescaling, O^T += V^T P^T from transposing reads), with the score products of block j + 1
// issued while block j's softmax runs.  In one wave the MFMAs of a block wait for its
// softmax and the softmax for its MFMAs; here the score MFMAs of the next block do not
// depend on the softmax of this one, so the two are interleaved (one MFMA, then a group of
// VALU instructions, fixed with scheduling groups) and the matrix and vector units run at
// the same time.  K is loaded two blocks ahead (its fragments are read one block early), V
// one block ahead; both rings have two slots, as before.
//   iteration j (scores of block j already in registers, masked):
//     load K(j+2) into K(j)'s slot, V(j+1) into V(j-1)'s slot; wait for K(j+1), V(j); barrier
//     scores of block j+1 (K(j+1) fragments, MFMAs)   interleaved with   softmax of block j
//     rescale O where the reference maximum moved; mask block j+1's scores if it is an edge
//     O^T += V(j)^T P(j)^T; barrier
// The scores of the block past the last (read from zeros) are computed and dropped.
template <int D, int OUT>
__global__ __launch_bounds__(256, 2) void attn_pipe_kernel(AttnArgs g) {
    using namespace at;
    constexpr int QT = 2, WQ = 32, BQ = 128;
    constexpr int ROWB = D * 2, CPR = D / 8, TILE = BKV * ROWB, RPI = 1024 / ROWB;
    constexpr int LPT = TILE / 1024 / 4;   // load instructions per wave per tile
    constexpr int KS = D / 32, DT = D / 16;
    __shared__ __attribute__((aligned(1024))) uint8_t kl[2][TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t vl[2][TILE];
    constexpr int RP = 256 / ROWB;
    auto kswz = [](int r) { return r & (CPR - 1); };
    auto vswz = [](int r) { return 2 * ((r / RP) & (CPR / 2 - 1)); };

    const int lane = lane_id(), w = wave_id();
    const int lg = lane >> 4, lq = lane & 15;
    int64_t b, h, qb;
    attn_block_of(g, b, h, qb);
    const int64_t gk = h / (g.Hq / g.Hkv);
    const int64_t q0 = qb * BQ, qw = q0 + WQ * w;
    const int64_t shift = g.Lk - g.Lq;
    const float sl2 = g.scale * 1.4426950408889634f;
    const uint16_t* Kb = g.K + (b * g.Hkv + gk) * g.Lk * D;
    const uint16_t* Vb = g.V + (b * g.Hkv + gk) * g.Lk * D;
    const int64_t q_last = min<int64_t>(q0 + BQ, g.Lq) - 1;
    int64_t kend = g.Lk;
    if (g.causal) kend = max<int64_t>(0, min<int64_t>(g.Lk, q_last + shift + 1));
    const int nblk = static_cast<int>((kend + BKV - 1) / BKV);

    bf16x8 qf[QT][KS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int64_t qi = qw + 16 * qt + lq;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (qi < g.Lq) v = *reinterpret_cast<const u32x4*>(g.Q + ((b * g.Hq + h) * g.Lq + qi) * D + 32 * kk + 8 * lg);
            qf[qt][kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // Direct-to-LDS loads of the K or V tile of key block j (rows past Lk, or a block wholly
    // past it, read zeros).
    const int lrow = lane / CPR, lchunk = lane % CPR;
    auto load_tile = [&](const uint16_t* base, bool is_v, int j, uint8_t* dst) {
        const int64_t kv0 = static_cast<int64_t>(j) * BKV;
        const int64_t rows = max<int64_t>(0, min<int64_t>(BKV, g.Lk - kv0));
        const auto r = make_rsrc(rows > 0 ? base + kv0 * D : base, static_cast<uint32_t>(rows * ROWB));
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int row = (4 * i + w) * RPI + lrow;
            const uint32_t off = static_cast<uint32_t>(row * ROWB) +
                                 16u * static_cast<uint32_t>(lchunk ^ (is_v ? vswz(row) : kswz(row)));
            load_lds_16(r, dst + (4 * i + w) * 1024, off, 0u);
        }
    };
    // S^T of the key block whose K tile is at Kt (4 key tiles x 2 query tiles).
    auto scores = [&](f32x4 (&sc)[4][QT], const uint8_t* Kt) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sc[t][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bf16x8 kf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * t + lq;
                kf[t] = *reinterpret_cast<const bf16x8*>(Kt + r * ROWB + 16 * ((4 * kk + lg) ^ kswz(r)));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) sc[t][qt] = mfma_16x16x32(kf[t], qf[qt][kk], sc[t][qt]);
        }
    };
    // Masked scores of block j at -inf (only blocks that reach past Lk or the diagonal): key
    // kv0 + o of query row qi is allowed when o < lim(qi), lim = min(Lk, qi + shift + 1) - kv0
    // clamped to [0, BKV]; one compare and select per score, no branches.
    auto mask = [&](f32x4 (&sc)[4][QT], int j) {
        const int64_t kv0 = static_cast<int64_t>(j) * BKV;
        if (kv0 + BKV > g.Lk || (g.causal && kv0 + BKV - 1 > qw + shift)) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                int64_t e = g.Lk;
                if (g.causal) e = min<int64_t>(e, qw + 16 * qt + lq + shift + 1);
                const int lim = static_cast<int>(max<int64_t>(0, min<int64_t>(BKV, e - kv0)));
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sc[t][qt][r] = 16 * t + 4 * lg + r < lim ? sc[t][qt][r] : -INFINITY;
            }
        }
    };

    f32x4 oacc[DT][QT];
    float m[QT], l[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[qt] = -INFINITY, l[qt] = 0.f;
    }

    f32x4 sc[4][QT];   // scores of the block being finished
    if (nblk > 0) {
        load_tile(Kb, false, 0, kl[0]);
        load_tile(Vb, true, 0, vl[0]);
        load_tile(Kb, false, 1, kl[1]);
        wait_vmcnt<2 * LPT>();   // K(0) has landed (this wave) ...
        barrier();               // ... and every wave's
        scores(sc, kl[0]);
        mask(sc, 0);
        barrier();               // every wave has read K(0) before K(2) is loaded into its slot
    }
    for (int j = 0; j < nblk; ++j) {
        load_tile(Kb, false, j + 2, kl[j & 1]);
        load_tile(Vb, true, j + 1, vl[(j + 1) & 1]);
        wait_vmcnt<2 * LPT>();   // K(j+1) and V(j) have landed (this wave) ...
        barrier();               // ... and every wave's

        // Scores of block j+1 interleaved with the softmax of block j.
        f32x4 sn[4][QT];
        scores(sn, kl[(j + 1) & 1]);
        u32x2 pb[QT][4];
        float alpha[QT];
        bool need[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            float mx4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                mx4[t] = fmaxf(fmaxf(sc[t][qt][0], sc[t][qt][1]), fmaxf(sc[t][qt][2], sc[t][qt][3]));
            float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
            mx = group4_max(mx) * sl2;
            need[qt] = m[qt] == -INFINITY || mx > m[qt] + 8.f;
            const float mn = need[qt] ? mx : m[qt];
            alpha[qt] = !need[qt] ? 1.f : (m[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[qt] - mn));
            const float nref = mn == -INFINITY ? 0.f : -mn;
            float sum4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[t][qt][r], sl2, nref));
                sum4[t] = (p[0] + p[1]) + (p[2] + p[3]);
                pb[qt][t] = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
            }
            l[qt] = l[qt] * alpha[qt] + group4_sum((sum4[0] + sum4[1]) + (sum4[2] + sum4[3]));
            m[qt] = mn;
        }
        // Scheduling groups: for every score MFMA, one MFMA and then up to TMM_ATTN_PIPE_VALU
        // vector instructions of the softmax (the fragment reads are left to the scheduler).
#pragma unroll
        for (int i = 0; i < 4 * KS * QT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, TMM_ATTN_PIPE_VALU, 0);   // VALU
        }
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            if (__builtin_amdgcn_ballot_w64(need[qt]) != 0) {   // wave-uniform
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[dt][qt][r] *= alpha[qt];
            }
        mask(sn, j + 1);

        // O^T += V(j)^T P(j)^T, as in attn_mfma_kernel.
        const uint8_t* Vt = vl[j & 1];
        u32x2 hv[2][DT][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    const int r = 16 * (2 * st + e2) + lane / 4;
                    const int c = 2 * dt + ((lane & 3) >> 1);
                    const int off = r * ROWB + 16 * (c ^ vswz(r)) + 8 * (lane & 1);
                    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(Vt + off)));
                    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hv[st][dt][e2]) : "v"(addr) : "memory");
                }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8 pf[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                pf[qt] = __builtin_bit_cast(bf16x8, u32x4{pb[qt][2 * st][0], pb[qt][2 * st][1], pb[qt][2 * st + 1][0],
                                                          pb[qt][2 * st + 1][1]});
            __builtin_amdgcn_sched_barrier(0);
            if (st == 0)
                wait_cnt<63, 2 * DT - 1>();
            else
                wait_cnt<63, 0>();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[st][dt][0], hv[st][dt][1], 0, 1, 2, 3));
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = mfma_16x16x32(vf, pf[qt], oacc[dt][qt]);
            }
        }
        barrier();   // every wave is done with K(j+1) and V(j) before their slots are refilled
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sc[t][qt] = sn[t][qt];
    }
    wait_vmcnt<0>();   // the loads past the last block have landed before the workgroup ends

#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int64_t qi = qw + 16 * qt + lq;
        if (qi >= g.Lq) continue;
        const float inv = l[qt] > 0.f ? 1.f / l[qt] : 0.f;
        const int64_t orow = ((b * g.Hq + h) * g.Lq + qi) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4 v = {oacc[dt][qt][0] * inv, oacc[dt][qt][1] * inv, oacc[dt][qt][2] * inv, oacc[dt][qt][3] * inv};
            const int64_t c = 16 * dt + 4 * lg;
            if constexpr (OUT == OUT_F32)
                *reinterpret_cast<f32x4*>(static_cast<float*>(g.O) + orow + c) = v;
            else
                *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.O) + orow + c) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        if (g.LSE && lg == 0)
            g.LSE[(b * g.Hq + h) * g.Lq + qi] = l[qt] > 0.f ? (m[qt] + log2f(l[qt])) * 0.6931471805599453f : -INFINITY;
    }
}

hipError_t launch_attention(const AttnArgs& g, int out, const Plan& p, hipStream_t s) {
    const dim3 grid(p.grid_x, p.grid_y, p.grid_z);
    if (p.kernel == K_ATTN_PIPE) {
        if (g.d == 128 && out == OUT_F32)
            hipLaunchKernelGGL((attn_pipe_kernel<128, OUT_F32>), grid, dim3(256), 0, s, g);
        else if (g.d == 128)
            hipLaunchKernelGGL((attn_pipe_kernel<128, OUT_BF16>), grid, dim3(256), 0, s, g);
        else if (out == OUT_F32)
            hipLaunchKernelGGL((attn_pipe_kernel<64, OUT_F32>), grid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((attn_pipe_kernel<64, OUT_BF16>), grid, dim3(256), 0, s, g);
    } else if (p.kernel == K_ATTN_MFMA) {
        constexpr int Q1 = TMM_ATTN_QT128, Q6 = TMM_ATTN_QT64;
        if (g.d == 128 && out == OUT_F32)
            hipLaunchKernelGGL((attn_mfma_kernel<128, OUT_F32, Q1>), grid, dim3(256), 0, s, g);
        else if (g.d == 128)
            hipLaunchKernelGGL((attn_mfma_kernel<128, OUT_BF16, Q1>), grid, dim3(256), 0, s, g);
        else if (out == OUT_F32)
            hipLaunchKernelGGL((attn_mfma_kernel<64, OUT_F32, Q6>), grid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((attn_mfma_kernel<64, OUT_BF16, Q6>), grid, dim3(256), 0, s, g);
    } else if (out == OUT_F32) {
        hipLaunchKernelGGL(attn_simple_kernel<OUT_F32>, grid, dim3(256), 0, s, g);
    } else {
        hipLaunchKernelGGL(attn_simple_kernel<OUT_BF16>, grid, dim3(256), 0, s, g);
    }
    return hipGetLastError();
}

}  // namespace tmm
