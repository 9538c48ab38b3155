// Shared device-side building blocks of the gfx950 GEMM kernels: vector types, the bf16
// conversions, the buffer-resource helpers used by the direct-to-LDS loads, and the
// XCD-aware tile order.  Internal to libgemm_bf16.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tmm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

enum { OUT_F32 = 0, OUT_BF16 = 1 };

// Problem description handed to every kernel by value.  Pointers are device pointers;
// leading dimensions and batch strides are in elements.  la / lb: operand layouts
// (LAYOUT_K: element (i, k) at i * ld + k; LAYOUT_MN: at k * ld + i).
enum { LAYOUT_K = 0, LAYOUT_MN = 1 };
struct GemmArgs {
    int64_t batch, M, N, K;
    const uint16_t* A;
    int64_t lda, sA;
    const uint16_t* B;
    int64_t ldb, sB;
    void* C;
    int64_t ldc, sC;
    int la = LAYOUT_K, lb = LAYOUT_K;
    // Split K: each tile's K blocks are divided into `splits` contiguous ranges; with
    // splits > 1 each range's fp32 partial product goes to ws[s][batch][M][N] and a reduction
    // writes C.
    float* ws = nullptr;
    int splits = 1;
};

// Tile grid of one launch: tiles_m x tiles_n tiles per batch item, `total` over the batch.
// Block-scaled 8-bit GEMM (gemm_mx): element formats (the codes the scaled MFMA takes) and
// arguments; pitches and sizes in bytes, one E8M0 scale byte per 32 k of a row.
enum { MX_E4M3 = 0, MX_E5M2 = 1 };
struct MxArgs {
    int64_t M, N, K;
    const uint8_t* A;
    int64_t lda;
    const uint8_t* SA;
    int64_t ldsa;
    const uint8_t* B;
    int64_t ldb;
    const uint8_t* SB;
    int64_t ldsb;
    void* C;
    int64_t ldc;
    int fa, fb;
};

// Attention forward (attention_fwd): [B][H][L][d] bf16 tensors, contiguous.
struct AttnArgs {
    int64_t B, Hq, Hkv, Lq, Lk, d;
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    void* O;
    float* LSE;
    float scale;
    int causal;
};

struct TileGrid {
    int tiles_m, tiles_n, total, group_m;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 b = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, b);
}

// Two values in one v_cvt_pk_bf16_f32 (lo in bits 0-15), rounded as f32_to_bf16 rounds.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Buffer resource over [base, base + bytes): raw (stride 0) addressing, so a lane whose
// offset is >= bytes reads zeros.  The fourth dword is the gfx9 raw-buffer format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// An offset no buffer of this library reaches (buffers are capped below 2^31 bytes).
constexpr uint32_t OOB = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global (through the buffer resource) straight into LDS at
// lds_base + 16 * lane; lds_base must be wave-uniform.
__device__ __forceinline__ void load_lds_16(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                            uint32_t voffset, uint32_t soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 16, voffset, soffset, 0, 0);
}

// Map a linear work index to a tile so that the workgroups one XCD runs get neighbouring
// tiles.  Workgroup ids are handed to the 8 XCDs round-robin, so index t runs on XCD t % 8;
// the bijection below gives XCD x a contiguous range of logical tiles, which are then
// rastered in groups of `group_m` tile rows so that the A and B panels they share stay in
// that XCD's L2.
// The XCD part of that order on n items: index t (on XCD t % 8) -> logical index, XCD x taking
// a contiguous range.  A bijection on [0, n).
__device__ __forceinline__ int xcd_order(int t, int n) {
    constexpr int XCD = 8;
    const int per = n / XCD, extra = n % XCD;
    const int x = t % XCD, local = t / XCD;
    return (x < extra) ? x * (per + 1) + local : extra * (per + 1) + (x - extra) * per + local;
}

// The raster part: logical index L -> (batch item, tile row, tile column), tile rows taken in
// groups of group_m.
__device__ __forceinline__ void raster_of(int L, const TileGrid& g, int& batch, int& tm, int& tn) {
    int tiles = g.tiles_m * g.tiles_n;
    batch = L / tiles;
    int r = L - batch * tiles;
    int group = g.group_m * g.tiles_n;
    int first_m = (r / group) * g.group_m;
    int gm = min(g.tiles_m - first_m, g.group_m);
    int within = r % group;
    tm = first_m + within % gm;
    tn = within / gm;
}

__device__ __forceinline__ void tile_of(int t, const TileGrid& g, int& batch, int& tm, int& tn) {
    raster_of(xcd_order(t, g.total), g, batch, tm, tn);
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier with no memory fence: the callers wait for their own loads with an
// explicit s_waitcnt first.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt through the builtin, so that the compiler's own wait insertion sees it.  gfx9
// encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]; an all-ones field
// does not wait on that counter.
template <int VM, int LGKM = 15>
__device__ __forceinline__ void wait_cnt() {
    static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "counter range");
    constexpr int enc = (VM & 15) | (7 << 4) | (LGKM << 8) | ((VM >> 4) << 14);
    __builtin_amdgcn_s_waitcnt(enc);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    wait_cnt<N, 15>();
}

}  // namespace tmm

namespace tmm {

// Write a wave's register-blocked accumulator to C.  The MFMA was issued with the B tile as
// its first operand and the A tile as its second, so accumulator fragment [fi][fj] holds
// D[n][m] = C[m][n] for a 16 (n) x 16 (m) block, and lane l, register r carries
//     m = m_base + 16*fj + (l % 16),   n = n_base + 16*fi + 4*(l / 16) + r,
// i.e. four consecutive n of one C row: one 16-byte (fp32) or 8-byte (bf16) store.
// `vec_ok`: C's base and pitch allow those vector stores.  Elements outside M x N are
// skipped.
template <int OUT, int FN, int FM>
__device__ __forceinline__ void store_acc(void* Cp, int64_t ldc, int64_t M, int64_t N,
                                          int64_t m_base, int64_t n_base,
                                          const f32x4 (&acc)[FN][FM], bool vec_ok) {
    const int lane = lane_id();
    const bool full = vec_ok && (m_base + 16 * FM <= M) && (n_base + 16 * FN <= N);
    if constexpr (OUT == OUT_F32) {
#pragma unroll
        for (int fj = 0; fj < FM; ++fj) {
            const int64_t m = m_base + 16 * fj + (lane & 15);
#pragma unroll
            for (int fi = 0; fi < FN; ++fi) {
                const int64_t n = n_base + 16 * fi + 4 * (lane >> 4);
                const f32x4 v = acc[fi][fj];
                float* row = static_cast<float*>(Cp) + m * ldc;
                if (full) {
                    *reinterpret_cast<f32x4*>(row + n) = v;
                } else if (m < M) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) row[n + r] = v[r];
                }
            }
        }
    } else {
        // Round every accumulator to bf16 first (halves the live registers), then store.
        u32x2 p[FN][FM];
#pragma unroll
        for (int fi = 0; fi < FN; ++fi)
#pragma unroll
            for (int fj = 0; fj < FM; ++fj)
                p[fi][fj] = u32x2{pack_bf16x2(acc[fi][fj][0], acc[fi][fj][1]),
                                  pack_bf16x2(acc[fi][fj][2], acc[fi][fj][3])};
#pragma unroll
        for (int fj = 0; fj < FM; ++fj) {
            const int64_t m = m_base + 16 * fj + (lane & 15);
#pragma unroll
            for (int fi = 0; fi < FN; ++fi) {
                const int64_t n = n_base + 16 * fi + 4 * (lane >> 4);
                uint16_t* row = static_cast<uint16_t*>(Cp) + m * ldc;
                if (full) {
                    *reinterpret_cast<u32x2*>(row + n) = p[fi][fj];
                } else if (m < M) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            row[n + r] = static_cast<uint16_t>(p[fi][fj][r >> 1] >> (16 * (r & 1)));
                }
            }
        }
    }
}

}  // namespace tmm

namespace tmm {

// One fragment row of store_acc: the four consecutive outputs (m, n .. n + 3) of one lane.
// `full`: the whole fragment lies inside M x N and C takes vector stores.
template <int OUT>
__device__ __forceinline__ void store_frag(void* Cp, int64_t ldc, int64_t M, int64_t N, int64_t m, int64_t n,
                                           f32x4 v, bool full) {
    if constexpr (OUT == OUT_F32) {
        float* row = static_cast<float*>(Cp) + m * ldc;
        if (full) {
            *reinterpret_cast<f32x4*>(row + n) = v;
        } else if (m < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) row[n + r] = v[r];
        }
    } else {
        uint16_t* row = static_cast<uint16_t*>(Cp) + m * ldc;
        const u32x2 p = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        if (full) {
            *reinterpret_cast<u32x2*>(row + n) = p;
        } else if (m < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) row[n + r] = static_cast<uint16_t>(p[r >> 1] >> (16 * (r & 1)));
        }
    }
}

// As store_acc, for v_mfma_f32_32x32x16_bf16 accumulators: fragment [fi][fj] holds
// D[n][m] = C[m][n] for a 32 (n) x 32 (m) block; lane l, register r carries
//     m = m_base + 32*fj + (l % 32),   n = n_base + 32*fi + 8*(r / 4) + 4*(l / 32) + (r % 4),
// so registers 4q .. 4q+3 are four consecutive n of one C row.
template <int OUT, int FN, int FM>
__device__ __forceinline__ void store_acc32(void* Cp, int64_t ldc, int64_t M, int64_t N,
                                            int64_t m_base, int64_t n_base,
                                            const f32x16 (&acc)[FN][FM], bool vec_ok) {
    const int lane = lane_id();
    const bool full = vec_ok && (m_base + 32 * FM <= M) && (n_base + 32 * FN <= N);
#pragma unroll
    for (int fj = 0; fj < FM; ++fj) {
        const int64_t m = m_base + 32 * fj + (lane & 31);
#pragma unroll
        for (int fi = 0; fi < FN; ++fi) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n_base + 32 * fi + 8 * q + 4 * (lane >> 5);
                const f32x4 v = {acc[fi][fj][4 * q], acc[fi][fj][4 * q + 1], acc[fi][fj][4 * q + 2],
                                 acc[fi][fj][4 * q + 3]};
                if constexpr (OUT == OUT_F32) {
                    float* row = static_cast<float*>(Cp) + m * ldc;
                    if (full) {
                        *reinterpret_cast<f32x4*>(row + n) = v;
                    } else if (m < M) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N) row[n + r] = v[r];
                    }
                } else {
                    uint16_t* row = static_cast<uint16_t*>(Cp) + m * ldc;
                    const u32x2 p = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    if (full) {
                        *reinterpret_cast<u32x2*>(row + n) = p;
                    } else if (m < M) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N) row[n + r] = static_cast<uint16_t>(p[r >> 1] >> (16 * (r & 1)));
                    }
                }
            }
        }
    }
}

}  // namespace tmm
