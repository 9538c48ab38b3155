// Host-side launchers of the kernel families, one per source file.  Each validates nothing
// (gemm_bf16.cpp does that) and returns the launch status.  Internal to libgemm_bf16.so.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace tmm {

// Kernel identifiers, reported by gemm_bf16_plan() and named by gemm_bf16_kernel_name().
enum KernelId {
    K_NONE = 0,
    K_ZERO_FILL = 1,        // K == 0: C = 0
    K_SIMPLE_64 = 2,        // ladder step 1: LDS-tiled, K loop, 2-D grid, fp32 VALU FMA
    K_MFMA_128 = 3,         // ladder step 3: MFMA register-blocked, one LDS stage, register loads
    K_PIPE_256 = 4,         // ladder step 2: direct-to-LDS ring, swizzle, 2-D grid, 256x256 tile
    K_PIPE_128 = 5,         //   same, 128x128 tile
    K_PERSIST_256 = 6,      // ladder step 4: persistent, XCD-aware grouped order, 256x256
    K_PERSIST_128 = 7,      //   same, 128x128
    K_SPEC_256 = 8,         // ladder step 5: wave-specialised, two consumer groups share B
    K_GEMV = 9,             // ladder step 6: skinny-M bandwidth path, MFMA form (M <= 16)
    K_GEMV_LDS = 10,        //   same, dot-product form: contiguous W rows, X staged in LDS
    K_PINGPONG_256 = 11,    // ladder steps 7-9: two wave groups alternate load and MFMA phases
    K_RING8_256 = 12,       // steps 4-6 with a five-slot 32-deep ring, loads spread over the K loop; 8 waves
    K_RING4_256 = 13,       //   same, 4 waves of 128 x 128 (AGPR accumulators)
    K_MX_RING_256 = 14,     // block-scaled 8-bit GEMM: the 4-wave ring with scaled MFMAs
    K_MX_SIMPLE_64 = 15,    //   general fallback (any K multiple of 32, pitch, alignment)
    K_ATTN_SIMPLE = 16,     // attention forward: one wave per query row (any d <= 256)
    K_ATTN_MFMA = 17,       //   MFMA tiles of queries x keys, online softmax (d = 64, 128)
    K_DTV_256 = 18,         // steps 4-6 with the A operand loaded straight into MFMA registers, B ring in LDS
    K_ATTN_PIPE = 19,       //   same, the next block's score MFMAs interleaved with this block's softmax
    K_ROLES = 20,           // step 7 with fixed roles: 4 load-only + 4 MFMA-only waves, 256 x 128 tile
    K_COUNT = 21
};

// Launch shape chosen for a problem (filled by the planner, consumed by the launchers).
struct Plan {
    int kernel = K_NONE;
    int vec = 1;            // global load width in elements for K_MFMA_128 (8, 4, 2 or 1)
    int vec_store = 0;      // C allows 16-byte (fp32) / 8-byte (bf16) stores
    TileGrid grid{};
    int grid_x = 0, grid_y = 0, grid_z = 0, block = 0;
};

hipError_t launch_zero_fill(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_simple(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_mfma(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_pipe(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_pingpong(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_ring(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_ring_streamk(const GemmArgs& g, int out, const Plan& p, int* ctr, float* part, int T_dp,
                               int T_sk, int G_sk, int L, hipStream_t s);
hipError_t launch_dtv(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_roles(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_splitk_reduce(const GemmArgs& g, int out, hipStream_t s);
hipError_t launch_gemv(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_mx(const MxArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_attention(const AttnArgs& g, int out, const Plan& p, hipStream_t s);
hipError_t launch_gemv_lds(const GemmArgs& g, int out, const Plan& p, hipStream_t s);
int gemv_lds_rows_per_workgroup();
int gemv_lds_threads();
int attn_rows_per_workgroup(int kernel, int d);

}  // namespace tmm
