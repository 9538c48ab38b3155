// The C ABI of libgemm_bf16.so (declared in include/gemm_bf16.h): argument validation, the
// planner that picks a kernel and launch shape, the gfx950 device check, and the launches.
// No device memory is allocated here or anywhere in the library.
#include <mutex>
#include <string.h>

#include "gemm_bf16.h"
#include "gemm_mx.h"
#include "attention.h"
#include "launch.hpp"
#include <math.h>

using namespace tmm;

namespace {

constexpr int kVersion = 10;
constexpr int kDefaultCUs = 256;        // MI355X
constexpr int64_t kMaxBatch = 65535;
constexpr int64_t k2G = int64_t(1) << 31;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --- device check ------------------------------------------------------------------------
struct DevInfo {
    bool known = false;
    bool ok = false;
    int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

// GEMM_OK and the CU count of the current device if it is a gfx950, else GEMM_ERR_ARCH.
int current_device(int* cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_ARCH;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DevInfo& d = g_dev[dev];
    if (!d.known) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_ARCH;
        d.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.cus = prop.multiProcessorCount;
        d.known = true;
    }
    if (!d.ok) return GEMM_ERR_ARCH;
    *cus = d.cus;
    return GEMM_OK;
}

// --- validation --------------------------------------------------------------------------
// la / lb: GEMM_LAYOUT_K_MAJOR (element (i, k) at i * ld + k: ld >= K) or
// GEMM_LAYOUT_MN_MAJOR (at k * ld + i: ld >= M for A, >= N for B).
int validate(int la, int lb, int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
             int64_t sA, const void* B, int64_t ldb, int64_t sB, const void* C, int64_t ldc,
             int64_t sC, int out) {
    if (out != GEMM_OUT_FP32 && out != GEMM_OUT_BF16) return GEMM_ERR_DTYPE;
    if ((la != GEMM_LAYOUT_K_MAJOR && la != GEMM_LAYOUT_MN_MAJOR) ||
        (lb != GEMM_LAYOUT_K_MAJOR && lb != GEMM_LAYOUT_MN_MAJOR))
        return GEMM_ERR_ARG;
    if (batch < 0 || batch > kMaxBatch || M < 0 || N < 0 || K < 0) return GEMM_ERR_ARG;
    const int64_t big = int64_t(1) << 40;   // keeps every index product inside int64
    if (M > big || N > big || K > big || lda > big || ldb > big || ldc > big) return GEMM_ERR_ARG;
    if (sA > big || sB > big || sC > big) return GEMM_ERR_ARG;
    const int64_t need_a = la == GEMM_LAYOUT_K_MAJOR ? K : M, need_b = lb == GEMM_LAYOUT_K_MAJOR ? K : N;
    if (lda < (need_a > 1 ? need_a : 1) || ldb < (need_b > 1 ? need_b : 1) || ldc < (N > 1 ? N : 1))
        return GEMM_ERR_ARG;
    if (sA < 0 || sB < 0 || sC < 0) return GEMM_ERR_ARG;
    if (batch == 0 || M == 0 || N == 0) return GEMM_OK;
    if (batch > 1 && sC < (M - 1) * ldc + N) return GEMM_ERR_ARG;
    // every tile id must fit in a 32-bit int (the smallest tile is 64 x 64)
    if (cdiv(M, 64) >= k2G || cdiv(N, 64) >= k2G) return GEMM_ERR_ARG;
    if (static_cast<__int128>(cdiv(M, 64)) * cdiv(N, 64) * batch >= k2G) return GEMM_ERR_ARG;
    if (C == nullptr) return GEMM_ERR_NULL;
    if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL;
    if (!aligned(A, 2) || !aligned(B, 2)) return GEMM_ERR_ARG;
    if (!aligned(C, out == GEMM_OUT_FP32 ? 4 : 2)) return GEMM_ERR_ARG;
    return GEMM_OK;
}

// --- planner -----------------------------------------------------------------------------
struct Shape {
    int64_t batch, M, N, K, lda, sA, ldb, sB, ldc, sC;
    const void *A, *B, *C;
    int out;
    int la = GEMM_LAYOUT_K_MAJOR, lb = GEMM_LAYOUT_K_MAJOR;
};

// The ping-pong kernel: 16-byte aligned rows, 16-byte chunks that never straddle K, 32-bit
// buffer offsets.
bool fast_loads_ok(const Shape& s, int rows) {
    if (!aligned(s.A, 16) || !aligned(s.B, 16)) return false;
    if (s.lda % 8 || s.ldb % 8 || s.K % 8) return false;
    if (s.batch > 1 && (s.sA % 8 || s.sB % 8)) return false;
    return int64_t(rows) * s.lda * 2 < k2G && int64_t(rows) * s.ldb * 2 < k2G;
}

// The pipelined kernels: the same 16-byte direct-to-LDS loads from rows that start on a
// 4-byte boundary (gfx950 serves unaligned buffer loads), with a ragged K tail added by
// one extra k step.
bool pipe_loads_ok(const Shape& s, int rows) {
    if (!aligned(s.A, 4) || !aligned(s.B, 4)) return false;
    if (s.lda % 2 || s.ldb % 2) return false;
    if (s.batch > 1 && (s.sA % 2 || s.sB % 2)) return false;
    return int64_t(rows) * s.lda * 2 < k2G && int64_t(rows) * s.ldb * 2 < k2G;
}

bool vec_store_ok(const Shape& s) {
    const uintptr_t a = s.out == GEMM_OUT_FP32 ? 16 : 8;
    return aligned(s.C, a) && s.ldc % 4 == 0 && (s.batch == 1 || s.sC % 4 == 0);
}

int widest_vec(const Shape& s) {
    for (int v = 8; v > 1; v /= 2) {
        if (aligned(s.A, 2 * v) && aligned(s.B, 2 * v) && s.lda % v == 0 && s.ldb % v == 0 &&
            s.K % v == 0 && (s.batch == 1 || (s.sA % v == 0 && s.sB % v == 0)))
            return v;
    }
    return 1;
}

void tile_grid(const Shape& s, int bm, int bn, Plan& p) {
    p.grid.tiles_m = static_cast<int>(cdiv(s.M, bm));
    p.grid.tiles_n = static_cast<int>(cdiv(s.N, bn));
    p.grid.total = static_cast<int>(p.grid.tiles_m * int64_t(p.grid.tiles_n) * s.batch);
    p.grid.group_m = 4;
}

// 2-D grid launches (tile column, tile row, batch item) of the generic kernels.
int plan_2d(const Shape& s, int kernel, int tile, Plan& p) {
    const int64_t tm = cdiv(s.M, tile), tn = cdiv(s.N, tile);
    if (tm > 65535 || tn >= k2G) return GEMM_ERR_UNSUPPORTED;
    p.kernel = kernel;
    p.grid_x = static_cast<int>(tn);
    p.grid_y = static_cast<int>(tm);
    p.grid_z = static_cast<int>(s.batch);
    p.block = 256;
    p.vec = widest_vec(s);
    p.vec_store = vec_store_ok(s);
    return GEMM_OK;
}

// Tile size of the pipelined kernels: 256 x 256 when that still gives most CUs a tile,
// otherwise 128 x 128.
bool use_big_tile(const Shape& s, int cus) {
    const int64_t big = cdiv(s.M, 256) * cdiv(s.N, 256) * s.batch;
    return big * 10 >= int64_t(cus) * 9;
}

int plan_pipe(const Shape& s, bool persistent, int cus, Plan& p) {
    const bool big = use_big_tile(s, cus);
    if (!pipe_loads_ok(s, big ? 256 : 128)) return GEMM_ERR_UNSUPPORTED;
    tile_grid(s, big ? 256 : 128, big ? 256 : 128, p);
    p.kernel = persistent ? (big ? K_PERSIST_256 : K_PERSIST_128) : (big ? K_PIPE_256 : K_PIPE_128);
    p.grid_x = persistent ? std::min(p.grid.total, cus) : p.grid.total;
    p.grid_y = p.grid_z = 1;
    p.block = 256;
    p.vec_store = vec_store_ok(s);
    return GEMM_OK;
}

// Eight waves, two consumer groups sharing the B tile; always 256 x 256 tiles, persistent.
// `kernel`: K_SPEC_256 (both groups load and multiply in lockstep) or K_PINGPONG_256 (the
// groups alternate load and MFMA phases).
int plan_spec(const Shape& s, int cus, Plan& p, int kernel = K_SPEC_256) {
    const bool kmajor = s.la == GEMM_LAYOUT_K_MAJOR && s.lb == GEMM_LAYOUT_K_MAJOR;
    if (kmajor && (kernel == K_PINGPONG_256 ? !fast_loads_ok(s, 256) : !pipe_loads_ok(s, 256)))
        return GEMM_ERR_UNSUPPORTED;
    tile_grid(s, 256, 256, p);
    p.kernel = kernel;
    p.grid_x = std::min(p.grid.total, cus);
    p.grid_y = p.grid_z = 1;
    p.block = kernel == K_RING4_256 ? 256 : 512;
    p.vec_store = vec_store_ok(s);
    return GEMM_OK;
}

// A in registers, B in an LDS ring: both operands K-major with 16-byte loads (the A
// fragments are 16-byte buffer loads into registers), 256 x 256 tiles, persistent.
int plan_dtv(const Shape& s, int cus, Plan& p) {
    if (s.la != GEMM_LAYOUT_K_MAJOR || s.lb != GEMM_LAYOUT_K_MAJOR || !fast_loads_ok(s, 256))
        return GEMM_ERR_UNSUPPORTED;
    tile_grid(s, 256, 256, p);
    p.kernel = K_DTV_256;
    p.grid_x = std::min(p.grid.total, cus);
    p.grid_y = p.grid_z = 1;
    p.block = 256;
    p.vec_store = vec_store_ok(s);
    return GEMM_OK;
}

// Fixed producer and consumer waves: K-major operands with the pipelined kernels' loads, K a
// multiple of 8, 256 x 128 tiles, persistent.
int plan_roles(const Shape& s, int cus, Plan& p) {
    if (s.la != GEMM_LAYOUT_K_MAJOR || s.lb != GEMM_LAYOUT_K_MAJOR || s.K % 8 || !pipe_loads_ok(s, 256))
        return GEMM_ERR_UNSUPPORTED;
    tile_grid(s, 256, 128, p);
    p.kernel = K_ROLES;
    p.grid_x = std::min(p.grid.total, cus);
    p.grid_y = p.grid_z = 1;
    p.block = 512;
    p.vec_store = vec_store_ok(s);
    return GEMM_OK;
}

bool gemv_ok(const Shape& s) {
    if (s.M > 16 || s.batch != 1) return false;
    if (!aligned(s.A, 16) || !aligned(s.B, 16) || s.lda % 8 || s.ldb % 8 || s.K % 8) return false;
    return 16 * s.lda * 2 < k2G && 16 * s.ldb * 2 < k2G && cdiv(s.N, 16) < k2G;
}

// Largest M that takes the dot-product form of the skinny-M path (above it, up to 16: the
// MFMA form).  Measured on MI355X at N = K = 4096: the dot form is faster up to M = 4
// (6.8 us at M = 1), the MFMA form from M = 8 (9.9 us at M = 8 and at M = 16).
#ifndef TMM_GEMV_DOT_MAX_M
#define TMM_GEMV_DOT_MAX_M 4
#endif

int plan_gemv(const Shape& s, Plan& p) {
    if (!gemv_ok(s)) return GEMM_ERR_UNSUPPORTED;
    if (s.M <= TMM_GEMV_DOT_MAX_M) {
        p.kernel = K_GEMV_LDS;
        p.grid_x = static_cast<int>(cdiv(s.N, gemv_lds_rows_per_workgroup()));
        p.block = gemv_lds_threads();
    } else {
        p.kernel = K_GEMV;
        p.grid_x = static_cast<int>(cdiv(s.N, 16));
        p.block = 512;
    }
    p.grid_y = p.grid_z = 1;
    return GEMM_OK;
}

// The ring kernel with MN-major operands: 4-byte aligned rows with even pitches (as for the
// K-major kernels), an MN-major operand's extent (M or N) a multiple of 8 (whole 16-byte
// chunks) and all of its rows within 32-bit buffer offsets.
bool ring_layout_ok(const Shape& s) {
    if (!aligned(s.A, 4) || !aligned(s.B, 4) || s.lda % 2 || s.ldb % 2) return false;
    if (s.batch > 1 && (s.sA % 2 || s.sB % 2)) return false;
    auto op_ok = [&](int lay, int64_t ld, int64_t ext) {
        if (lay == GEMM_LAYOUT_K_MAJOR) return 256 * ld * 2 < k2G;
        return ext % 8 == 0 && ((s.K - 1) * ld + ext) * 2 < k2G;
    };
    return op_ok(s.la, s.lda, s.M) && op_ok(s.lb, s.ldb, s.N);
}

// MN-major operands: AUTO takes the ring kernel (4 waves) where its preconditions hold and
// the simple kernel otherwise; of the forced variants only those two take such operands.
int plan_layout(int variant, const Shape& s, int cus, Plan& p) {
    switch (variant) {
        case GEMM_VARIANT_SIMPLE: return plan_2d(s, K_SIMPLE_64, 64, p);
        case GEMM_VARIANT_RING4:
            return ring_layout_ok(s) ? plan_spec(s, cus, p, K_RING4_256) : GEMM_ERR_UNSUPPORTED;
        case GEMM_VARIANT_AUTO:
            if (ring_layout_ok(s) && plan_spec(s, cus, p, K_RING4_256) == GEMM_OK) return GEMM_OK;
            return plan_2d(s, K_SIMPLE_64, 64, p) == GEMM_OK ? GEMM_OK : GEMM_ERR_ARG;
        default: return GEMM_ERR_UNSUPPORTED;
    }
}

int make_plan(int variant, const Shape& s, int cus, Plan& p) {
    if (variant < GEMM_VARIANT_AUTO || variant > GEMM_VARIANT_ROLES) return GEMM_ERR_ARG;
    p = Plan{};
    if (s.batch == 0 || s.M == 0 || s.N == 0) {
        p.kernel = K_NONE;
        return GEMM_OK;
    }
    if (s.K == 0) {  // every variant: the empty sum
        p.kernel = K_ZERO_FILL;
        p.grid_x = static_cast<int>(std::min<int64_t>(cdiv(s.M * s.N * s.batch, 256), 65536));
        p.grid_y = p.grid_z = 1;
        p.block = 256;
        return GEMM_OK;
    }
    if (s.la != GEMM_LAYOUT_K_MAJOR || s.lb != GEMM_LAYOUT_K_MAJOR) return plan_layout(variant, s, cus, p);
    switch (variant) {
        case GEMM_VARIANT_SIMPLE: return plan_2d(s, K_SIMPLE_64, 64, p);
        case GEMM_VARIANT_MFMA: return plan_2d(s, K_MFMA_128, 128, p);
        case GEMM_VARIANT_PIPELINED: return plan_pipe(s, false, cus, p);
        case GEMM_VARIANT_PERSISTENT: return plan_pipe(s, true, cus, p);
        case GEMM_VARIANT_SPECIALIZED: return plan_spec(s, cus, p);
        case GEMM_VARIANT_GEMV: return plan_gemv(s, p);
        case GEMM_VARIANT_PINGPONG: return plan_spec(s, cus, p, K_PINGPONG_256);
        case GEMM_VARIANT_RING8: return plan_spec(s, cus, p, K_RING8_256);
        case GEMM_VARIANT_RING4: return plan_spec(s, cus, p, K_RING4_256);
        case GEMM_VARIANT_DTV: return plan_dtv(s, cus, p);
        case GEMM_VARIANT_ROLES: return plan_roles(s, cus, p);
        default: break;
    }
    // AUTO
    if (gemv_ok(s)) return plan_gemv(s, p);
    if (use_big_tile(s, cus) && plan_spec(s, cus, p, K_RING4_256) == GEMM_OK) return GEMM_OK;
    if (plan_pipe(s, true, cus, p) == GEMM_OK) return GEMM_OK;
    int rc = plan_2d(s, K_MFMA_128, 128, p);
    if (rc == GEMM_OK) return rc;
    return GEMM_ERR_ARG;  // no kernel can take this shape (tile grid beyond launch limits)
}

int run(int variant, const Shape& s, void* stream) {
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    if (variant < GEMM_VARIANT_AUTO || variant > GEMM_VARIANT_ROLES) return GEMM_ERR_ARG;
    if (s.batch == 0 || s.M == 0 || s.N == 0) return GEMM_OK;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != GEMM_OK) return rc;
    Plan p;
    rc = make_plan(variant, s, cus, p);
    if (rc != GEMM_OK) return rc;
    GemmArgs g{s.batch, s.M, s.N, s.K,
               static_cast<const uint16_t*>(s.A), s.lda, s.sA,
               static_cast<const uint16_t*>(s.B), s.ldb, s.sB,
               const_cast<void*>(s.C), s.ldc, s.sC, s.la, s.lb};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    switch (p.kernel) {
        case K_NONE: return GEMM_OK;
        case K_ZERO_FILL: e = launch_zero_fill(g, s.out, p, st); break;
        case K_SIMPLE_64: e = launch_simple(g, s.out, p, st); break;
        case K_MFMA_128: e = launch_mfma(g, s.out, p, st); break;
        case K_PIPE_256:
        case K_PIPE_128:
        case K_PERSIST_256:
        case K_PERSIST_128:
        case K_SPEC_256: e = launch_pipe(g, s.out, p, st); break;
        case K_PINGPONG_256: e = launch_pingpong(g, s.out, p, st); break;
        case K_RING8_256:
        case K_RING4_256: e = launch_ring(g, s.out, p, st); break;
        case K_DTV_256: e = launch_dtv(g, s.out, p, st); break;
        case K_ROLES: e = launch_roles(g, s.out, p, st); break;
        case K_GEMV: e = launch_gemv(g, s.out, p, st); break;
        case K_GEMV_LDS: e = launch_gemv_lds(g, s.out, p, st); break;
        default: return GEMM_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// --- split K --------------------------------------------------------------------------
// Number of K ranges for gemm_bf16_splitk: `splits` if > 0 (capped at the K blocks of 64),
// else (auto, `auto_tiles` = tiles of the kernel the planner would run without splitting):
// one range when those tiles keep at least half the CUs busy, else the most ranges of at
// least 8 K blocks that fill the CUs with 256 x 256 tiles and fit in the workspace.
int choose_splits(const Shape& s, int splits, int64_t ws_bytes, int cus, int64_t auto_tiles) {
    const int64_t nk = cdiv(s.K, 64);
    const int64_t per = s.batch * s.M * s.N * 4;   // workspace bytes per range
    const int64_t tiles = cdiv(s.M, 256) * cdiv(s.N, 256) * s.batch;
    int64_t S;
    if (splits > 0) {
        S = std::min<int64_t>(splits, nk);
    } else {
        if (auto_tiles * 2 > cus) return 1;
        S = std::min<int64_t>(cus / tiles, nk / 8);
        S = std::min<int64_t>(S, ws_bytes / per);
    }
    S = std::min<int64_t>(S, 256);
    if (tiles * S >= k2G) S = k2G / tiles - 1;
    return static_cast<int>(std::max<int64_t>(S, 1));
}

// Plan of gemm_bf16_splitk: *S = ranges (1: an ordinary gemm_bf16_layout call with AUTO).
int plan_splitk(const Shape& s, int splits, const void* ws, int64_t ws_bytes, int cus, int* S, Plan& p) {
    if (splits < 0 || ws_bytes < 0) return GEMM_ERR_ARG;
    *S = 1;
    if (s.batch == 0 || s.M == 0 || s.N == 0 || s.K == 0) return make_plan(GEMM_VARIANT_AUTO, s, cus, p);
    int64_t auto_tiles = 0;
    if (splits == 0) {   // only where the library would run a tiled MFMA kernel anyway
        int rc = make_plan(GEMM_VARIANT_AUTO, s, cus, p);
        if (rc != GEMM_OK) return rc;
        if (p.kernel != K_RING4_256 && p.kernel != K_PERSIST_128 && p.kernel != K_PERSIST_256) return GEMM_OK;
        auto_tiles = p.grid.total;
    }
    const int want = choose_splits(s, splits, ws_bytes, cus, auto_tiles);
    if (want > 1 && !ring_layout_ok(s)) {   // the ring kernel's own preconditions
        if (splits > 1) return GEMM_ERR_UNSUPPORTED;
        return make_plan(GEMM_VARIANT_AUTO, s, cus, p);
    }
    if (want <= 1) return make_plan(GEMM_VARIANT_AUTO, s, cus, p);
    if (ws == nullptr) return GEMM_ERR_NULL;
    if (!aligned(ws, 16) || ws_bytes < int64_t(want) * s.batch * s.M * s.N * 4) return GEMM_ERR_ARG;
    int rc = plan_spec(s, cus, p, K_RING4_256);
    if (rc != GEMM_OK) return rc;
    p.grid_x = static_cast<int>(std::min<int64_t>(int64_t(p.grid.total) * want, cus));
    *S = want;
    return GEMM_OK;
}

int run_splitk(const Shape& s, int splits, void* ws, int64_t ws_bytes, void* stream) {
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    if (s.batch == 0 || s.M == 0 || s.N == 0) return GEMM_OK;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != GEMM_OK) return rc;
    Plan p;
    int S = 1;
    rc = plan_splitk(s, splits, ws, ws_bytes, cus, &S, p);
    if (rc != GEMM_OK) return rc;
    if (S == 1) return run(GEMM_VARIANT_AUTO, s, stream);
    GemmArgs g{s.batch, s.M, s.N, s.K,
               static_cast<const uint16_t*>(s.A), s.lda, s.sA,
               static_cast<const uint16_t*>(s.B), s.ldb, s.sB,
               const_cast<void*>(s.C), s.ldc, s.sC, s.la, s.lb,
               static_cast<float*>(ws), S};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_ring(g, s.out, p, st);
    if (e == hipSuccess) e = launch_splitk_reduce(g, s.out, st);
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// --- split K without a workspace argument ----------------------------------------------
// The fp32 partials of gemm_bf16_splitk_noalloc live here: GEMM_SCRATCH_BYTES per device, in
// the code object's device memory.  Host code never passes `scratch` itself to a kernel (in
// host code the name is a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and kept.
__device__ __align__(256) float scratch[GEMM_SCRATCH_BYTES / 4];

std::mutex g_scratch_mu;
void* g_scratch[64];

void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

int run_splitk_noalloc(const Shape& s, int splits, void* stream) {
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    if (splits < 0) return GEMM_ERR_ARG;
    if (s.batch == 0 || s.M == 0 || s.N == 0) return GEMM_OK;
    if (splits > 0 && s.K > 0) {   // an explicit count must fit (S capped at the K blocks)
        const __int128 S = std::min<int64_t>(splits, cdiv(s.K, 64));
        if (S > 1 && S * s.batch * s.M * s.N * 4 > GEMM_SCRATCH_BYTES) return GEMM_ERR_SCRATCH;
    }
    int cus = 0;
    rc = current_device(&cus);
    if (rc != GEMM_OK) return rc;
    void* ws = scratch_on_current_device();
    if (ws == nullptr) return GEMM_ERR_LAUNCH;
    return run_splitk(s, splits, ws, GEMM_SCRATCH_BYTES, stream);
}

// --- stream-K with atomic work claiming ---------------------------------------------------
struct SkPlan {
    int T_dp = 0, T_sk = 0, G_sk = 0, grid = 0, L = 1;
    int64_t ctr_ints = 0, part_bytes = 0, ws_bytes = 0;
};

constexpr int kSkMinBlocks = 4;            // K blocks per stream-K slot, at least
// The counters sit in the first kSkCtrBytes of the workspace whatever the call, and the partials
// after them, so that no call's partials land on another call's counters.
constexpr int64_t kSkCtrBytes = 16384;
constexpr int64_t kSkMaxIters = 1 << 22;   // stream-K iterations (the slot arithmetic's range)

// Work of gemm_bf16_streamk on `cus` compute units: 256 x 256 tiles of the 4-wave ring kernel;
// the last T_sk tiles as stream-K slots, the others whole (see gemm_ring.hip).
int plan_streamk(int mode, const Shape& s, int cus, SkPlan& sp, Plan& p) {
    if (mode < GEMM_STREAMK_AUTO || mode > GEMM_STREAMK_ALL) return GEMM_ERR_ARG;
    if (s.la != GEMM_LAYOUT_K_MAJOR || s.lb != GEMM_LAYOUT_K_MAJOR || !ring_layout_ok(s)) return GEMM_ERR_UNSUPPORTED;
    int rc = plan_spec(s, cus, p, K_RING4_256);
    if (rc != GEMM_OK) return rc;
    const int64_t T = p.grid.total, nk = cdiv(s.K, 64);
    int64_t T_sk = 0;
    if (mode != GEMM_STREAMK_DP) {
        // the last partly filled wave together with the full wave before it (so that every
        // slot holds more than one tile's K blocks and each cut tile has few pieces)
        if (T > cus && T % cus != 0) T_sk = cus + T % cus;
        else if (T < cus && mode == GEMM_STREAMK_ALL) T_sk = T;      // every tile
    }
    if (T_sk * nk >= kSkMaxIters) T_sk = 0;
    sp = SkPlan{};
    sp.T_sk = static_cast<int>(T_sk);
    sp.T_dp = static_cast<int>(T - T_sk);
    if (T_sk > 0) {
        const int64_t I = T_sk * nk;
        const int64_t G = std::min<int64_t>(cus, std::max<int64_t>(1, I / kSkMinBlocks));
        const int64_t L = cdiv(I, G);
        sp.L = static_cast<int>(L);
        sp.G_sk = static_cast<int>(cdiv(I, L));   // every slot starts below I
    }
    const int64_t units = sp.T_dp + sp.G_sk;
    sp.grid = static_cast<int>(std::min<int64_t>(units, cus));
    sp.ctr_ints = 2 + sp.grid + 4 * T_sk;   // T_sk < 2 cus
    if (sp.ctr_ints * 4 > kSkCtrBytes) return GEMM_ERR_UNSUPPORTED;   // beyond 800 compute units
    sp.part_bytes = int64_t(sp.G_sk) * 2 * 256 * 256 * 4;
    sp.ws_bytes = kSkCtrBytes + sp.part_bytes;
    p.grid_x = sp.grid;
    return GEMM_OK;
}

int run_streamk(int mode, const Shape& s, void* ws, int64_t ws_bytes, void* stream) {
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    if (mode < GEMM_STREAMK_AUTO || mode > GEMM_STREAMK_ALL || ws_bytes < 0) return GEMM_ERR_ARG;
    if (s.batch == 0 || s.M == 0 || s.N == 0) return GEMM_OK;
    if (s.K == 0) return run(GEMM_VARIANT_AUTO, s, stream);
    int cus = 0;
    rc = current_device(&cus);
    if (rc != GEMM_OK) return rc;
    Plan p;
    SkPlan sp;
    rc = plan_streamk(mode, s, cus, sp, p);
    if (rc != GEMM_OK) return rc;
    if (ws == nullptr) return GEMM_ERR_NULL;
    if (!aligned(ws, 256) || ws_bytes < sp.ws_bytes) return GEMM_ERR_ARG;
    GemmArgs g{s.batch, s.M, s.N, s.K,
               static_cast<const uint16_t*>(s.A), s.lda, s.sA,
               static_cast<const uint16_t*>(s.B), s.ldb, s.sB,
               const_cast<void*>(s.C), s.ldc, s.sC, s.la, s.lb};
    int* ctr = static_cast<int*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + kSkCtrBytes);
    hipError_t e = launch_ring_streamk(g, s.out, p, ctr, part, sp.T_dp, sp.T_sk, sp.G_sk, sp.L,
                                       static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

Shape shape(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int64_t sA,
            const void* B, int64_t ldb, int64_t sB, const void* C, int64_t ldc, int64_t sC, int out,
            int la = GEMM_LAYOUT_K_MAJOR, int lb = GEMM_LAYOUT_K_MAJOR) {
    return Shape{batch, M, N, K, lda, sA, ldb, sB, ldc, sC, A, B, C, out, la, lb};
}

int plan_into(int variant, const Shape& s, int num_cus, int* kernel_id, int64_t* grid_x, int* block) {
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    if (variant < GEMM_VARIANT_AUTO || variant > GEMM_VARIANT_ROLES) return GEMM_ERR_ARG;
    Plan p;
    rc = make_plan(variant, s, num_cus > 0 ? num_cus : kDefaultCUs, p);
    if (rc != GEMM_OK) return rc;
    if (kernel_id) *kernel_id = p.kernel;
    if (grid_x) *grid_x = int64_t(p.grid_x) * (p.grid_y ? p.grid_y : 1) * (p.grid_z ? p.grid_z : 1);
    if (block) *block = p.block;
    return GEMM_OK;
}

// --- block-scaled 8-bit GEMM (gemm_mx) ------------------------------------------------------
struct MxShape {
    int fa, fb;
    int64_t M, N, K;
    const void *A, *SA, *B, *SB;
    int64_t lda, ldsa, ldb, ldsb;
    const void* C;
    int64_t ldc;
    int out;
};

int validate_mx(const MxShape& s) {
    if (s.out != GEMM_OUT_FP32 && s.out != GEMM_OUT_BF16) return GEMM_ERR_DTYPE;
    if ((s.fa != GEMM_MX_E4M3 && s.fa != GEMM_MX_E5M2) || (s.fb != GEMM_MX_E4M3 && s.fb != GEMM_MX_E5M2))
        return GEMM_ERR_ARG;
    if (s.M < 0 || s.N < 0 || s.K < 0 || s.K % 32) return GEMM_ERR_ARG;
    const int64_t kb = std::max<int64_t>(s.K / 32, 1);
    if (s.lda < std::max<int64_t>(s.K, 1) || s.ldb < std::max<int64_t>(s.K, 1) || s.ldsa < kb || s.ldsb < kb ||
        s.ldc < std::max<int64_t>(s.N, 1))
        return GEMM_ERR_ARG;
    if (cdiv(s.M, 64) > 65535 || cdiv(s.N, 64) >= k2G) return GEMM_ERR_ARG;
    if (static_cast<__int128>(s.M) * s.lda >= (int64_t(1) << 62) ||
        static_cast<__int128>(s.N) * s.ldb >= (int64_t(1) << 62))
        return GEMM_ERR_ARG;
    if (s.M > 0 && s.N > 0 && s.C == nullptr) return GEMM_ERR_NULL;
    if (s.K > 0 && s.M > 0 && s.N > 0 &&
        (s.A == nullptr || s.SA == nullptr || s.B == nullptr || s.SB == nullptr))
        return GEMM_ERR_NULL;
    return GEMM_OK;
}

// Preconditions of the scaled-MFMA ring kernel: whole 128-deep blocks, 4-byte aligned rows of
// the operands (16-byte direct-to-LDS loads) and of the scales (dword loads), tile extents
// addressable by 32-bit buffer offsets.
bool mx_ring_ok(const MxShape& s) {
    if (s.K % 128) return false;
    if (!aligned(s.A, 4) || !aligned(s.B, 4) || !aligned(s.SA, 4) || !aligned(s.SB, 4)) return false;
    if (s.lda % 4 || s.ldb % 4 || s.ldsa % 4 || s.ldsb % 4) return false;
    return 256 * s.lda < k2G && 256 * s.ldb < k2G && 256 * s.ldsa < k2G && 256 * s.ldsb < k2G;
}

int plan_mx(int variant, const MxShape& s, int cus, Plan& p) {
    if (variant < GEMM_MX_VARIANT_AUTO || variant > GEMM_MX_VARIANT_RING) return GEMM_ERR_ARG;
    p = Plan{};
    if (s.M == 0 || s.N == 0) {
        p.kernel = K_NONE;
        return GEMM_OK;
    }
    if (s.K == 0) {
        p.kernel = K_ZERO_FILL;
        p.grid_x = static_cast<int>(std::min<int64_t>(cdiv(s.M * s.N, 256), 65536));
        p.grid_y = p.grid_z = 1;
        p.block = 256;
        return GEMM_OK;
    }
    const bool ring = mx_ring_ok(s);
    if (variant == GEMM_MX_VARIANT_RING && !ring) return GEMM_ERR_UNSUPPORTED;
    if (ring && variant != GEMM_MX_VARIANT_SIMPLE) {
        p.kernel = K_MX_RING_256;
        p.grid.tiles_m = static_cast<int>(cdiv(s.M, 256));
        p.grid.tiles_n = static_cast<int>(cdiv(s.N, 256));
        if (int64_t(p.grid.tiles_m) * p.grid.tiles_n >= k2G) return GEMM_ERR_UNSUPPORTED;
        p.grid.total = p.grid.tiles_m * p.grid.tiles_n;
        p.grid.group_m = 4;
        p.grid_x = std::min(p.grid.total, cus);
        p.grid_y = p.grid_z = 1;
        p.block = 256;
        const uintptr_t ca = s.out == GEMM_OUT_FP32 ? 16 : 8;
        p.vec_store = aligned(s.C, ca) && s.ldc % 4 == 0;
        return GEMM_OK;
    }
    p.kernel = K_MX_SIMPLE_64;
    p.grid_x = static_cast<int>(cdiv(s.N, 64));
    p.grid_y = static_cast<int>(cdiv(s.M, 64));
    p.grid_z = 1;
    p.block = 256;
    return GEMM_OK;
}

int run_mx(int variant, const MxShape& s, void* stream) {
    int rc = validate_mx(s);
    if (rc != GEMM_OK) return rc;
    if (s.M == 0 || s.N == 0) return GEMM_OK;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != GEMM_OK) return rc;
    Plan p;
    rc = plan_mx(variant, s, cus, p);
    if (rc != GEMM_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (p.kernel == K_ZERO_FILL) {
        GemmArgs g{1, s.M, s.N, 0, nullptr, 0, 0, nullptr, 0, 0, const_cast<void*>(s.C), s.ldc, 0};
        e = launch_zero_fill(g, s.out, p, st);
    } else {
        MxArgs g{s.M, s.N, s.K,
                 static_cast<const uint8_t*>(s.A), s.lda, static_cast<const uint8_t*>(s.SA), s.ldsa,
                 static_cast<const uint8_t*>(s.B), s.ldb, static_cast<const uint8_t*>(s.SB), s.ldsb,
                 const_cast<void*>(s.C), s.ldc, s.fa, s.fb};
        e = launch_mx(g, s.out, p, st);
    }
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// --- attention forward (attention_fwd) ---------------------------------------------------
struct AttnShape {
    int64_t B, Hq, Hkv, Lq, Lk, d;
    const void *Q, *K, *V, *O;
    float scale;
    int causal, out;
};

int validate_attn(const AttnShape& s) {
    if (s.out != GEMM_OUT_FP32 && s.out != GEMM_OUT_BF16) return GEMM_ERR_DTYPE;
    if (s.B < 1 || s.B > 65535 || s.Hq < 1 || s.Hq > 65535 || s.Hkv < 1 || s.Hq % s.Hkv) return GEMM_ERR_ARG;
    if (s.Lq < 0 || s.Lk < 0 || s.d < 8 || s.d > 256 || s.d % 8) return GEMM_ERR_ARG;
    if (s.causal != 0 && s.causal != 1) return GEMM_ERR_ARG;
    if (!std::isfinite(s.scale)) return GEMM_ERR_ARG;
    // every element index fits comfortably in int64 and the query blocks in a grid dimension
    if (static_cast<__int128>(s.B) * s.Hq * std::max<int64_t>(s.Lq, s.Lk) * s.d >= (int64_t(1) << 62)) return GEMM_ERR_ARG;
    if (cdiv(s.Lq, 4) >= k2G) return GEMM_ERR_ARG;
    if (s.Lq > 0 && (s.Q == nullptr || s.O == nullptr)) return GEMM_ERR_NULL;
    if (s.Lq > 0 && s.Lk > 0 && (s.K == nullptr || s.V == nullptr)) return GEMM_ERR_NULL;
    return GEMM_OK;
}

// The MFMA kernel: head dimension 64 or 128; Q, K, V, O 16-byte aligned (16-byte loads of
// Q rows and of K and V rows into LDS, vector stores of O).
bool attn_mfma_ok(const AttnShape& s) {
    if (s.d != 64 && s.d != 128) return false;
    if (!(s.scale > 0.f)) return false;   // the kernel scales the row maximum once
    if (!aligned(s.Q, 16) || !aligned(s.K, 16) || !aligned(s.V, 16) || !aligned(s.O, 16)) return false;
    return s.Lk * s.d * 2 < k2G && cdiv(s.Lq, 128) < k2G;
}

// AUTO's choice between the two MFMA attention kernels (1: attn_pipe, 0: attn_mfma).
#ifndef TMM_ATTN_AUTO_PIPE
#define TMM_ATTN_AUTO_PIPE 0
#endif

int plan_attn(int variant, const AttnShape& s, int cus, Plan& p) {
    (void)cus;
    if (variant < ATTN_VARIANT_AUTO || variant > ATTN_VARIANT_PIPE) return GEMM_ERR_ARG;
    p = Plan{};
    if (s.Lq == 0) {
        p.kernel = K_NONE;
        return GEMM_OK;
    }
    const bool mfma = attn_mfma_ok(s);
    if ((variant == ATTN_VARIANT_MFMA || variant == ATTN_VARIANT_PIPE) && !mfma) return GEMM_ERR_UNSUPPORTED;
    if (mfma && variant != ATTN_VARIANT_SIMPLE) {
        p.kernel = variant == ATTN_VARIANT_PIPE || (variant == ATTN_VARIANT_AUTO && TMM_ATTN_AUTO_PIPE)
                       ? K_ATTN_PIPE
                       : K_ATTN_MFMA;
        p.grid_x = static_cast<int>(cdiv(s.Lq, attn_rows_per_workgroup(p.kernel, static_cast<int>(s.d))));
        p.grid_y = static_cast<int>(s.Hq);
        p.grid_z = static_cast<int>(s.B);
        p.block = 256;
        return GEMM_OK;
    }
    p.kernel = K_ATTN_SIMPLE;
    p.grid_x = static_cast<int>(cdiv(s.Lq, 4));
    p.grid_y = static_cast<int>(s.Hq);
    p.grid_z = static_cast<int>(s.B);
    p.block = 256;
    return GEMM_OK;
}

int run_attn(int variant, const AttnShape& s, float* lse, void* stream) {
    int rc = validate_attn(s);
    if (rc != GEMM_OK) return rc;
    if (s.Lq == 0) return GEMM_OK;
    int cus = 0;
    rc = current_device(&cus);
    if (rc != GEMM_OK) return rc;
    Plan p;
    rc = plan_attn(variant, s, cus, p);
    if (rc != GEMM_OK) return rc;
    AttnArgs g{s.B, s.Hq, s.Hkv, s.Lq, s.Lk, s.d,
               static_cast<const uint16_t*>(s.Q), static_cast<const uint16_t*>(s.K),
               static_cast<const uint16_t*>(s.V), const_cast<void*>(s.O), lse, s.scale, s.causal};
    hipError_t e = launch_attention(g, s.out, p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
              int64_t ldb, void* C, int64_t ldc, int out_dtype, void* stream) {
    return run(GEMM_VARIANT_AUTO, shape(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, out_dtype), stream);
}

int gemm_bf16_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A,
                              int64_t lda, int64_t strideA, const void* B, int64_t ldb,
                              int64_t strideB, void* C, int64_t ldc, int64_t strideC,
                              int out_dtype, void* stream) {
    return run(GEMM_VARIANT_AUTO,
               shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype), stream);
}

int gemm_bf16_variant(int variant, int64_t batch, int64_t M, int64_t N, int64_t K, const void* A,
                      int64_t lda, int64_t strideA, const void* B, int64_t ldb, int64_t strideB,
                      void* C, int64_t ldc, int64_t strideC, int out_dtype, void* stream) {
    return run(variant, shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype),
               stream);
}

int gemm_bf16_validate(int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       int64_t strideA, const void* B, int64_t ldb, int64_t strideB, const void* C,
                       int64_t ldc, int64_t strideC, int out_dtype) {
    return validate(GEMM_LAYOUT_K_MAJOR, GEMM_LAYOUT_K_MAJOR, batch, M, N, K, A, lda, strideA, B, ldb, strideB,
                    C, ldc, strideC, out_dtype);
}

int gemm_bf16_plan(int variant, int64_t batch, int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, int64_t strideA, const void* B, int64_t ldb, int64_t strideB,
                   const void* C, int64_t ldc, int64_t strideC, int out_dtype, int num_cus,
                   int* kernel_id, int64_t* grid_x, int* block) {
    return plan_into(variant, shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype),
                     num_cus, kernel_id, grid_x, block);
}

int gemm_bf16_layout(int a_layout, int b_layout, int variant, int64_t batch, int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb, int64_t strideB,
                     void* C, int64_t ldc, int64_t strideC, int out_dtype, void* stream) {
    return run(variant,
               shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype, a_layout, b_layout),
               stream);
}

int gemm_bf16_layout_validate(int a_layout, int b_layout, int64_t batch, int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb,
                              int64_t strideB, const void* C, int64_t ldc, int64_t strideC, int out_dtype) {
    return validate(a_layout, b_layout, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                    out_dtype);
}

int gemm_bf16_layout_plan(int a_layout, int b_layout, int variant, int64_t batch, int64_t M, int64_t N,
                          int64_t K, const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb,
                          int64_t strideB, const void* C, int64_t ldc, int64_t strideC, int out_dtype,
                          int num_cus, int* kernel_id, int64_t* grid_x, int* block) {
    return plan_into(variant,
                     shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype, a_layout,
                           b_layout),
                     num_cus, kernel_id, grid_x, block);
}

int gemm_bf16_splitk(int a_layout, int b_layout, int splits, int64_t batch, int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb, int64_t strideB,
                     void* C, int64_t ldc, int64_t strideC, int out_dtype, void* workspace,
                     int64_t workspace_bytes, void* stream) {
    return run_splitk(
        shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype, a_layout, b_layout),
        splits, workspace, workspace_bytes, stream);
}

int gemm_bf16_splitk_noalloc(int a_layout, int b_layout, int splits, int64_t batch, int64_t M, int64_t N,
                             int64_t K, const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb,
                             int64_t strideB, void* C, int64_t ldc, int64_t strideC, int out_dtype, void* stream) {
    return run_splitk_noalloc(
        shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype, a_layout, b_layout),
        splits, stream);
}

int gemm_bf16_streamk(int mode, int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                      int64_t strideA, const void* B, int64_t ldb, int64_t strideB, void* C, int64_t ldc,
                      int64_t strideC, int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    return run_streamk(mode, shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype),
                       workspace, workspace_bytes, stream);
}

int gemm_bf16_streamk_plan(int mode, int64_t batch, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                           int64_t strideA, const void* B, int64_t ldb, int64_t strideB, const void* C,
                           int64_t ldc, int64_t strideC, int out_dtype, int num_cus, int64_t* workspace_bytes,
                           int* dp_tiles, int* sk_tiles, int* sk_slots, int64_t* grid_x) {
    const Shape s = shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype);
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    if (mode < GEMM_STREAMK_AUTO || mode > GEMM_STREAMK_ALL) return GEMM_ERR_ARG;
    SkPlan sp;
    if (s.batch == 0 || s.M == 0 || s.N == 0 || s.K == 0) {
        sp = SkPlan{};
    } else {
        Plan p;
        rc = plan_streamk(mode, s, num_cus > 0 ? num_cus : kDefaultCUs, sp, p);
        if (rc != GEMM_OK) return rc;
    }
    if (workspace_bytes) *workspace_bytes = sp.ws_bytes;
    if (dp_tiles) *dp_tiles = sp.T_dp;
    if (sk_tiles) *sk_tiles = sp.T_sk;
    if (sk_slots) *sk_slots = sp.G_sk;
    if (grid_x) *grid_x = sp.grid;
    return GEMM_OK;
}

int gemm_bf16_splitk_plan(int a_layout, int b_layout, int splits, int64_t batch, int64_t M, int64_t N,
                          int64_t K, const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb,
                          int64_t strideB, const void* C, int64_t ldc, int64_t strideC, int out_dtype,
                          const void* workspace, int64_t workspace_bytes, int num_cus, int* splits_out,
                          int* kernel_id, int64_t* grid_x) {
    const Shape s =
        shape(batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_dtype, a_layout, b_layout);
    int rc = validate(s.la, s.lb, s.batch, s.M, s.N, s.K, s.A, s.lda, s.sA, s.B, s.ldb, s.sB, s.C, s.ldc, s.sC,
                      s.out);
    if (rc != GEMM_OK) return rc;
    Plan p;
    int S = 1;
    rc = plan_splitk(s, splits, workspace, workspace_bytes, num_cus > 0 ? num_cus : kDefaultCUs, &S, p);
    if (rc != GEMM_OK) return rc;
    if (splits_out) *splits_out = S;
    if (kernel_id) *kernel_id = p.kernel;
    if (grid_x) *grid_x = int64_t(p.grid_x) * (p.grid_y ? p.grid_y : 1) * (p.grid_z ? p.grid_z : 1);
    return GEMM_OK;
}

int gemm_mx(int a_format, int b_format, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
            const void* A_scale, int64_t lda_scale, const void* B, int64_t ldb, const void* B_scale,
            int64_t ldb_scale, void* C, int64_t ldc, int out_dtype, void* stream) {
    return run_mx(GEMM_MX_VARIANT_AUTO,
                  MxShape{a_format, b_format, M, N, K, A, A_scale, B, B_scale, lda, lda_scale, ldb, ldb_scale, C,
                          ldc, out_dtype},
                  stream);
}

int gemm_mx_variant(int variant, int a_format, int b_format, int64_t M, int64_t N, int64_t K, const void* A,
                    int64_t lda, const void* A_scale, int64_t lda_scale, const void* B, int64_t ldb,
                    const void* B_scale, int64_t ldb_scale, void* C, int64_t ldc, int out_dtype, void* stream) {
    return run_mx(variant,
                  MxShape{a_format, b_format, M, N, K, A, A_scale, B, B_scale, lda, lda_scale, ldb, ldb_scale, C,
                          ldc, out_dtype},
                  stream);
}

int gemm_mx_validate(int a_format, int b_format, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                     const void* A_scale, int64_t lda_scale, const void* B, int64_t ldb, const void* B_scale,
                     int64_t ldb_scale, const void* C, int64_t ldc, int out_dtype) {
    return validate_mx(MxShape{a_format, b_format, M, N, K, A, A_scale, B, B_scale, lda, lda_scale, ldb,
                               ldb_scale, C, ldc, out_dtype});
}

int gemm_mx_plan(int variant, int a_format, int b_format, int64_t M, int64_t N, int64_t K, const void* A,
                 int64_t lda, const void* A_scale, int64_t lda_scale, const void* B, int64_t ldb,
                 const void* B_scale, int64_t ldb_scale, const void* C, int64_t ldc, int out_dtype, int num_cus,
                 int* kernel_id, int64_t* grid_x, int* block) {
    const MxShape s{a_format, b_format, M, N, K, A, A_scale, B, B_scale, lda, lda_scale, ldb, ldb_scale, C,
                    ldc, out_dtype};
    int rc = validate_mx(s);
    if (rc != GEMM_OK) return rc;
    Plan p;
    rc = plan_mx(variant, s, num_cus > 0 ? num_cus : kDefaultCUs, p);
    if (rc != GEMM_OK) return rc;
    if (kernel_id) *kernel_id = p.kernel;
    if (grid_x) *grid_x = int64_t(p.grid_x) * (p.grid_y ? p.grid_y : 1) * (p.grid_z ? p.grid_z : 1);
    if (block) *block = p.block;
    return GEMM_OK;
}

int attention_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d, const void* Q,
                  const void* K, const void* V, void* O, float* LSE, float scale, int causal, int out_dtype,
                  void* stream) {
    return run_attn(ATTN_VARIANT_AUTO, AttnShape{B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, scale, causal, out_dtype}, LSE,
                    stream);
}

int attention_fwd_variant(int variant, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                          const void* Q, const void* K, const void* V, void* O, float* LSE, float scale, int causal,
                          int out_dtype, void* stream) {
    return run_attn(variant, AttnShape{B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, scale, causal, out_dtype}, LSE, stream);
}

int attention_fwd_validate(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d, const void* Q,
                           const void* K, const void* V, const void* O, float scale, int causal, int out_dtype) {
    return validate_attn(AttnShape{B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, scale, causal, out_dtype});
}

int attention_fwd_plan(int variant, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t d,
                       const void* Q, const void* K, const void* V, const void* O, float scale, int causal,
                       int out_dtype, int num_cus, int* kernel_id, int64_t* grid_x, int* block) {
    const AttnShape s{B, Hq, Hkv, Lq, Lk, d, Q, K, V, O, scale, causal, out_dtype};
    int rc = validate_attn(s);
    if (rc != GEMM_OK) return rc;
    Plan p;
    rc = plan_attn(variant, s, num_cus > 0 ? num_cus : kDefaultCUs, p);
    if (rc != GEMM_OK) return rc;
    if (kernel_id) *kernel_id = p.kernel;
    if (grid_x) *grid_x = int64_t(p.grid_x) * (p.grid_y ? p.grid_y : 1) * (p.grid_z ? p.grid_z : 1);
    if (block) *block = p.block;
    return GEMM_OK;
}

const char* gemm_bf16_kernel_name(int k) {
    switch (k) {
        case K_NONE: return "none";
        case K_ZERO_FILL: return "zero_fill";
        case K_SIMPLE_64: return "simple_64";
        case K_MFMA_128: return "mfma_128";
        case K_PIPE_256: return "pipe_256";
        case K_PIPE_128: return "pipe_128";
        case K_PERSIST_256: return "persist_256";
        case K_PERSIST_128: return "persist_128";
        case K_SPEC_256: return "spec_256";
        case K_PINGPONG_256: return "pingpong_256";
        case K_RING8_256: return "ring8_256";
        case K_RING4_256: return "ring4_256";
        case K_DTV_256: return "dtv_256";
        case K_ROLES: return "roles_256x128";
        case K_MX_RING_256: return "mx_ring_256";
        case K_MX_SIMPLE_64: return "mx_simple_64";
        case K_ATTN_SIMPLE: return "attn_simple";
        case K_ATTN_MFMA: return "attn_mfma";
        case K_ATTN_PIPE: return "attn_pipe";
        case K_GEMV: return "gemv";
        case K_GEMV_LDS: return "gemv_lds";
        default: return "?";
    }
}

const char* gemm_bf16_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_ARG: return "GEMM_ERR_ARG: invalid size, pitch, stride or variant";
        case GEMM_ERR_NULL: return "GEMM_ERR_NULL: null pointer for an operand with nonzero extent";
        case GEMM_ERR_DTYPE: return "GEMM_ERR_DTYPE: out_dtype must be GEMM_OUT_FP32 or GEMM_OUT_BF16";
        case GEMM_ERR_ARCH: return "GEMM_ERR_ARCH: current device is not a gfx950 (MI355X)";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: the HIP runtime rejected the launch";
        case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: variant cannot run these arguments";
        case GEMM_ERR_SCRATCH: return "GEMM_ERR_SCRATCH: the partials exceed the library's 64 MiB scratch";
        default: return "unknown status";
    }
}

int gemm_bf16_version(void) { return kVersion; }

}  // extern "C"
