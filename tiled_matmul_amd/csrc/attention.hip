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

hipError_t launch_attention(const AttnArgs& g, int out, const Plan& p, hipStream_t s) {
    const dim3 grid(p.grid_x, p.grid_y, p.grid_z);
    if (out == OUT_F32)
        hipLaunchKernelGGL(attn_simple_kernel<OUT_F32>, grid, dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL(attn_simple_kernel<OUT_BF16>, grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace tmm
