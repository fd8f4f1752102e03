// quant_kernels.hip -- quantize_scatter and swiglu_q8 for gfx950.
//
// Both steps are bound by HBM traffic: one wavefront per row, each lane owns
// 8 consecutive values (two 16-byte loads), a 32-value q8_1 block spans 4
// lanes, and a 512-value slab of the row is quantized per iteration.  The q
// bytes of a slab leave as one 8-byte store per lane (512 contiguous bytes
// per wavefront), d and s as one 4-byte store from the first lane of each
// block.
#include "internal.h"
#include "q8_1.cuh"

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kQuantWaves = 4;  // wavefronts (rows) per 256-thread workgroup

__device__ __forceinline__ void store_q8(uint8_t *row, int cols, int v0, const Q8Lane &q,
                                         int lane) {
    *reinterpret_cast<uint2 *>(row + v0) = make_uint2(q.q_lo, q.q_hi);
    if ((lane & 3) == 0) {
        const int blk = v0 >> 5;
        const int nb = cols >> 5;
        reinterpret_cast<float *>(row + cols)[blk] = q.d;
        reinterpret_cast<int32_t *>(row + cols + 4 * nb)[blk] = q.s;
    }
}

// "Strata" PR #3752, commit list: quantize_scatter -- every token's row is
// quantized once and written to the expert-sorted row of each of its topk
// (token, expert) pairs.
__global__ __launch_bounds__(256) void quantize_scatter_kernel(const float *__restrict__ x,
                                                               int tokens, int hidden, int topk,
                                                               const int32_t *__restrict__ inv,
                                                               uint8_t *__restrict__ xq) {
    const int lane = threadIdx.x & 63;
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kQuantWaves + (threadIdx.x >> 6));
    if (t >= tokens) return;
    const size_t rb = size_t(hidden) + size_t(hidden >> 5) * 8;
    const float *xr = x + size_t(t) * hidden;
    for (int base = 0; base < hidden; base += 512) {
        const int v0 = base + lane * 8;
        float v[8];
        if (v0 < hidden) {
            const float4 a = *reinterpret_cast<const float4 *>(xr + v0);
            const float4 b = *reinterpret_cast<const float4 *>(xr + v0 + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        }
        const Q8Lane q = q8_1_quantize8(v);
        if (v0 < hidden) {
            for (int k = 0; k < topk; ++k) {
                const int r = inv[size_t(t) * topk + k];
                store_q8(xq + size_t(r) * rb, hidden, v0, q, lane);
            }
        }
    }
}

// "Strata" PR #3752, swiglu_quant commit: swiglu of each gate/up row and q8_1
// of each 32-value block of the result in one pass; H never reaches memory.
// silu(g) = g / (1 + E) in fp32 with IEEE division, E = e^-g rounded once to
// binary32 from a binary64 exponential, so E is the nearest binary32 value
// except when e^-g lies within about 2^-29 of a rounding boundary.
__global__ __launch_bounds__(256) void swiglu_q8_kernel(const float *__restrict__ gu, int rows,
                                                        int n_ff, uint8_t *__restrict__ hq) {
    const int lane = threadIdx.x & 63;
    const int r = __builtin_amdgcn_readfirstlane(blockIdx.x * kQuantWaves + (threadIdx.x >> 6));
    if (r >= rows) return;
    const size_t rb = size_t(n_ff) + size_t(n_ff >> 5) * 8;
    const float *g_row = gu + size_t(r) * 2 * n_ff;
    const float *u_row = g_row + n_ff;
    uint8_t *out = hq + size_t(r) * rb;
    for (int base = 0; base < n_ff; base += 512) {
        const int j0 = base + lane * 8;
        float h[8];
        if (j0 < n_ff) {
            const float4 g0 = *reinterpret_cast<const float4 *>(g_row + j0);
            const float4 g1 = *reinterpret_cast<const float4 *>(g_row + j0 + 4);
            const float4 u0 = *reinterpret_cast<const float4 *>(u_row + j0);
            const float4 u1 = *reinterpret_cast<const float4 *>(u_row + j0 + 4);
            const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e = static_cast<float>(exp(-static_cast<double>(g[i])));
                const float silu = g[i] / (1.0f + e);
                h[i] = silu * u[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = 0.0f;
        }
        const Q8Lane q = q8_1_quantize8(h);
        if (j0 < n_ff) store_q8(out, n_ff, j0, q, lane);
    }
}

hipError_t launch_quantize_scatter(const float *x, int tokens, int hidden, int topk,
                                   const int32_t *inv, uint8_t *xq, hipStream_t stream) {
    const int blocks = (tokens + kQuantWaves - 1) / kQuantWaves;
    hipLaunchKernelGGL(quantize_scatter_kernel, dim3(blocks), dim3(64 * kQuantWaves), 0, stream,
                       x, tokens, hidden, topk, inv, xq);
    return hipGetLastError();
}

hipError_t launch_swiglu_q8(const float *gu, int rows, int n_ff, uint8_t *hq,
                            hipStream_t stream) {
    const int blocks = (rows + kQuantWaves - 1) / kQuantWaves;
    hipLaunchKernelGGL(swiglu_q8_kernel, dim3(blocks), dim3(64 * kQuantWaves), 0, stream, gu,
                       rows, n_ff, hq);
    return hipGetLastError();
}

}  // namespace moe
