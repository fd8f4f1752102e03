// quant_kernels.hip -- quantize_scatter and swiglu_q8 for gfx950.
//
// Both steps are bound by HBM traffic.  Each is a flat list of 32-value
// blocks: a block spans 4 consecutive lanes, each lane owns 8 consecutive
// values (two 16-byte loads), so a wavefront covers 16 blocks and there is no
// idle lane at any row length.  The q bytes leave as one 8-byte store per
// lane (contiguous within a row), d and s as one 4-byte store each from the
// first lane of each block.
#include "internal.h"
#include "q8_1.cuh"
#include "swiglu.cuh"

#include <hip/hip_runtime.h>

namespace moe {

constexpr int kQuantWaves = 4;  // wavefronts per 256-thread workgroup

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
// (token, expert) pairs.  The 32-value blocks of all tokens form one flat
// list (row-major), four lanes per block, sixteen consecutive blocks per
// wavefront.
__global__ __launch_bounds__(256) void quantize_scatter_kernel(const float *__restrict__ x,
                                                               int tokens, int hidden, int topk,
                                                               const int32_t *__restrict__ inv,
                                                               uint8_t *__restrict__ xq) {
    const int lane = threadIdx.x & 63;
    const int nb = hidden >> 5;
    const size_t n_blocks = size_t(tokens) * nb;
    const size_t b = (size_t(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6)) * 16 + (lane >> 2);
    // lanes of blocks past the end repeat the last block; only real blocks store
    const size_t bc = b < n_blocks ? b : n_blocks - 1;
    const int t = int(bc / nb);
    const int blk = int(bc - size_t(t) * nb);
    const int v0 = blk * 32 + (lane & 3) * 8;
    const float *xr = x + size_t(t) * hidden;
    const float4 a = *reinterpret_cast<const float4 *>(xr + v0);
    const float4 c = *reinterpret_cast<const float4 *>(xr + v0 + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    const Q8Lane q = q8_1_quantize8(v);
    if (b < n_blocks) {
        const size_t rb = size_t(hidden) + size_t(nb) * 8;
        for (int k = 0; k < topk; ++k) {
            const int r = inv[size_t(t) * topk + k];
            store_q8(xq + size_t(r) * rb, hidden, v0, q, lane);
        }
    }
}

// "Strata" PR #3752, swiglu_quant commit: swiglu of each gate/up row and q8_1
// of each 32-value block of the result in one pass; H never reaches memory.
// silu(g) = g / (1 + E) in fp32 with IEEE division, E = e^-g rounded to the
// nearest binary32 (swiglu.cuh).
// The blocks of all rows form one flat list (row-major), four lanes per
// block, sixteen consecutive blocks per wavefront, so no lane idles when
// n_ff is not a multiple of 512.
__global__ __launch_bounds__(256) void swiglu_q8_kernel(const float *__restrict__ gu, int rows,
                                                        int n_ff, uint8_t *__restrict__ hq) {
    const int lane = threadIdx.x & 63;
    const int nb = n_ff >> 5;
    const size_t n_blocks = size_t(rows) * nb;
    const size_t b = (size_t(blockIdx.x) * kQuantWaves + (threadIdx.x >> 6)) * 16 + (lane >> 2);
    // lanes of blocks past the end repeat the last block (same values, same
    // bytes) so that the quad reductions stay full; only real blocks store
    const size_t bc = b < n_blocks ? b : n_blocks - 1;
    const int r = int(bc / nb);
    const int blk = int(bc - size_t(r) * nb);
    const int j0 = blk * 32 + (lane & 3) * 8;
    const float *g_row = gu + size_t(r) * 2 * n_ff;
    const float4 g0 = *reinterpret_cast<const float4 *>(g_row + j0);
    const float4 g1 = *reinterpret_cast<const float4 *>(g_row + j0 + 4);
    const float4 u0 = *reinterpret_cast<const float4 *>(g_row + n_ff + j0);
    const float4 u1 = *reinterpret_cast<const float4 *>(g_row + n_ff + j0 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float silu = g[i] / (1.0f + exp_neg_rn32(g[i]));
        h[i] = silu * u[i];
    }
    const Q8Lane q = q8_1_quantize8(h);
    if (b < n_blocks) {
        const size_t rb = size_t(n_ff) + size_t(nb) * 8;
        store_q8(hq + size_t(r) * rb, n_ff, j0, q, lane);
    }
}

hipError_t launch_quantize_scatter(const float *x, int tokens, int hidden, int topk,
                                   const int32_t *inv, uint8_t *xq, hipStream_t stream) {
    const size_t n_blocks = size_t(tokens) * size_t(hidden >> 5);
    const size_t per_wg = size_t(16) * kQuantWaves;
    const int blocks = int((n_blocks + per_wg - 1) / per_wg);
    hipLaunchKernelGGL(quantize_scatter_kernel, dim3(blocks), dim3(64 * kQuantWaves), 0, stream,
                       x, tokens, hidden, topk, inv, xq);
    return hipGetLastError();
}

hipError_t launch_swiglu_q8(const float *gu, int rows, int n_ff, uint8_t *hq,
                            hipStream_t stream) {
    const size_t n_blocks = size_t(rows) * size_t(n_ff >> 5);
    const size_t per_wg = size_t(16) * kQuantWaves;
    const int blocks = int((n_blocks + per_wg - 1) / per_wg);
    hipLaunchKernelGGL(swiglu_q8_kernel, dim3(blocks), dim3(64 * kQuantWaves), 0, stream, gu,
                       rows, n_ff, hq);
    return hipGetLastError();
}

}  // namespace moe
