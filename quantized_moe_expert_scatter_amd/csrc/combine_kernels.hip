// combine_kernels.hip -- the MoE combine after the down product: each token's
// output row is the routing-weighted sum of its topk expert rows.
//
// "Strata" PR #3752 names the combine among the prompt-path fusions its port
// leaves out and prints no formula; the reading here is the plain weighted
// sum, one fp32 fused multiply-add per term in slot order from zero:
//   out[t][n] = fmaf(w[t][K-1], dm[t*K+K-1][n], ... fmaf(w[t][0], dm[t*K][n], 0))
// The down product writes dm in (token, slot) order, so a token's K rows are
// consecutive and every read and write is a contiguous float4 run: the kernel
// is bound by HBM (K + 1 rows of H floats per token).  When dm is larger than
// the 256 MB infinity cache it is read and the output written non-temporally
// (10 % faster at 16K tokens); a smaller dm, which the down product has just
// written, is still in that cache and is read normally.
#include "internal.h"

#include <hip/hip_runtime.h>

namespace moe {

namespace {

constexpr int kCombineThreads = 256;   // one float4 of one token per thread, over the flat range
constexpr int kCombineBatch = 16;      // slots whose loads are issued together (all of top-10)

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool STREAM>
__device__ __forceinline__ f32x4 load4(const f32x4 *p) {
    if constexpr (STREAM) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool STREAM>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *dm, const float *w,
                                                                  float *out, int topk, int h4,
                                                                  long long n4) {
    // one float4 of one token per thread over the flat (token, float4) range
    const long long g = (long long)blockIdx.x * kCombineThreads + threadIdx.x;
    if (g >= n4) return;
    const int t = int(g / h4);
    const int c = int(g - (long long)t * h4);
    const f32x4 *src = reinterpret_cast<const f32x4 *>(dm) + size_t(t) * topk * h4 + c;
    const float *wt = w + size_t(t) * topk;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < topk; k0 += kCombineBatch) {
        f32x4 d[kCombineBatch];
        float wk[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            if (k0 + j < topk) {
                d[j] = load4<STREAM>(src + size_t(k0 + j) * h4);
                wk[j] = wt[k0 + j];
            }
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            if (k0 + j < topk) {
                acc.x = __builtin_fmaf(wk[j], d[j].x, acc.x);
                acc.y = __builtin_fmaf(wk[j], d[j].y, acc.y);
                acc.z = __builtin_fmaf(wk[j], d[j].z, acc.z);
                acc.w = __builtin_fmaf(wk[j], d[j].w, acc.w);
            }
    }
    f32x4 *dst = reinterpret_cast<f32x4 *>(out) + size_t(t) * h4 + c;
    if constexpr (STREAM) __builtin_nontemporal_store(acc, dst);
    else *dst = acc;
}

}  // namespace

hipError_t launch_combine(const float *dm, const float *w, int tokens, int topk, int hidden,
                          float *out, hipStream_t stream) {
    if (tokens <= 0 || hidden <= 0) return hipSuccess;
    const int h4 = hidden / 4;
    const long long n4 = (long long)tokens * h4;
    const dim3 grid(unsigned((n4 + kCombineThreads - 1) / kCombineThreads)), block(kCombineThreads);
    const size_t dm_bytes = size_t(tokens) * size_t(topk) * size_t(hidden) * 4u;
    if (dm_bytes > (size_t(256) << 20))
        hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, dm, w, out, topk, h4, n4);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, dm, w, out, topk, h4, n4);
    return hipGetLastError();
}

}  // namespace moe
