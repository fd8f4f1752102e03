// q8_1.cuh -- wavefront q8_1 quantization of 8 consecutive values per lane.
//
// q8_1 (the int8 activation format of "Strata" PR #3752's quantize_scatter
// and swiglu_quant): 32-value blocks, d = max|x|/127 in fp32, q = x/d rounded
// half away from zero (clamped to +-127, reachable only for a subnormal d),
// s = sum of q.  A block spans 4 consecutive lanes; amax and s are reduced
// across those lanes with two butterfly steps.  Division is the IEEE
// correctly rounded fp32 divide (the library is built without fast-math), so
// the bytes do not depend on the reduction order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

struct Q8Lane {
    uint32_t q_lo, q_hi;  // 8 int8 values, value i in byte i%4 of word i/4
    float d;              // the block's scale (same on the 4 lanes of a block)
    int32_t s;            // the block's sum (same on the 4 lanes of a block)
};

__device__ __forceinline__ int8_t q8_round(float x, float d) {
    float y = __builtin_roundf(x / d);
    y = __builtin_fminf(__builtin_fmaxf(y, -127.0f), 127.0f);
    return static_cast<int8_t>(static_cast<int>(y));
}

__device__ __forceinline__ Q8Lane q8_1_quantize8(const float (&v)[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2));
    const float d = amax / 127.0f;
    uint32_t w[2] = {0u, 0u};
    int32_t s = 0;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int8_t q = q8_round(v[i], d);
            s += q;
            w[i / 4] |= static_cast<uint32_t>(static_cast<uint8_t>(q)) << (8 * (i % 4));
        }
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    return Q8Lane{w[0], w[1], d, s};
}

}  // namespace moe
