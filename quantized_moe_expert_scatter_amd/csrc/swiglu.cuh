// swiglu.cuh -- the SwiGLU arithmetic shared by every kernel that computes H.
//
// "Strata" PR #3752, swiglu_quant commit: h = silu(g) * u for each gate/up
// pair, silu(g) = g / (1 + E) in fp32 with E = e^-g rounded to binary32.
// Every kernel computes E and the quotient with these functions, so the
// fused gate/up epilogue, the standalone swiglu pass and the small-chunk
// kernel write the same bytes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// E = e^-g rounded to the nearest binary32, for every binary32 g.
// Binary64 steps: x = -g clamped to [-104, 89] (beyond it e^x rounds to 0 or
// overflows binary32, as it does at the clamp); n = nearest integer to
// x / ln 2, read from the low bits of x * log2(e) + 1.5 * 2^52; r = x - n ln 2
// with ln 2 split into a 32-bit head (n * head is exact) and a rounded tail;
// e^r by its Taylor polynomial to degree 13 in Horner form (truncation below
// 0.05 of a binary64 ulp for |r| <= ln2 / 2); the result scaled by 2^n and
// rounded once to binary32.  Checked on the host against the C library's
// binary64 exponential and an 80-bit one, rounded to binary32: equal for every
// binary32 g in [-89, 104] and beyond both ends.
__device__ __forceinline__ float exp_neg_rn32(float g) {
    const float gc = __builtin_amdgcn_fmed3f(g, -89.0f, 104.0f);
    const double x = -static_cast<double>(gc);
    const double t = __builtin_fma(x, 0x1.71547652b82fep+0, 0x1.8p52);
    const double n = t - 0x1.8p52;
    const int ni = static_cast<int>(static_cast<uint32_t>(__builtin_bit_cast(uint64_t, t)));
    double r = __builtin_fma(-n, 0x1.62e42fee00000p-1, x);
    r = __builtin_fma(-n, 0x1.a39ef35793c76p-33, r);
    double p = 1.0 / 6227020800.0;
    p = __builtin_fma(p, r, 1.0 / 479001600.0);
    p = __builtin_fma(p, r, 1.0 / 39916800.0);
    p = __builtin_fma(p, r, 1.0 / 3628800.0);
    p = __builtin_fma(p, r, 1.0 / 362880.0);
    p = __builtin_fma(p, r, 1.0 / 40320.0);
    p = __builtin_fma(p, r, 1.0 / 5040.0);
    p = __builtin_fma(p, r, 1.0 / 720.0);
    p = __builtin_fma(p, r, 1.0 / 120.0);
    p = __builtin_fma(p, r, 1.0 / 24.0);
    p = __builtin_fma(p, r, 1.0 / 6.0);
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    return static_cast<float>(__builtin_ldexp(p, ni));
}

// g / s for s = 1 + E >= 1, correctly rounded to binary32 as the fp32 divide
// gives it, without the divide: a binary64 reciprocal of s refined by two
// Newton steps (relative error far below 2^-50), times g, rounded to
// binary32.  The quotient of two binary32 values is never a binary32 rounding
// boundary and lies at least 2^-49 of its size from one, so that rounding is
// the correctly rounded quotient; a quotient below the normal range comes
// only from |g| < 2^-125, where s = 2 and the product is exact.  s = inf (e^-g
// beyond binary32) is taken as 2^1000: the product then rounds to the signed
// zero that g / inf is.
__device__ __forceinline__ float silu_div(double gd, float s) {
    const double sd = __builtin_fmin(static_cast<double>(s), 0x1p1000);
    double r = __builtin_amdgcn_rcp(sd);
    r = __builtin_fma(r, __builtin_fma(-sd, r, 1.0), r);
    r = __builtin_fma(r, __builtin_fma(-sd, r, 1.0), r);
    return static_cast<float>(gd * r);
}

}  // namespace moe
