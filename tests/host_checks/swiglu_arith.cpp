// Host harness for the device arithmetic of swiglu.cuh: the test compiles the
// device functions' own text (extracted from swiglu.cuh into swiglu_host.inc)
// with g++, the two device builtins replaced by host stand-ins:
//   __builtin_amdgcn_fmed3f(x, lo, hi) -> the median of the three
//   __builtin_amdgcn_rcp(x)             -> a reciprocal seed no better than 2^-20
// Mode "exp": every binary32 g in [-89, 104] and 2^21 values beyond each end;
// E must equal the C library's binary64 exponential rounded to binary32, and
// the 80-bit one rounded to binary32.  Mode "silu": 2^26 pseudo-random
// (g, E) pairs over all magnitudes (and E = inf); silu_div must equal the
// binary32 division g / (1 + E).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

static inline float host_med3(float x, float lo, float hi) { return std::fmin(std::fmax(x, lo), hi); }
static inline double host_rcp_seed(double x) {
    // 1/x with a relative error of about 2^-20 (a poor hardware seed)
    return (1.0 / x) * (1.0 + 0x1p-20);
}
#define __device__
#define __forceinline__ inline
#define __builtin_amdgcn_fmed3f host_med3
#define __builtin_amdgcn_rcp host_rcp_seed
namespace moe {
#include "swiglu_host.inc"
}

static float f32(uint32_t b) { float f; std::memcpy(&f, &b, 4); return f; }

int main(int argc, char **argv) {
    if (argc > 1 && std::strcmp(argv[1], "silu") == 0) {
        long long bad = 0, n = 0;
        uint64_t s = 0x9E3779B97F4A7C15ull;
        for (long long i = 0; i < (1ll << 26); ++i) {
            s ^= s << 13; s ^= s >> 7; s ^= s << 17;
            const float g = f32(uint32_t(s) & 0xFF7FFFFFu);          // finite, any sign
            float e = f32(uint32_t(s >> 32) & 0x7F7FFFFFu);           // finite, >= 0
            if ((i & 1023) == 0) e = INFINITY;
            const float sum = 1.0f + e;
            const float ref = g / sum;
            const float got = moe::silu_div(double(g), sum);
            ++n;
            if (std::memcmp(&ref, &got, 4) != 0) ++bad;
        }
        std::printf("silu pairs %lld mismatches %lld\n", n, bad);
        return bad != 0;
    }
    long long n = 0, bad_lib = 0, bad_ext = 0;
    for (int sign = 0; sign < 2; ++sign) {
        const float lim = sign ? 89.0f : 104.0f;
        uint32_t top;
        std::memcpy(&top, &lim, 4);
#pragma omp parallel for reduction(+ : n, bad_lib, bad_ext) schedule(static, 1 << 20)
        for (long long b = 0; b <= (long long)top + (1 << 21); ++b) {
            const uint32_t bits = uint32_t(b) | (sign ? 0x80000000u : 0u);
            const float g = f32(bits);
            if (std::isnan(g)) continue;
            const float got = moe::exp_neg_rn32(g);
            const float lib = float(std::exp(-double(g)));
            const float ext = float(std::exp(-(long double)g));
            ++n;
            if (std::memcmp(&got, &lib, 4) != 0) ++bad_lib;
            if (std::memcmp(&got, &ext, 4) != 0) ++bad_ext;
        }
    }
    std::printf("exp inputs %lld mismatches vs binary64 %lld vs 80-bit %lld\n", n, bad_lib, bad_ext);
    return (bad_lib != 0 || bad_ext != 0);
}
