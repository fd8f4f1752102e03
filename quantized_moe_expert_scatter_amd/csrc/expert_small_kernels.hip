// expert_small_kernels.hip -- the expert products for chunks of a few rows.
//
// A chunk of R <= 8 rows (a short prompt, or the tail of an expert's rows)
// would fill a 32-row MFMA tile mostly with padding, and the product kernel
// decodes every weight block into MFMA operands however few rows use it.
// Here each lane owns one weight row: it reads its row's 16-byte block of the
// tiled layout (a wave reads 1 KB contiguous per block), expands the codes to
// int8, and takes the exact int32 dot of each 32-value block with every row of
// the chunk by v_dot4_i32_i8 (four products per instruction).  The chunk's
// q8_1 rows sit in LDS, read as broadcasts.  The epilogue is the product
// kernel's, operation for operation:
//   acc = fmaf(dx_b, dw_b * (float)dot_b, acc),  blocks b in K order,
// so results equal the MFMA path's bit for bit ("Strata" PR #2145
// description: exact int32 block sums; PR #3752 commit list: a per-32-value
// fp32 epilogue in K order).  Q2_0 codes c in {0..3} enter the dot as int8
// and the weight's -2 offset comes from the q8_1 block sum s:
//   sum (c - 2) q = sum c q - 2 s.
// NL4 codes index the sorted int8 codebook through two byte permutes.
#include "internal.h"
#include "q8_1.cuh"
#include "swiglu.cuh"

#include <hip/hip_runtime.h>

namespace moe {

namespace {

constexpr int kModeOut = 0, kModeDots = 1, kModeSwiglu = 2;   // as in the product kernel
constexpr int kSmallWaves = 4;        // 256 weight rows per workgroup, one per lane
// weight blocks loaded ahead: Q2_0 8 (168 VGPRs, still three waves per
// SIMD), NL4 4 (eight measured slower)
template <int WTYPE>
constexpr int small_slots() { return WTYPE == 1 ? 8 : 4; }

struct SmallRaw {
    uint4 c;          // the lane's 16 code bytes of one block
    uint32_t s;       // its binary16 scale
};

__device__ __forceinline__ float half_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// Q2_0 in the tiled layout: for the block's values 32 h + 16 g + 8 kq + p,
// dword 2 kq + h holds the code of p = 2 k in bits 2 g of byte k and that of
// p = 2 k + 1 in bits 2 g + 4.  Its codes as int8 0..3, the even p in one
// dword and the odd p in the other (k = 0..3 in byte k).
template <int G>
__device__ __forceinline__ void q2_codes(uint32_t w, uint32_t &even, uint32_t &odd) {
    even = (G == 0 ? w : w >> 2) & 0x03030303u;
    odd = (w >> (2 * G + 4)) & 0x03030303u;
}

// NL4: four 4-bit codes (one per byte) -> four int8 codebook entries.
__device__ __forceinline__ uint32_t nl4_lookup4(uint32_t idx, const uint32_t (&cb)[4]) {
    const uint32_t i7 = idx & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(cb[1], cb[0], i7);      // entries 0..7
    const uint32_t hi = __builtin_amdgcn_perm(cb[3], cb[2], i7);      // entries 8..15
    // byte k from hi where bit 3 of its code is set: selector 4 + k, else k
    const uint32_t sel = ((idx & 0x08080808u) >> 1) | 0x03020100u;
    return __builtin_amdgcn_perm(hi, lo, sel);
}

template <int WTYPE, int MODE>
__global__ __launch_bounds__(64 * kSmallWaves) void expert_small_kernel(ProductArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t s_act[kSmallActBytes];

    const int bid = blockIdx.x;
    const int xcd = bid % kXcds;
    const int jj = bid / kXcds;
    const int xcnt = a.xcd_small[kXcds + xcd];
    if (jj >= xcnt * a.n_tiles) return;
    const int c = a.xcd_small[xcd] + jj / a.n_tiles;
    const int tile = jj % a.n_tiles;
    const int expert = a.chunks[4 * c + 0];
    const int row0 = a.chunks[4 * c + 1];
    const int nrows = a.chunks[4 * c + 2];
    if (nrows > a.small_rows) return;                 // never: the lists hold small experts only

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;                       // which of the wave's two 32-row tiles
    const int col = lane & 31;
    const int cols = a.cols;
    constexpr int WB = WTYPE == 1 ? 64 : 32;          // values per weight block
    const int nbw = cols / WB;
    const int nb32 = cols >> 5;
    const uint32_t arb = uint32_t(cols) + uint32_t(nb32) * 8u;      // q8_1 row bytes
    const uint32_t lstride = (arb + 15u) & ~15u;                    // LDS row stride

    // the wave's rows: as in the product kernel, gate/up fused takes gate rows
    // j0..j0+31 in lanes 0..31 and the up rows of the same j's in lanes 32..63
    const int n_ff = a.out_rows >> 1;
    const int n0 = tile * (MODE == kModeSwiglu ? 128 : 256);
    const int nw = MODE == kModeSwiglu ? n0 + 32 * wave : n0 + 64 * wave;
    const bool wave_on = nw < (MODE == kModeSwiglu ? n_ff : a.out_rows);
    const int tb = half == 0 ? nw : (MODE == kModeSwiglu ? n_ff + nw : nw + 32);
    const int wrow = tb + col;
    const uint32_t wr = uint32_t(min(wrow, a.out_rows - 1));
    const uint8_t *wexp = a.w_base + a.w_off[expert];
    // the expert's codes and scales planes through one buffer descriptor: the
    // lane's offsets stay in registers, the block's offset is a scalar
    const uint32_t codes_bytes = uint32_t(a.out_rows) * uint32_t(nbw) * 16u;
    const __amdgpu_buffer_rsrc_t wres =
        __builtin_amdgcn_make_buffer_rsrc((void *)wexp, 0, int(codes_bytes + codes_bytes / 8u), 0x00020000);
    const uint32_t soff = (wr & ~31u) * uint32_t(nbw) + (wr & 31u);  // tiled slot of block 0
    auto wload = [&](int blk) {
        const int b = min(blk, nbw - 1);
        SmallRaw r;
        r.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, soff * 16u, b * 512, 0));
        r.s = __builtin_amdgcn_raw_buffer_load_b16(wres, soff * 2u, int(codes_bytes) + b * 64, 0);
        return r;
    };

    constexpr int kSlots = small_slots<WTYPE>();
    SmallRaw slot[kSlots];
#pragma unroll
    for (int x = 0; x < kSlots; ++x) slot[x] = wload(x);

    // the chunk's q8_1 rows into LDS, 8 bytes at a time (rows are 8-byte
    // aligned): every load of the thread is issued before the first store
    {
        constexpr int kPer = kSmallActBytes / 8 / (64 * kSmallWaves);
        const uint8_t *src = a.act + size_t(row0) * arb;
        const uint32_t per_row = arb / 8u;
        const uint32_t n = uint32_t(nrows) * per_row;
        uint2 v[kPer];
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            const uint32_t i = uint32_t(tid) + uint32_t(x) * (64 * kSmallWaves);
            const uint32_t r = i / per_row, k = i - r * per_row;
            if (i < n) v[x] = *reinterpret_cast<const uint2 *>(src + size_t(r) * arb + 8u * k);
        }
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            const uint32_t i = uint32_t(tid) + uint32_t(x) * (64 * kSmallWaves);
            const uint32_t r = i / per_row, k = i - r * per_row;
            if (i < n) {
                uint2 o = v[x];
                // Q2_0: a group of eight q as its even then its odd values
                if (WTYPE == 1 && k < uint32_t(cols) / 8u)
                    o = uint2{__builtin_amdgcn_perm(v[x].y, v[x].x, 0x06040200u),
                              __builtin_amdgcn_perm(v[x].y, v[x].x, 0x07050301u)};
                *reinterpret_cast<uint2 *>(s_act + r * lstride + 8u * k) = o;
            }
        }
    }
    __syncthreads();

    uint32_t cb[4] = {0u, 0u, 0u, 0u};
    if constexpr (WTYPE == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cb[i] = uint32_t(uint8_t(a.codebook[4 * i])) | (uint32_t(uint8_t(a.codebook[4 * i + 1])) << 8) |
                    (uint32_t(uint8_t(a.codebook[4 * i + 2])) << 16) |
                    (uint32_t(uint8_t(a.codebook[4 * i + 3])) << 24);
    }

    float acc[kMaxSmallRows];
#pragma unroll
    for (int i = 0; i < kMaxSmallRows; ++i) acc[i] = 0.0f;

    const uint8_t *dx_base = s_act + cols;                      // fp32 d of each 32-block
    const uint8_t *s_base = s_act + cols + 4 * nb32;            // int32 s of each 32-block

    // one weight block: its int32 dots with every row, then the epilogue
    auto block = [&](const SmallRaw &w, int blk) {
        const float dw = half_to_float(w.s);
        const uint32_t cw[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
        if constexpr (WTYPE == 1) {
            // group (h, g, kq) of eight values: h picks the q8_1 block (2 blk + h)
            uint32_t e[2][2][2][2];          // [h][g][kq][even, odd]
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    q2_codes<0>(cw[2 * kq + h], e[h][0][kq][0], e[h][0][kq][1]);
                    q2_codes<1>(cw[2 * kq + h], e[h][1][kq][0], e[h][1][kq][1]);
                }
            uint32_t chain = 0u;
#pragma unroll
            for (int i = 0; i < kMaxSmallRows; ++i) {
                if (i >= nrows) break;
                // the row's LDS offset passes through an empty asm that also
                // takes the previous row's dot: the compiler then cannot read
                // every row's operands up front, which held eight rows' worth
                // of registers and halved the waves per SIMD
                uint32_t roff = uint32_t(i) * lstride;
                asm volatile("" : "+v"(roff) : "v"(chain));
                const uint8_t *arow = s_act + roff;
                // the row's q, each group of eight staged as its even then its odd values
                const uint4 *q = reinterpret_cast<const uint4 *>(arow + 64 * blk);
                const uint4 q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
                const uint32_t qv[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                                         q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
                // each dot starts from the -2 s of its block, so the chain of
                // four-wide dots ends at sum (c - 2) q (integer, exact)
                const int2 sb = *reinterpret_cast<const int2 *>(s_base + roff + 8 * blk);
                const float2 dxb = *reinterpret_cast<const float2 *>(dx_base + roff + 8 * blk);
                int d0 = -2 * sb.x, d1 = -2 * sb.y;
                // group (h, g, kq) is q dwords 2 (4 h + 2 g + kq) (even) and + 1 (odd)
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
                        for (int eo = 0; eo < 2; ++eo) {
                            d0 = __builtin_amdgcn_sdot4(int(e[0][g][kq][eo]), int(qv[2 * (2 * g + kq) + eo]), d0, false);
                            d1 = __builtin_amdgcn_sdot4(int(e[1][g][kq][eo]), int(qv[2 * (4 + 2 * g + kq) + eo]), d1, false);
                        }
                chain = uint32_t(d0);
                if constexpr (MODE == kModeDots) {
                    const int rr = row0 + i - a.dots_row_begin;
                    if (wave_on && wrow < a.out_rows && rr >= 0 && rr < a.dots_n_rows) {
                        int32_t *dst = a.dots + (size_t(rr) * a.out_rows + wrow) * nb32 + 2 * blk;
                        dst[0] = d0;
                        dst[1] = d1;
                    }
                } else {
                    acc[i] = __builtin_fmaf(dxb.x, dw * static_cast<float>(d0), acc[i]);
                    acc[i] = __builtin_fmaf(dxb.y, dw * static_cast<float>(d1), acc[i]);
                }
            }
        } else {
            // NL4: low nibbles of dword m are values 4 m..4 m+3, high nibbles 16 + 4 m..
            uint32_t e[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                e[m] = nl4_lookup4(cw[m] & 0x0F0F0F0Fu, cb);
                e[4 + m] = nl4_lookup4((cw[m] >> 4) & 0x0F0F0F0Fu, cb);
            }
#pragma unroll
            for (int i = 0; i < kMaxSmallRows; ++i) {
                if (i >= nrows) break;
                const uint8_t *arow = s_act + i * lstride;
                const uint4 *q = reinterpret_cast<const uint4 *>(arow + 32 * blk);
                const uint4 q0 = q[0], q1 = q[1];
                const uint32_t qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                int d = 0;
#pragma unroll
                for (int m = 0; m < 8; ++m) d = __builtin_amdgcn_sdot4(int(e[m]), int(qv[m]), d, false);
                const float dx = *reinterpret_cast<const float *>(dx_base + i * lstride + 4 * blk);
                if constexpr (MODE == kModeDots) {
                    const int rr = row0 + i - a.dots_row_begin;
                    if (wave_on && wrow < a.out_rows && rr >= 0 && rr < a.dots_n_rows)
                        a.dots[(size_t(rr) * a.out_rows + wrow) * nb32 + blk] = d;
                } else {
                    acc[i] = __builtin_fmaf(dx, dw * static_cast<float>(d), acc[i]);
                }
            }
        }
    };

    // the block stream, kSlots ahead; loads past the end are clamped
    for (int b0 = 0; b0 < nbw; b0 += kSlots) {
#pragma unroll
        for (int x = 0; x < kSlots; ++x) {
            const int blk = b0 + x;
            if (blk < nbw) block(slot[x], blk);
            slot[x] = wload(blk + kSlots);
        }
    }

    if constexpr (MODE == kModeSwiglu) {
        if (!wave_on) return;
        const size_t hrb = size_t(n_ff) + size_t(n_ff >> 5) * 8;
        const int j = nw + col;                                   // the lane's j
#pragma unroll
        for (int i = 0; i < kMaxSmallRows; ++i) {
            if (i >= nrows) break;
            // lanes 0..31 hold gate, 32..63 up of the same j
            const float g = acc[i];
            const float u = __shfl_xor(acc[i], 32);
            const float h = g / (1.0f + exp_neg_rn32(g)) * u;
            float amax = __builtin_fabsf(h);
#pragma unroll
            for (int s = 1; s < 32; s <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, s));
            const float d = amax / 127.0f;
            const int q = d != 0.0f ? int(q8_round(h, d)) : 0;
            int sum = q;
#pragma unroll
            for (int s = 1; s < 32; s <<= 1) sum += __shfl_xor(sum, s);
            uint8_t *hrow = a.hq + size_t(row0 + i) * hrb;
            if (half == 0) {
                hrow[j] = uint8_t(int8_t(q));
                if (col == 0) {
                    reinterpret_cast<float *>(hrow + n_ff)[j >> 5] = d;
                    reinterpret_cast<int32_t *>(hrow + n_ff + 4 * (n_ff >> 5))[j >> 5] = sum;
                }
            }
        }
    } else if constexpr (MODE == kModeOut) {
        if (!wave_on || wrow >= a.out_rows) return;
#pragma unroll
        for (int i = 0; i < kMaxSmallRows; ++i) {
            if (i >= nrows) break;
            const int rr = row0 + i;
            const size_t orow = a.perm ? size_t(a.perm[rr]) : size_t(rr);
            a.out[orow * a.out_rows + wrow] = acc[i];
        }
    }
}

}  // namespace

hipError_t launch_expert_small(const ProductArgs &a, hipStream_t stream) {
    if (a.max_items <= 0 || a.small_rows <= 0) return hipSuccess;
    const dim3 grid(kXcds * a.max_items), block(64 * kSmallWaves);
    if (a.wtype == 1) {
        if (a.dots)
            hipLaunchKernelGGL((expert_small_kernel<1, kModeDots>), grid, block, 0, stream, a);
        else if (a.hq)
            hipLaunchKernelGGL((expert_small_kernel<1, kModeSwiglu>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((expert_small_kernel<1, kModeOut>), grid, block, 0, stream, a);
    } else {
        if (a.dots)
            hipLaunchKernelGGL((expert_small_kernel<2, kModeDots>), grid, block, 0, stream, a);
        else if (a.hq)
            hipLaunchKernelGGL((expert_small_kernel<2, kModeSwiglu>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((expert_small_kernel<2, kModeOut>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace moe
