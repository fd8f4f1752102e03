// expert_kernels.hip -- the two expert products (gate/up and down) for gfx950.
//
// "Strata" PR #3752 (commit list, Approach): one launch per product covers all
// experts; workgroups take row chunks of the experts from a chunk table,
// largest expert first, each expert at its own row count; each weight block is
// decoded once per pass; every product keeps the int8 values, the scales and
// a per-32-value fp32 epilogue in K order, the 32-value integer sums being
// exact.  PR #2145 (description): Q2_0 weights, int8 MMA with int32 sums,
// and a magic constant fed to the accumulator input.
//
// gfx950 design:
//  * A workgroup is one chunk (<= 64 expert-sorted activation rows) against a
//    tile of 256 weight rows of that chunk's expert; its 4 wavefronts own 64
//    weight rows each.  The chunk's q8_1 rows are staged K-step by K-step in
//    LDS (shared by the 4 wavefronts); each wavefront streams its own weight
//    rows straight from HBM into registers and decodes every weight block
//    once, then reuses it against both 32-row activation tiles.
//  * v_mfma_i32_32x32x32_i8: K = 32 is exactly one q8_1 block, so each MFMA
//    yields the exact int32 dot of one 32-value block for a 32x32 tile.  A =
//    activation rows, B = weight rows: a lane's 16 results share one weight
//    row (one scale d_w) and cover 16 activation rows.
//  * The accumulator input C is the bit pattern of 1.5 * 2^23, so
//    D = bits(1.5 * 2^23) + dot and, read as a float, D is 1.5 * 2^23 + dot
//    exactly.  fmaf(d_w, D, -d_w * 1.5 * 2^23) is then d_w * dot rounded once
//    (exact for Q2_0, whose 11-bit scale times a 14-bit dot fits in 24 bits),
//    and fmaf(d_x, that, acc) is the per-32-value epilogue step: two VALU
//    operations per (row, output, block) and no int-to-float conversion.
//  * Work lists are grouped per XCD (workgroup id i runs on XCD i % 8): all
//    chunks of an expert land on one XCD, so the 5 or 10 weight tiles and
//    the chunk's activation rows are re-read from that XCD's L2.
#include "internal.h"

#include <hip/hip_runtime.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kKStep = 256;                 // contraction values staged per step
constexpr int kQStride = kKStep + 16;       // LDS bytes per activation row (padded)
constexpr float kMagicF = 12582912.0f;      // 1.5 * 2^23

// Q2_0 block -> the 16 signed int8 weights a lane feeds to the MFMA.
// Lane group g (lanes 32g..32g+31) supplies values 16g..16g+15 of a 32-value
// half h; those are field j = 2h + g (bits 2j..2j+1) of the block's 16 bytes.
// v_perm_b32 maps each 2-bit code c to the byte c - 2 through the table
// {0xFE, 0xFF, 0x00, 0x01} (given in both sources so selectors 0-3 and 4-7
// agree).
__device__ __forceinline__ v4i q2_0_operand(const uint4 &codes, int j) {
    const uint32_t kTable = 0x0100FFFEu;
    const int sh = 2 * j;
    v4i r;
    r.x = __builtin_amdgcn_perm(kTable, kTable, (codes.x >> sh) & 0x03030303u);
    r.y = __builtin_amdgcn_perm(kTable, kTable, (codes.y >> sh) & 0x03030303u);
    r.z = __builtin_amdgcn_perm(kTable, kTable, (codes.z >> sh) & 0x03030303u);
    r.w = __builtin_amdgcn_perm(kTable, kTable, (codes.w >> sh) & 0x03030303u);
    return r;
}

// NL4 block -> 16 int8 codebook entries: lane group 0 takes the low nibbles
// (values 0..15), group 1 the high nibbles (values 16..31).  Two byte-select
// lookups (entries 0-7 and 8-15) are merged on bit 3 of each code.
__device__ __forceinline__ uint32_t nl4_lookup(uint32_t c, uint32_t cb0, uint32_t cb1,
                                               uint32_t cb2, uint32_t cb3) {
    const uint32_t lo3 = c & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(cb1, cb0, lo3);   // entries 0..7
    const uint32_t hi = __builtin_amdgcn_perm(cb3, cb2, lo3);   // entries 8..15
    // selector 0x0C yields 0x00 and 0x0D yields 0xFF
    const uint32_t msel = ((c >> 3) & 0x01010101u) | 0x0C0C0C0Cu;
    const uint32_t mask = __builtin_amdgcn_perm(0u, 0u, msel);
    return (hi & mask) | (lo & ~mask);
}

__device__ __forceinline__ v4i nl4_operand(const uint4 &codes, int g, const uint32_t (&cb)[4]) {
    const int sh = 4 * g;
    v4i r;
    r.x = nl4_lookup((codes.x >> sh) & 0x0F0F0F0Fu, cb[0], cb[1], cb[2], cb[3]);
    r.y = nl4_lookup((codes.y >> sh) & 0x0F0F0F0Fu, cb[0], cb[1], cb[2], cb[3]);
    r.z = nl4_lookup((codes.z >> sh) & 0x0F0F0F0Fu, cb[0], cb[1], cb[2], cb[3]);
    r.w = nl4_lookup((codes.w >> sh) & 0x0F0F0F0Fu, cb[0], cb[1], cb[2], cb[3]);
    return r;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return static_cast<float>(v);
}

// Output row of MFMA result register v for lane group g (32x32 layout).
__device__ __forceinline__ int tile_row(int v, int g) { return (v & 3) + 8 * (v >> 2) + 4 * g; }

template <int WTYPE, bool DOTS>
__global__ __launch_bounds__(256, 2) void expert_product_kernel(ProductArgs a) {
    constexpr int WB = WTYPE == 1 ? 64 : 32;       // values per weight block
    constexpr int HALVES = WB / 32;                // q8_1 blocks per weight block
    constexpr int MAXWB = kKStep / WB;             // weight blocks per K-step

    __shared__ __attribute__((aligned(16))) uint8_t q_lds[64 * kQStride];
    __shared__ __attribute__((aligned(16))) float dx_lds[(kKStep / 32) * 64];

    // ---- work item: (chunk, weight tile) from this XCD's list
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds;
    const int j = bid / kXcds;
    const int xcnt = a.xcd[kXcds + xcd];
    if (j >= xcnt * a.n_tiles) return;
    const int c = a.xcd[xcd] + j / a.n_tiles;
    const int tile = j % a.n_tiles;
    const int expert = a.chunks[4 * c + 0];
    const int row0 = a.chunks[4 * c + 1];
    const int nrows = a.chunks[4 * c + 2];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 5;
    const int col = lane & 31;
    const int n_wave = tile * kTileRows + wave * 64;     // first weight row of this wave
    const bool wave_on = n_wave < a.out_rows;

    const int cols = a.cols;
    const int nb32 = cols >> 5;
    const size_t arb = size_t(cols) + size_t(nb32) * 8;  // q8_1 row bytes
    const int nbw = cols / WB;                            // weight blocks per row
    const uint8_t *wexp = a.w_base + a.w_off[expert];
    const uint8_t *wcodes = wexp;
    const uint16_t *wscales = reinterpret_cast<const uint16_t *>(wexp + size_t(a.out_rows) * nbw * 16);

    uint32_t cb[4] = {0u, 0u, 0u, 0u};
    if constexpr (WTYPE == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            cb[i] = uint32_t(uint8_t(a.codebook[4 * i])) | (uint32_t(uint8_t(a.codebook[4 * i + 1])) << 8) |
                    (uint32_t(uint8_t(a.codebook[4 * i + 2])) << 16) |
                    (uint32_t(uint8_t(a.codebook[4 * i + 3])) << 24);
    }

    v16i magic;
#pragma unroll
    for (int v = 0; v < 16; ++v) magic[v] = int(kMagicBits);

    v16f acc[2][2];
#pragma unroll
    for (int at = 0; at < 2; ++at)
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[at][bt][v] = 0.0f;

    for (int k0 = 0; k0 < cols; k0 += kKStep) {
        const int ks = min(kKStep, cols - k0);
        const int nbk = ks >> 5;  // q8_1 blocks in this step

        __syncthreads();
        // ---- stage the chunk's activation q bytes and scales for this step
        {
            const int r = tid >> 2;
            const int seg = (tid & 3) * 64;
            const uint8_t *src = a.act + size_t(row0 + r) * arb + k0 + seg;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int off = seg + 16 * p;
                if (off < ks) {
                    uint4 v = make_uint4(0u, 0u, 0u, 0u);
                    if (r < nrows) v = *reinterpret_cast<const uint4 *>(src + 16 * p);
                    *reinterpret_cast<uint4 *>(q_lds + r * kQStride + off) = v;
                }
            }
            const int rr = tid & 63;
            for (int kb = tid >> 6; kb < nbk; kb += 4) {
                float d = 0.0f;
                if (rr < nrows)
                    d = reinterpret_cast<const float *>(a.act + size_t(row0 + rr) * arb + cols)[(k0 >> 5) + kb];
                dx_lds[kb * 64 + rr] = d;
            }
        }
        __syncthreads();
        if (!wave_on) continue;

        // ---- this wave's weight blocks for the step (two 32-row B tiles)
        const int nwb = ks / WB;
        uint4 codes[2][MAXWB];
        float dwf[2][MAXWB];
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) {
            const int n = n_wave + bt * 32 + col;
            const size_t blk0 = size_t(n) * nbw + (k0 / WB);
#pragma unroll
            for (int wb = 0; wb < MAXWB; ++wb) {
                if (wb < nwb) {
                    codes[bt][wb] = *reinterpret_cast<const uint4 *>(wcodes + (blk0 + wb) * 16);
                    dwf[bt][wb] = half_bits_to_float(wscales[blk0 + wb]);
                } else {
                    codes[bt][wb] = make_uint4(0u, 0u, 0u, 0u);
                    dwf[bt][wb] = 0.0f;
                }
            }
        }

#pragma unroll
        for (int wb = 0; wb < MAXWB; ++wb) {
            if (wb >= nwb) break;
#pragma unroll
            for (int h = 0; h < HALVES; ++h) {
                const int kb = wb * HALVES + h;   // q8_1 block within the step
                v4i bop[2];
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) {
                    if constexpr (WTYPE == 1)
                        bop[bt] = q2_0_operand(codes[bt][wb], 2 * h + g);
                    else
                        bop[bt] = nl4_operand(codes[bt][wb], g, cb);
                }
#pragma unroll
                for (int at = 0; at < 2; ++at) {
                    const v4i aop = *reinterpret_cast<const v4i *>(
                        q_lds + (at * 32 + col) * kQStride + kb * 32 + 16 * g);
                    float dxv[16];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float4 d4 = *reinterpret_cast<const float4 *>(
                            dx_lds + kb * 64 + at * 32 + 8 * m + 4 * g);
                        dxv[4 * m + 0] = d4.x;
                        dxv[4 * m + 1] = d4.y;
                        dxv[4 * m + 2] = d4.z;
                        dxv[4 * m + 3] = d4.w;
                    }
#pragma unroll
                    for (int bt = 0; bt < 2; ++bt) {
                        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop[bt], magic, 0, 0, 0);
                        if constexpr (DOTS) {
                            const int n = n_wave + bt * 32 + col;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int rl = at * 32 + tile_row(v, g);
                                const int r = row0 + rl - a.dots_row_begin;
                                if (rl < nrows && r >= 0 && r < a.dots_n_rows)
                                    a.dots[(size_t(r) * a.out_rows + n) * nb32 + (k0 >> 5) + kb] =
                                        D[v] - int(kMagicBits);
                            }
                        } else {
                            const float dw = dwf[bt][wb];
                            const float ndwm = -dw * kMagicF;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const float p = __builtin_fmaf(dw, __int_as_float(D[v]), ndwm);
                                acc[at][bt][v] = __builtin_fmaf(dxv[v], p, acc[at][bt][v]);
                            }
                        }
                    }
                }
            }
        }
    }

    if constexpr (!DOTS) {
        if (!wave_on) return;
#pragma unroll
        for (int at = 0; at < 2; ++at)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rl = at * 32 + tile_row(v, g);
                if (rl >= nrows) continue;
                const int r = row0 + rl;
                const size_t orow = a.perm ? size_t(a.perm[r]) : size_t(r);
                float *dst = a.out + orow * a.out_rows + n_wave + col;
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) dst[bt * 32] = acc[at][bt][v];
            }
    }
}

hipError_t launch_expert_product(const ProductArgs &a, hipStream_t stream) {
    if (a.max_items <= 0) return hipSuccess;
    const dim3 grid(kXcds * a.max_items), block(256);
    if (a.wtype == 1) {
        if (a.dots)
            hipLaunchKernelGGL((expert_product_kernel<1, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((expert_product_kernel<1, false>), grid, block, 0, stream, a);
    } else {
        if (a.dots)
            hipLaunchKernelGGL((expert_product_kernel<2, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((expert_product_kernel<2, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace moe
