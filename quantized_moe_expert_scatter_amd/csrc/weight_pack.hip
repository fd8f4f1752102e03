// weight_pack.hip -- the product kernels' weight layout, written once when a
// layer's weights are loaded.
//
// A Q2_0 or NL4 matrix arrives as two row-major planes: the 16-byte code
// blocks in (row, block) order, then the binary16 scales in the same order.
// The product kernels read one K stage of a 32-row MFMA tile at a time, so
// the packed planes order the blocks (row tile, block, row in tile): the 32
// rows' codes of one block are 512 contiguous bytes and their scales 64.  In
// row-major order the same reads touch 32 cache lines per tile and stage, each
// for 16 bytes (or 2), and the L2-to-L1 traffic becomes several times the
// weights' size.  Every plane keeps its size and place, so an expert's offset
// is the same in both layouts.
#include "internal.h"

#include <hip/hip_runtime.h>

namespace moe {

namespace {

// Q2_0 codes of one 64-value block in the kernels' order.  Byte 8 kq + 4 h + k
// of the packed block holds nibble h of source byte 8 kq + 2 k in its low
// nibble and nibble h of source byte 8 kq + 2 k + 1 in its high nibble: the
// values 32 h + 16 g + 8 kq + p (p = 2 k, 2 k + 1) at bits 2 g + 4 (p & 1),
// so that the product kernel's lane half kq finds the eight values of its
// MFMA (h, g) in the pairs 00cc of word h's bytes after one mask.
__device__ __forceinline__ uint4 q2_tiled_block(uint4 c) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[4];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
        const uint32_t s0 = w[2 * kq], s1 = w[2 * kq + 1];
        const uint32_t ev = __builtin_amdgcn_perm(s1, s0, 0x06040200u);   // bytes 8kq + 2k
        const uint32_t od = __builtin_amdgcn_perm(s1, s0, 0x07050301u);   // bytes 8kq + 2k + 1
        o[2 * kq] = (ev & 0x0F0F0F0Fu) | ((od & 0x0F0F0F0Fu) << 4);
        o[2 * kq + 1] = ((ev >> 4) & 0x0F0F0F0Fu) | (od & 0xF0F0F0F0u);
    }
    return uint4{o[0], o[1], o[2], o[3]};
}

// One thread per block slot of the packed order: slot d is (tile i, block b,
// row r) with d = (i * nb + b) * 32 + r, filled from block b of row 32 i + r
// (of row 2n or 2(n - half) + 1 for packed row n when the source alternates
// gate and up rows).  Writes are contiguous in d; reads gather 16-byte blocks.
__global__ __launch_bounds__(256) void weight_pack_kernel(const uint8_t *src, uint8_t *dst,
                                                          uint64_t expert_stride, uint32_t n_blocks,
                                                          uint32_t nb, uint32_t half, uint32_t q2) {
    const uint32_t d = blockIdx.x * 256u + threadIdx.x;
    if (d >= n_blocks) return;
    const uint64_t e = uint64_t(blockIdx.y) * expert_stride;
    const uint8_t *s_codes = src + e;
    uint8_t *d_codes = dst + e;
    const uint32_t r = d & 31u;
    const uint32_t q = d >> 5;
    const uint32_t b = q % nb;
    const uint32_t i = q / nb;
    const uint32_t row = 32u * i + r;
    const uint32_t src_row = half == 0 ? row : (row < half ? 2u * row : 2u * (row - half) + 1u);
    const uint32_t s = src_row * nb + b;
    uint4 c = *reinterpret_cast<const uint4 *>(s_codes + size_t(s) * 16);
    if (q2) c = q2_tiled_block(c);
    *reinterpret_cast<uint4 *>(d_codes + size_t(d) * 16) = c;
    const uint16_t *s_scales = reinterpret_cast<const uint16_t *>(s_codes + size_t(n_blocks) * 16);
    uint16_t *d_scales = reinterpret_cast<uint16_t *>(d_codes + size_t(n_blocks) * 16);
    d_scales[d] = s_scales[s];
}

}  // namespace

hipError_t launch_weight_pack(const uint8_t *src, uint8_t *dst, uint64_t expert_stride,
                              int n_expert, int rows, int blocks_per_row, int half, bool q2,
                              hipStream_t stream) {
    const uint32_t n_blocks = uint32_t(rows) * uint32_t(blocks_per_row);
    if (n_blocks == 0 || n_expert <= 0) return hipSuccess;
    const dim3 grid((n_blocks + 255u) / 256u, uint32_t(n_expert)), block(256);
    hipLaunchKernelGGL(weight_pack_kernel, grid, block, 0, stream, src, dst, expert_stride, n_blocks,
                       uint32_t(blocks_per_row), uint32_t(half), uint32_t(q2));
    return hipGetLastError();
}

}  // namespace moe
