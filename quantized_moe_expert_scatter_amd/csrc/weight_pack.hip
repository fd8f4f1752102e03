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

// One thread per block slot of the packed order: slot d is (tile i, block b,
// row r) with d = (i * nb + b) * 32 + r, filled from block b of row 32 i + r
// (of row 2n or 2(n - half) + 1 for packed row n when the source alternates
// gate and up rows).  Writes are contiguous in d; reads gather 16-byte blocks.
__global__ __launch_bounds__(256) void weight_pack_kernel(const uint8_t *src, uint8_t *dst,
                                                          uint64_t expert_stride, uint32_t n_blocks,
                                                          uint32_t nb, uint32_t half) {
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
    *reinterpret_cast<uint4 *>(d_codes + size_t(d) * 16) =
        *reinterpret_cast<const uint4 *>(s_codes + size_t(s) * 16);
    const uint16_t *s_scales = reinterpret_cast<const uint16_t *>(s_codes + size_t(n_blocks) * 16);
    uint16_t *d_scales = reinterpret_cast<uint16_t *>(d_codes + size_t(n_blocks) * 16);
    d_scales[d] = s_scales[s];
}

}  // namespace

hipError_t launch_weight_pack(const uint8_t *src, uint8_t *dst, uint64_t expert_stride,
                              int n_expert, int rows, int blocks_per_row, int half,
                              hipStream_t stream) {
    const uint32_t n_blocks = uint32_t(rows) * uint32_t(blocks_per_row);
    if (n_blocks == 0 || n_expert <= 0) return hipSuccess;
    const dim3 grid((n_blocks + 255u) / 256u, uint32_t(n_expert)), block(256);
    hipLaunchKernelGGL(weight_pack_kernel, grid, block, 0, stream, src, dst, expert_stride, n_blocks,
                       uint32_t(blocks_per_row), uint32_t(half));
    return hipGetLastError();
}

}  // namespace moe
