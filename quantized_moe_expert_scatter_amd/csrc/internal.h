// internal.h -- shared between the host boundary (moe_prefill.cpp) and the
// HIP kernels: the device plan layout and the launcher entry points.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace moe {

constexpr int kXcds = 8;           // MI355X: 8 accelerator dies, each with its own L2
constexpr int kMaxChunkRows = 128;  // rows of one chunk = four 32-row MFMA tiles
constexpr int kTileRows = 256;     // weight rows (outputs) per workgroup: 4 waves x 64
constexpr int kMaxSmallRows = 8;      // chunks of at most this many rows take the small kernel
constexpr int kSmallActBytes = 32768; // its LDS for the chunk's q8_1 rows
// A product whose small experts make fewer chunks than this, beside large
// ones, runs them on the product kernel instead: a launch of a few
// small-chunk workgroups, each streaming an expert's weights, costs its full
// latency (about 47 us for gate/up at 8,192 lognormal tokens) where a few
// more items in the product launch cost next to nothing.
constexpr int kSmallMinChunks = 96;
// Threads per workgroup of both product kernels; a launch takes kXcds
// workgroups per item of the longest XCD list, and HIP caps a launch at
// 2^32 - 1 threads.
constexpr int kProductThreads = 256;
constexpr long long kMaxLaunchThreads = 0xFFFFFFFFLL;

constexpr size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

inline int max_chunks(int rows, int n_expert, int chunk_rows) {
    return rows / chunk_rows + n_expert + 1;
}

// Byte offsets of the sections of the device plan workspace.  Every section
// is 16-byte aligned.
struct PlanLayout {
    size_t perm;     // int32 [R]     sorted row -> t*K+k
    size_t inv;      // int32 [R]     t*K+k -> sorted row
    size_t chunks;   // int32 [maxc][4] chunk table grouped by XCD (see xcd)
    size_t xcd;      // int32 [kXcdRows][kXcds]: the XCD lists, see XcdRow
    size_t gu_off;   // uint64 [E]    gate/up expert byte offsets
    size_t dn_off;   // uint64 [E]    down expert byte offsets
    // built on the device only (moe_prefill_plan_device); zero in a host plan
    size_t counts;   // int32 [E+1]   rows per expert, then ids out of range
    size_t offsets;  // int32 [E+2]   exclusive prefix of counts
    size_t aux;      // int32 [kPlanAux(E)]: see PlanAux
    size_t tiles;    // int32 [E+1][n_tiles]: per id tile, rows of each bucket, then
                     // (after the scan) the bucket's rows in earlier tiles
    size_t total;
};

// Experts a device-built plan takes (its scheduling workgroup stages four
// int32 arrays of this length in LDS, 40 KB).
constexpr int kPlanMaxExperts = 2048;
// The device plan splits the routing ids into tiles of a multiple of 2048
// consecutive ids (one workgroup each, 8 ids per thread and pass), at most
// kPlanMaxTiles of them.
constexpr int kPlanPassIds = 2048;
constexpr int kPlanMaxTiles = 256;
inline int plan_tile_ids(long long rows) {
    const long long per = (rows + kPlanMaxTiles - 1) / kPlanMaxTiles;
    const long long t = (per + kPlanPassIds - 1) / kPlanPassIds * kPlanPassIds;
    return int(t > kPlanPassIds ? t : kPlanPassIds);
}
inline int plan_n_tiles(long long rows) {
    const long long t = plan_tile_ids(rows);
    return rows > 0 ? int((rows + t - 1) / t) : 1;
}

// Rows of the XCD table (kXcds entries each).  List x is chunks
// [start[x], start[x] + count[x]) of the XCD-grouped chunk table, experts in
// rank order, each expert's chunks together; for product p (0 gate/up, 1
// down) the chunks of experts with more rows than small_rows_for(that
// product's contraction length) come first ("large", the product kernel's
// items) and the rest follow ("small", the small kernel's).  Each view is a
// (start, count) pair of rows, so a kernel reads xcd[x] and xcd[kXcds + x].
enum XcdRow {
    kXcdStart = 0, kXcdCount = 1,
    kXcdLarge = 2,    // + 4 p: start, count of product p's large chunks
    kXcdSmall = 4,    // + 4 p: start, count of product p's small chunks
    kXcdRows = 10
};

// Scratch of the device-built plan, int32 indices into the aux section.
struct PlanAux {
    static constexpr int order(int e) { return e; }                        // experts by rank
    static constexpr int xcd_of(int n_expert, int e) { return n_expert + e; }   // XCD of expert e
    static constexpr int base_of(int n_expert, int e) { return 2 * n_expert + e; }  // first slot in its list
    static constexpr int status(int n_expert) { return 3 * n_expert; }     // ids out of range
    static constexpr int size(int n_expert) { return 3 * n_expert + 4; }
};

inline PlanLayout plan_layout(int tokens, int topk, int n_expert, int chunk_rows) {
    PlanLayout L{};
    const size_t R = size_t(tokens) * size_t(topk);
    size_t o = 0;
    L.perm = o;   o += align16(R * 4);
    L.inv = o;    o += align16(R * 4);
    L.chunks = o; o += align16(size_t(max_chunks(int(R), n_expert, chunk_rows)) * 16);
    L.xcd = o;    o += align16(size_t(kXcdRows * kXcds) * 4);
    L.gu_off = o; o += align16(size_t(n_expert) * 8);
    L.dn_off = o; o += align16(size_t(n_expert) * 8);
    L.counts = o; o += align16(size_t(n_expert + 1) * 4);
    L.offsets = o; o += align16(size_t(n_expert + 2) * 4);
    L.aux = o;    o += align16(size_t(PlanAux::size(n_expert)) * 4);
    L.tiles = o;  o += align16(size_t(n_expert + 1) * size_t(plan_n_tiles((long long)R)) * 4);
    L.total = o;
    return L;
}

// Arguments of one expert product launch (gate/up or down).
struct ProductArgs {
    const uint8_t *act;        // q8_1 rows in sorted order
    const uint8_t *w_base;     // weight buffer
    const uint64_t *w_off;     // device: expert byte offsets
    const int32_t *chunks;     // device: XCD-grouped chunk table
    const int32_t *xcd;        // device: per-XCD (start, count) rows of this launch's items
    const int32_t *xcd_small;  // device: the same for the small kernel's items
    const int32_t *perm;       // device: sorted row -> output row (NULL: identity)
    float *out;                // fp32 outputs
    uint8_t *hq;               // gate/up fused with swiglu: q8_1 rows of H (else NULL)
    int32_t *dots;             // debug: int32 block dots instead of outputs
    int wtype;                 // 1 Q2_0, 2 NL4
    int cols;                  // contraction length
    int out_rows;              // weight rows of one expert = output columns
    int n_tiles;               // ceil(out_rows / kTileRows)
    int max_items;             // items per XCD list (grid = kXcds * max_items)
    int dots_row_begin;
    int dots_n_rows;
    int small_rows;            // chunks of <= small_rows rows go to the small kernel (0: none)
    // Weight tiles per work item of the product kernel (0 or 1: one).  More
    // than one only for Q2_0 fp32 outputs (not the fused mode, not the block
    // dots), every N tile full (out_rows a multiple of kTileRows), the stage
    // count a multiple of kStreamStages and every chunk of at most 64 rows
    // (the launch takes it for short items only); an item's tiles then run as
    // one stream of stages.
    int group;
    int8_t codebook[16];
};

// Stages of prefetch of the product kernel's items of at most 64 rows, and
// what the stage count must be a multiple of for items of several tiles (it
// takes every prefetch depth of the Q2_0 items: 5 for these, 2 for larger).
constexpr int kStreamU = 5;
constexpr int kStreamStages = 10;

// Launchers (defined in the .hip files).  Return hipSuccess or the launch error.
hipError_t launch_quantize_scatter(const float *x, int tokens, int hidden, int topk,
                                   const int32_t *inv, uint8_t *xq, hipStream_t stream);
hipError_t launch_swiglu_q8(const float *gu, int rows, int n_ff, uint8_t *hq,
                            hipStream_t stream);
hipError_t launch_expert_product(const ProductArgs &args, hipStream_t stream);
// The same product for the items whose chunk has at most args.small_rows rows
// (one lane per weight row, int8 dot products); launch_expert_product skips them.
hipError_t launch_expert_small(const ProductArgs &args, hipStream_t stream);
// Rows a chunk may have to take the small kernel at this contraction length.
inline int small_rows_for(int cols) {
    const int lstride = int(align16(size_t(cols) + size_t(cols / 32) * 8));
    const int fit = kSmallActBytes / lstride;
    return fit < kMaxSmallRows ? fit : kMaxSmallRows;
}
// The plan built on the device from device routing ids (see plan_kernels.hip):
// the perm, inv, chunk, xcd, counts, offsets and aux sections of `ws`.
hipError_t launch_device_plan(const int32_t *ids, int rows, int n_expert, int chunk_rows,
                              int small_gu, int small_dn, uint8_t *ws, const PlanLayout &L,
                              hipStream_t stream);
// out[t] = sum over k of w[t*topk+k] * dm[t*topk+k] (fmaf, k ascending);
// the grid is tokens * ceil(hidden / 1024) workgroups of 256 threads.
hipError_t launch_combine(const float *dm, const float *w, int tokens, int topk, int hidden,
                          float *out, hipStream_t stream);
// The library's own plan workspace on each device (plan_scratch.hip), for
// plans built without caller memory: its size, and its device address on the
// current device (looked up once per device).
constexpr size_t kScratchBytes = size_t(4) << 20;
hipError_t scratch_workspace(void **ptr);
// Weight offset tables of experts at a constant stride, written on the device.
hipError_t launch_stride_offsets(uint64_t *gu_off, uint64_t gu_first, uint64_t gu_stride,
                                 uint64_t *dn_off, uint64_t dn_first, uint64_t dn_stride,
                                 int n_expert, hipStream_t stream);
// Packs n_expert matrices of rows x blocks_per_row blocks into the tiled
// layout; expert e's planes start at src/dst + e * expert_stride.  half > 0:
// the source rows alternate gate/up (2j gate j, 2j+1 up j, j < half) and the
// packed rows are in split order.  q2: Q2_0 blocks, whose codes are also
// rearranged within each block (weight_pack.hip).
hipError_t launch_weight_pack(const uint8_t *src, uint8_t *dst, uint64_t expert_stride,
                              int n_expert, int rows, int blocks_per_row, int half, bool q2,
                              hipStream_t stream);

}  // namespace moe
