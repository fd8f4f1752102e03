// plan_kernels.hip -- the layer's plan built on the device from routing ids
// that already live there.
//
// The same plan moe_prefill_plan builds on the host ("Strata" PR #3752,
// commit list and Approach: each expert's rows made contiguous, the chunk
// table taken largest expert first, every expert at its own row count), byte
// for byte in the sections the kernels read.  The routing ids are cut into
// tiles of consecutive ids (a multiple of 2048, at most kPlanMaxTiles tiles):
//   1. count  one workgroup per tile: the tile's rows per bucket (expert e,
//             or bucket E for an id outside [0, E), which no product reads and
//             the plan query reports), binned in LDS and written whole, no
//             global atomics; the same launch clears the chunk table (a fill,
//             no memset);
//   2. scan   one wave per bucket: its rows in the tiles before each tile
//             (exclusive prefix down the bucket's column) and its total;
//   3. one launch of two roles that need only the counts:
//        block 0   offsets (exclusive prefix), experts ranked by row count
//                  (ties by id) with a bitonic sort, dealt largest first to
//                  the XCD with the fewest rows so far, each XCD's list;
//        block 1+t the rows of tile t in ascending t*K+k order within each
//                  bucket (stable): a row's place is its bucket's offset, the
//                  bucket's rows in earlier tiles, earlier waves and earlier
//                  lanes of the tile; lanes of one bucket find each other by
//                  ballots over the bucket's bits.  Writes perm and its inverse;
//   4. one thread per expert: its chunks, in row order, into its XCD's list.
// All integer work: the result does not depend on scheduling.
#include "internal.h"

#include <hip/hip_runtime.h>

#include <type_traits>

namespace moe {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPer = kPlanPassIds / kPlanThreads;      // ids per thread and pass
constexpr int kBuckets = kPlanMaxExperts + 4;          // LDS stride of a bucket array
static_assert(kXcds == 8, "the dealing's 8-lane butterfly assumes eight XCDs");
static_assert(kPer == 8, "a pass is eight ids per thread");

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ int bucket_of(int e, int n_expert) {
    return (e < 0 || e >= n_expert) ? n_expert : e;
}

// Rows per bucket of tile t, and the chunk table and the alignment padding
// after perm and inv cleared (a host-built plan's upload zeroes them too).
__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(const int32_t *ids, int rows,
                                                                  int n_expert, int tile_ids,
                                                                  int n_tiles, int32_t *tiles,
                                                                  int32_t *chunks, int n_chunk_ints,
                                                                  int32_t *perm_pad, int32_t *inv_pad,
                                                                  int n_pad) {
    __shared__ int32_t bins[kBuckets];
    const int tid = threadIdx.x;
    const int t = blockIdx.x;
    const int nb = n_expert + 1;
    for (int i = t * kPlanThreads + tid; i < n_chunk_ints; i += n_tiles * kPlanThreads) chunks[i] = 0;
    if (t == 0 && tid < n_pad) {
        perm_pad[tid] = 0;
        inv_pad[tid] = 0;
    }
    for (int b = tid; b < nb; b += kPlanThreads) bins[b] = 0;
    __syncthreads();
    const long long begin = (long long)t * tile_ids;
    const int end = int(min((long long)rows, begin + tile_ids));
    for (int first = int(begin) + kPer * tid; first < end; first += kPlanPassIds) {
        int e[kPer];
        if (first + kPer <= end) {
            const int4 v0 = *reinterpret_cast<const int4 *>(ids + first);
            const int4 v1 = *reinterpret_cast<const int4 *>(ids + first + 4);
            e[0] = v0.x; e[1] = v0.y; e[2] = v0.z; e[3] = v0.w;
            e[4] = v1.x; e[5] = v1.y; e[6] = v1.z; e[7] = v1.w;
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) e[j] = first + j < end ? ids[first + j] : 0;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (first + j < end) atomicAdd(&bins[bucket_of(e[j], n_expert)], 1);
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kPlanThreads) tiles[size_t(b) * n_tiles + t] = bins[b];
}

__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t up = __shfl_up(v, d, 64);
        v += lane >= d ? up : 0;
    }
    return v;
}

// Wave b (of the launch) takes bucket b: its rows in tiles 0..t-1 replace its
// count of tile t, and the total goes to counts[b].
__global__ __launch_bounds__(kPlanThreads) void plan_scan_kernel(int32_t *tiles, int n_tiles, int nb,
                                                                 int32_t *counts) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kPlanWaves + (threadIdx.x >> 6);
    if (b >= nb) return;
    int32_t *col = tiles + size_t(b) * n_tiles;
    int32_t run = 0;
    for (int t0 = 0; t0 < n_tiles; t0 += 64) {
        const int t = t0 + lane;
        const int32_t v = t < n_tiles ? col[t] : 0;
        const int32_t incl = wave_inclusive_sum(v, lane);
        if (t < n_tiles) col[t] = run + incl - v;
        run += __shfl(incl, 63, 64);
    }
    if (lane == 0) counts[b] = run;
}

// s[0..nb) (LDS, the counts) becomes its exclusive prefix; returns the total.
// Every thread takes a contiguous segment of buckets.
__device__ int32_t block_exclusive_prefix(int32_t *s, int nb, int32_t *s_wave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = (nb + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(nb, tid * seg), hi = min(nb, lo + seg);
    int32_t local = 0;
    for (int b = lo; b < hi; ++b) local += s[b];
    const int32_t incl = wave_inclusive_sum(local, lane);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int32_t run = incl - local, total = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
        run += w < wave ? s_wave[w] : 0;
        total += s_wave[w];
    }
    for (int b = lo; b < hi; ++b) {
        const int32_t v = s[b];
        s[b] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

// The scheduling role: offsets, the ranking, the dealing, the XCD table.
__device__ void plan_schedule(uint8_t *smem, const int32_t *counts, int n_expert, int chunk_rows,
                              int small_gu, int small_dn, int32_t *offsets, int32_t *aux,
                              int32_t *xcd_tab) {
    int32_t *s_counts = reinterpret_cast<int32_t *>(smem);                // [nb] counts
    int32_t *s_off = s_counts + kBuckets;                                  // [nb] offsets
    uint64_t *s_key = reinterpret_cast<uint64_t *>(s_off + kBuckets);      // [np2] sort keys
    int32_t *s_xcd = reinterpret_cast<int32_t *>(s_key + kPlanMaxExperts); // [E] XCD of rank r
    int32_t *s_base = s_xcd + kPlanMaxExperts;                             // [E] its first slot
    __shared__ int32_t s_wave[kPlanWaves];
    __shared__ int32_t s_part[kXcds][kPlanWaves];
    __shared__ int32_t s_listed[3][kXcds];      // chunks, and the large ones of each product
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = n_expert + 1;
    for (int b = tid; b < nb; b += kPlanThreads) s_counts[b] = s_off[b] = counts[b];
    if (tid < 3 * kXcds) s_listed[tid / kXcds][tid % kXcds] = 0;
    // experts ranked by rows descending, then id: a bitonic sort of the keys
    // (2^31 - 1 - rows) << 32 | id, padded to a power of two with the largest key
    int np2 = 1;
    while (np2 < n_expert) np2 <<= 1;
    __syncthreads();
    for (int e = tid; e < np2; e += kPlanThreads)
        s_key[e] = e < n_expert ? (uint64_t(0x7FFFFFFFu - uint32_t(s_counts[e])) << 32) | uint32_t(e)
                                : ~0ull;
    const int32_t total = block_exclusive_prefix(s_off, nb, s_wave);
    for (int b = tid; b < nb; b += kPlanThreads) offsets[b] = s_off[b];
    if (tid == 0) {
        offsets[nb] = total;
        aux[PlanAux::status(n_expert)] = s_counts[n_expert];
    }
    for (int k = 2; k <= np2; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < np2; i += kPlanThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t a = s_key[i], b = s_key[ixj];
                    if ((a > b) == ((i & k) == 0)) {
                        s_key[i] = b;
                        s_key[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }

    // the greedy dealing, sequential in rank order, on wave 0: lane x < 8
    // holds key = (XCD x's rows so far) << 3 | x; a step finds the least key
    // of lanes 0..7 by an 8-lane butterfly (two quad permutes and a half-row
    // mirror), the lane that holds it adds the expert's rows (<< 3), and lane
    // r of the wave records the XCD of rank r0 + r.  The butterfly never
    // crosses an 8-lane group, so what lanes 8..63 hold does not matter.
    if (wave == 0) {
        uint32_t key = uint32_t(lane & 7);
        for (int r0 = 0; r0 < n_expert; r0 += 64) {
            const int n = min(64, n_expert - r0);
            const int32_t cvec = lane < n ? s_counts[uint32_t(s_key[r0 + lane])] : 0;
            const uint32_t c8 = uint32_t(cvec) << 3;
            int32_t xs = -1;
            static_for<0, 64>([&](auto J) {
                constexpr int j = decltype(J)::value;
                const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(c8), j));
                uint32_t m = key;
                m = min(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0xB1, 0xF, 0xF, false)));
                m = min(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x4E, 0xF, 0xF, false)));
                m = min(m, uint32_t(__builtin_amdgcn_update_dpp(0, int(m), 0x141, 0xF, 0xF, false)));
                key += key == m ? c : 0u;
                const int x = __builtin_amdgcn_readfirstlane(int(m)) & 7;
                xs = lane == j ? x : xs;
            });
            if (lane < n) s_xcd[r0 + lane] = cvec == 0 ? -1 : xs;
        }
    }
    __syncthreads();

    // each XCD's list in rank order: an expert's first slot is the chunks of
    // the earlier ranks dealt to the same XCD (a scan per XCD over ranks, each
    // thread a contiguous segment), and the list totals
    const int seg = (n_expert + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(n_expert, tid * seg), hi = min(n_expert, lo + seg);
    int32_t local[kXcds];
#pragma unroll
    for (int x = 0; x < kXcds; ++x) local[x] = 0;
    for (int r = lo; r < hi; ++r) {
        const int x = s_xcd[r];
        const int32_t c = s_counts[uint32_t(s_key[r])];
        const int32_t nch = (c + chunk_rows - 1) / chunk_rows;
#pragma unroll
        for (int X = 0; X < kXcds; ++X) local[X] += x == X ? nch : 0;
        if (x >= 0) {
            if (c > small_gu) atomicAdd(&s_listed[1][x], nch);
            if (c > small_dn) atomicAdd(&s_listed[2][x], nch);
        }
    }
    int32_t run[kXcds];
#pragma unroll
    for (int x = 0; x < kXcds; ++x) {
        run[x] = wave_inclusive_sum(local[x], lane);
        if (lane == 63) s_part[x][wave] = run[x];
        run[x] -= local[x];
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kXcds; ++x) {
        int32_t before = 0, sum = 0;
#pragma unroll
        for (int w = 0; w < kPlanWaves; ++w) {
            before += w < wave ? s_part[x][w] : 0;
            sum += s_part[x][w];
        }
        run[x] += before;
        if (tid == 0) s_listed[0][x] = sum;
    }
    for (int r = lo; r < hi; ++r) {
        const int x = s_xcd[r];
        const int32_t c = s_counts[uint32_t(s_key[r])];
        const int32_t nch = (c + chunk_rows - 1) / chunk_rows;
        int32_t base = 0;
#pragma unroll
        for (int X = 0; X < kXcds; ++X) {
            base = x == X ? run[X] : base;
            run[X] += x == X ? nch : 0;
        }
        s_base[r] = base;
    }
    __syncthreads();
    for (int r = tid; r < n_expert; r += kPlanThreads) {
        const int e = int(uint32_t(s_key[r]));
        aux[PlanAux::order(r)] = e;
        aux[PlanAux::xcd_of(n_expert, e)] = s_xcd[r];
        aux[PlanAux::base_of(n_expert, e)] = s_base[r];
    }
    if (tid == 0) {
        // a few small experts beside large ones join the product kernel's
        // view (the rule of the host plan)
        bool fold[2];
        for (int q = 0; q < 2; ++q) {
            int32_t tot_small = 0, tot_large = 0;
            for (int x = 0; x < kXcds; ++x) {
                tot_large += s_listed[1 + q][x];
                tot_small += s_listed[0][x] - s_listed[1 + q][x];
            }
            fold[q] = tot_small < kSmallMinChunks && tot_large > 0;
        }
        int32_t start = 0;
        for (int x = 0; x < kXcds; ++x) {
            const int32_t cnt = s_listed[0][x];
            xcd_tab[kXcdStart * kXcds + x] = start;
            xcd_tab[kXcdCount * kXcds + x] = cnt;
            for (int q = 0; q < 2; ++q) {
                const int32_t large = fold[q] ? cnt : s_listed[1 + q][x];
                xcd_tab[(kXcdLarge + 4 * q) * kXcds + x] = start;
                xcd_tab[(kXcdLarge + 4 * q + 1) * kXcds + x] = large;
                xcd_tab[(kXcdSmall + 4 * q) * kXcds + x] = start + large;
                xcd_tab[(kXcdSmall + 4 * q + 1) * kXcds + x] = cnt - large;
            }
            start += cnt;
        }
    }
}

// The scatter role for tile t.  A pass is 2048 ids: wave w takes ids
// 512 w .. 512 w + 511 of it, lane l id 64 i + l of those in round i.  The
// waves first count their ids per bucket, which gives each wave's first place
// in each bucket; then round by round a lane's place is that of its wave plus
// the lanes below it with the same bucket, and the bucket's last lane moves
// the wave's place on.
__device__ void plan_scatter(uint8_t *smem, const int32_t *ids, int rows, int n_expert, int tile_ids,
                             int n_tiles, int t, const int32_t *counts, const int32_t *tiles,
                             int32_t *perm, int32_t *inv) {
    int32_t *pos = reinterpret_cast<int32_t *>(smem);      // [nb] the tile's next place per bucket
    int32_t *wpos = pos + kBuckets;                         // [kPlanWaves][nb] per wave
    __shared__ int32_t s_wave[kPlanWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = n_expert + 1;
    for (int b = tid; b < nb; b += kPlanThreads) pos[b] = counts[b];
    __syncthreads();
    block_exclusive_prefix(pos, nb, s_wave);
    for (int b = tid; b < nb; b += kPlanThreads) pos[b] += tiles[size_t(b) * n_tiles + t];
    int nbits = 0;                    // bits of the largest bucket, n_expert
    while ((n_expert >> nbits) != 0) ++nbits;
    const uint64_t below = (uint64_t(1) << lane) - 1u;
    int32_t *mine = wpos + wave * kBuckets;
    const long long begin = (long long)t * tile_ids;
    const int end = int(min((long long)rows, begin + tile_ids));
    for (int p0 = int(begin); p0 < end; p0 += kPlanPassIds) {
        for (int b = lane; b < nb; b += 64) mine[b] = 0;
        const int w0 = p0 + 512 * wave;
        int e[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = w0 + 64 * i + lane;
            e[i] = idx < end ? bucket_of(ids[idx], n_expert) : -1;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (e[i] >= 0) atomicAdd(&mine[e[i]], 1);
        __syncthreads();
        for (int b = tid; b < nb; b += kPlanThreads) {
            int32_t p = pos[b];
#pragma unroll
            for (int w = 0; w < kPlanWaves; ++w) {
                const int32_t c = wpos[w * kBuckets + b];
                wpos[w * kBuckets + b] = p;
                p += c;
            }
            pos[b] = p;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const bool valid = e[i] >= 0;
            uint64_t peers = __ballot(valid);
            for (int k = 0; k < nbits; ++k) {
                const bool bit = ((e[i] >> k) & 1) != 0;
                const uint64_t set = __ballot(bit);
                peers &= bit ? set : ~set;
            }
            if (valid) {
                const int b = e[i];
                const int32_t p = mine[b] + int32_t(__popcll(peers & below));
                const int idx = w0 + 64 * i + lane;
                perm[p] = idx;
                inv[idx] = p;
                if ((peers >> lane) == 1u) mine[b] = p + 1;     // the bucket's last lane
            }
        }
        __syncthreads();          // the wave arrays are rewritten by the next pass
    }
}

constexpr size_t kScheduleLds = size_t(kBuckets) * 8 + size_t(kPlanMaxExperts) * 16;
constexpr size_t kScatterLds = size_t(kBuckets) * 4 * (1 + kPlanWaves);
constexpr size_t kBuildLds = kScheduleLds > kScatterLds ? kScheduleLds : kScatterLds;

// Block 0 schedules; block 1 + t scatters tile t.  Both read only the counts
// and the scanned tiles, so they run side by side.
__global__ __launch_bounds__(kPlanThreads) void plan_build_kernel(
    const int32_t *ids, int rows, int n_expert, int chunk_rows, int small_gu, int small_dn,
    int tile_ids, int n_tiles, const int32_t *counts, const int32_t *tiles, int32_t *offsets,
    int32_t *aux, int32_t *xcd_tab, int32_t *perm, int32_t *inv) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kBuildLds];
    if (blockIdx.x == 0)
        plan_schedule(smem, counts, n_expert, chunk_rows, small_gu, small_dn, offsets, aux, xcd_tab);
    else
        plan_scatter(smem, ids, rows, n_expert, tile_ids, n_tiles, int(blockIdx.x) - 1, counts, tiles,
                     perm, inv);
}

__global__ __launch_bounds__(kPlanThreads) void plan_chunks_kernel(const int32_t *counts,
                                                                   const int32_t *offsets,
                                                                   const int32_t *aux,
                                                                   const int32_t *xcd_tab,
                                                                   int n_expert, int chunk_rows,
                                                                   int32_t *chunks, int max_chunks) {
    const int e = blockIdx.x * kPlanThreads + threadIdx.x;
    if (e >= n_expert) return;
    const int32_t c = counts[e];
    if (c == 0) return;
    const int x = aux[PlanAux::xcd_of(n_expert, e)];
    if (x < 0 || x >= kXcds) return;
    const int32_t first = xcd_tab[x] + aux[PlanAux::base_of(n_expert, e)];
    for (int32_t r0 = 0, j = 0; r0 < c; r0 += chunk_rows, ++j) {
        const int32_t idx = first + j;
        if (idx < 0 || idx >= max_chunks) break;
        int32_t *dst = chunks + 4 * size_t(idx);
        dst[0] = e;
        dst[1] = offsets[e] + r0;
        dst[2] = min(chunk_rows, c - r0);
        dst[3] = 0;
    }
}

unsigned blocks_for(long long n) { return unsigned((n + kPlanThreads - 1) / kPlanThreads); }

}  // namespace

hipError_t launch_device_plan(const int32_t *ids, int rows, int n_expert, int chunk_rows,
                              int small_gu, int small_dn, uint8_t *ws, const PlanLayout &L,
                              hipStream_t stream) {
    auto at = [&](size_t off) { return reinterpret_cast<int32_t *>(ws + off); };
    int32_t *perm = at(L.perm), *inv = at(L.inv), *chunks = at(L.chunks), *xcd = at(L.xcd);
    int32_t *counts = at(L.counts), *offsets = at(L.offsets), *aux = at(L.aux), *tiles = at(L.tiles);
    const int maxc = max_chunks(rows, n_expert, chunk_rows);
    const int n_pad = int(align16(size_t(rows) * 4) / 4) - rows;      // 0..3
    const int tile_ids = plan_tile_ids(rows);
    const int n_tiles = plan_n_tiles(rows);
    const int nb = n_expert + 1;
    hipLaunchKernelGGL(plan_count_kernel, dim3(n_tiles), dim3(kPlanThreads), 0, stream, ids, rows,
                       n_expert, tile_ids, n_tiles, tiles, chunks, 4 * maxc, perm + rows, inv + rows,
                       n_pad);
    hipLaunchKernelGGL(plan_scan_kernel, dim3((nb + kPlanWaves - 1) / kPlanWaves), dim3(kPlanThreads), 0,
                       stream, tiles, n_tiles, nb, counts);
    hipLaunchKernelGGL(plan_build_kernel, dim3(1 + (rows > 0 ? n_tiles : 0)), dim3(kPlanThreads), 0,
                       stream, ids, rows, n_expert, chunk_rows, small_gu, small_dn, tile_ids, n_tiles,
                       counts, tiles, offsets, aux, xcd, perm, inv);
    hipLaunchKernelGGL(plan_chunks_kernel, dim3(blocks_for(n_expert)), dim3(kPlanThreads), 0, stream,
                       counts, offsets, aux, xcd, n_expert, chunk_rows, chunks, maxc);
    return hipGetLastError();
}

}  // namespace moe
