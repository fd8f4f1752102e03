// plan_kernels.hip -- the layer's plan built on the device from routing ids
// that already live there.
//
// The same plan moe_prefill_plan builds on the host ("Strata" PR #3752,
// commit list and Approach: each expert's rows made contiguous, the chunk
// table taken largest expert first, every expert at its own row count), byte
// for byte in the sections the kernels read:
//   1. clear  the counters and the chunk table (a fill kernel, no memset);
//   2. count  rows per expert with integer atomics; an id outside [0, E)
//             goes to an extra bucket E, which no product reads, and is
//             reported by the plan query;
//   3. one workgroup: offsets (exclusive prefix), experts ranked by row count
//             (ties by id) with a bitonic sort, dealt largest first to the XCD
//             with the fewest rows so far, each XCD's list start and length;
//   4. one workgroup per bucket: the bucket's rows in ascending t*K+k order by
//             a ballot compaction over all ids (stable, no atomics), writing
//             perm and its inverse;
//   5. one thread per expert: its chunks, in row order, into its XCD's list.
// All integer work: the result does not depend on scheduling.
#include "internal.h"

#include <hip/hip_runtime.h>

namespace moe {

namespace {

constexpr int kPlanThreads = 256;
static_assert(kXcds == 8, "the dealing's argmin tree assumes eight XCDs");

// Zeroes the counters, the chunk table and the alignment padding after perm
// and inv (a host-built plan's upload zeroes them too).
__global__ __launch_bounds__(kPlanThreads) void plan_clear_kernel(int32_t *counts, int n_counts,
                                                                  int32_t *chunks, int n_chunk_ints,
                                                                  int32_t *perm_pad, int32_t *inv_pad,
                                                                  int n_pad) {
    const int i = blockIdx.x * kPlanThreads + threadIdx.x;
    if (i < n_counts) counts[i] = 0;
    if (i < n_chunk_ints) chunks[i] = 0;
    if (i < n_pad) {
        perm_pad[i] = 0;
        inv_pad[i] = 0;
    }
}

// Rows per bucket: each workgroup counts 2048 ids into LDS bins, then adds
// its non-zero bins to the global counts (integer atomics: the totals do not
// depend on the order).
__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(const int32_t *ids, int rows,
                                                                  int n_expert, int32_t *counts) {
    constexpr int kPer = 8;
    __shared__ int32_t bins[kPlanMaxExperts + 1];
    const int tid = threadIdx.x;
    for (int e = tid; e <= n_expert; e += kPlanThreads) bins[e] = 0;
    __syncthreads();
    const int first = (blockIdx.x * kPlanThreads + tid) * kPer;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (first + j < rows) {
            int e = ids[first + j];
            if (e < 0 || e >= n_expert) e = n_expert;
            atomicAdd(&bins[e], 1);
        }
    __syncthreads();
    for (int e = tid; e <= n_expert; e += kPlanThreads)
        if (bins[e]) atomicAdd(&counts[e], bins[e]);
}

// One workgroup on the counts staged in LDS: the offsets by a parallel
// prefix, the ranking by a bitonic sort, then the greedy dealing, which is
// sequential in rank order: wave 0 runs it on rows and chunk counts gathered
// in rank order beforehand, and the results go back to memory in parallel.
__global__ __launch_bounds__(kPlanThreads) void plan_schedule_kernel(const int32_t *counts,
                                                                     int n_expert, int chunk_rows,
                                                                     int small_gu, int small_dn,
                                                                     int32_t *offsets, int32_t *aux,
                                                                     int32_t *xcd_tab) {
    __shared__ int32_t s_counts[kPlanMaxExperts + 1];
    __shared__ uint64_t s_key[kPlanMaxExperts];     // (rows descending, id) sort keys
    __shared__ int32_t s_rows[kPlanMaxExperts];     // rows of the expert of rank r, then its XCD
    __shared__ int32_t s_base[kPlanMaxExperts];     // its first slot in that XCD's list
    __shared__ int32_t s_wave[kPlanThreads / 64];
    __shared__ int32_t s_listed[3][kXcds];     // chunks, and the large ones of each product
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb = n_expert + 1;
    for (int b = tid; b < nb; b += kPlanThreads) s_counts[b] = counts[b];
    __syncthreads();

    // offsets: each thread a contiguous segment of buckets
    const int seg = (nb + kPlanThreads - 1) / kPlanThreads;
    const int lo = min(nb, tid * seg), hi = min(nb, lo + seg);
    int32_t local = 0;
    for (int b = lo; b < hi; ++b) local += s_counts[b];
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t up = __shfl_up(incl, d, 64);
        incl += lane >= d ? up : 0;
    }
    if (lane == 63) s_wave[wave] = incl;
    // experts ranked by rows descending, then id: a bitonic sort of the keys
    // (2^31 - 1 - rows) << 32 | id, padded to a power of two with the largest key
    int np2 = 1;
    while (np2 < n_expert) np2 <<= 1;
    for (int e = tid; e < np2; e += kPlanThreads)
        s_key[e] = e < n_expert ? (uint64_t(0x7FFFFFFFu - uint32_t(s_counts[e])) << 32) | uint32_t(e)
                                : ~0ull;
    __syncthreads();
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
    int32_t run = incl - local;
    for (int w = 0; w < wave; ++w) run += s_wave[w];
    for (int b = lo; b < hi; ++b) {
        offsets[b] = run;
        run += s_counts[b];
    }
    if (tid == kPlanThreads - 1) offsets[nb] = run;
    if (tid == 0) aux[PlanAux::status(n_expert)] = s_counts[n_expert];
    for (int r = tid; r < n_expert; r += kPlanThreads) s_rows[r] = s_counts[uint32_t(s_key[r])];
    __syncthreads();

    if (wave == 0) {
        // lane x < 8 holds XCD x's rows so far and its list length; a step
        // takes the first XCD of least rows as the least (rows << 3 | x) key
        // of lanes 0..7, by three DPP shifts of a prefix minimum
        uint32_t load = lane < kXcds ? 0u : 0x1FFFFFFFu;
        int32_t listed = 0, large_gu = 0, large_dn = 0;
        for (int r0 = 0; r0 < n_expert; r0 += 64) {
            const int n = min(64, n_expert - r0);
            const int32_t cvec = lane < n ? s_rows[r0 + lane] : 0;
            const int32_t nvec = (cvec + chunk_rows - 1) / chunk_rows;
            int32_t xs = -1, bases = 0;
            for (int j = 0; j < n; ++j) {
                const int32_t c = __builtin_amdgcn_readlane(cvec, j);
                if (c == 0) break;                  // ranks past here have no rows
                uint32_t key = (load << 3) | uint32_t(lane & 7);
                key = min(key, uint32_t(__builtin_amdgcn_update_dpp(int(key), int(key), 0x111, 0xF, 0xF, false)));
                key = min(key, uint32_t(__builtin_amdgcn_update_dpp(int(key), int(key), 0x112, 0xF, 0xF, false)));
                key = min(key, uint32_t(__builtin_amdgcn_update_dpp(int(key), int(key), 0x114, 0xF, 0xF, false)));
                const int x = __builtin_amdgcn_readlane(int(key), 7) & 7;
                const int32_t base = __builtin_amdgcn_readlane(listed, x);
                const int32_t nch = __builtin_amdgcn_readlane(nvec, j);
                const bool mine = lane == x;            // no branch: both adds run
                load += mine ? uint32_t(c) : 0u;
                listed += mine ? nch : 0;
                large_gu += mine && c > small_gu ? nch : 0;
                large_dn += mine && c > small_dn ? nch : 0;
                xs = lane == j ? x : xs;
                bases = lane == j ? base : bases;
            }
            if (lane < n) {
                s_rows[r0 + lane] = cvec == 0 ? -1 : xs;
                s_base[r0 + lane] = cvec == 0 ? 0 : bases;
            }
        }
        if (lane < kXcds) {
            s_listed[0][lane] = listed;
            s_listed[1][lane] = large_gu;
            s_listed[2][lane] = large_dn;
        }
    }
    __syncthreads();
    for (int r = tid; r < n_expert; r += kPlanThreads) {
        const int e = int(uint32_t(s_key[r]));
        aux[PlanAux::order(r)] = e;
        aux[PlanAux::xcd_of(n_expert, e)] = s_rows[r];
        aux[PlanAux::base_of(n_expert, e)] = s_base[r];
    }
    if (tid == 0) {
        int32_t start = 0;
        for (int x = 0; x < kXcds; ++x) {
            const int32_t cnt = s_listed[0][x];
            xcd_tab[kXcdStart * kXcds + x] = start;
            xcd_tab[kXcdCount * kXcds + x] = cnt;
            for (int q = 0; q < 2; ++q) {
                const int32_t large = s_listed[1 + q][x];
                xcd_tab[(kXcdLarge + 4 * q) * kXcds + x] = start;
                xcd_tab[(kXcdLarge + 4 * q + 1) * kXcds + x] = large;
                xcd_tab[(kXcdSmall + 4 * q) * kXcds + x] = start + large;
                xcd_tab[(kXcdSmall + 4 * q + 1) * kXcds + x] = cnt - large;
            }
            start += cnt;
        }
    }
}

// Workgroup b collects the rows of bucket b (expert b, or the out-of-range ids
// for b == E) in ascending index order.  Each pass covers 2048 ids, eight
// consecutive ones per thread: a thread's matches are numbered after those of
// the threads before it (a wave prefix sum by shuffles, then the waves' totals).
__global__ __launch_bounds__(kPlanThreads) void plan_scatter_kernel(const int32_t *ids, int rows,
                                                                    int n_expert,
                                                                    const int32_t *counts,
                                                                    const int32_t *offsets,
                                                                    int32_t *perm, int32_t *inv) {
    constexpr int kPer = 8;
    __shared__ int32_t wave_total[kPlanThreads / 64];
    const int b = blockIdx.x;
    const int32_t cnt = counts[b];
    if (cnt == 0) return;
    const int32_t base = offsets[b];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    int32_t found = 0;
    for (int i0 = 0; i0 < rows && found < cnt; i0 += kPer * kPlanThreads) {
        const int first = i0 + kPer * tid;
        int e[kPer];
        if (first + kPer <= rows) {
            const int4 v0 = *reinterpret_cast<const int4 *>(ids + first);
            const int4 v1 = *reinterpret_cast<const int4 *>(ids + first + 4);
            e[0] = v0.x; e[1] = v0.y; e[2] = v0.z; e[3] = v0.w;
            e[4] = v1.x; e[5] = v1.y; e[6] = v1.z; e[7] = v1.w;
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) e[j] = first + j < rows ? ids[first + j] : -1;
        }
        unsigned bits = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            int ej = e[j];
            if (ej < 0 || ej >= n_expert) ej = n_expert;
            bits |= (first + j < rows && ej == b) ? (1u << j) : 0u;
        }
        const int mine = __popc(bits);
        int incl = mine;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int up = __shfl_up(incl, d, 64);
            incl += lane >= d ? up : 0;
        }
        if (lane == 63) wave_total[wave] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kPlanThreads / 64; ++w) {
            before += w < wave ? wave_total[w] : 0;
            total += wave_total[w];
        }
        int32_t pos = found + before + incl - mine;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (bits & (1u << j)) {
                if (pos < cnt) {
                    perm[base + pos] = first + j;
                    inv[first + j] = base + pos;
                }
                ++pos;
            }
        found += total;
        __syncthreads();          // wave_total is rewritten by the next pass
    }
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
    int32_t *counts = at(L.counts), *offsets = at(L.offsets), *aux = at(L.aux);
    const int maxc = max_chunks(rows, n_expert, chunk_rows);
    const int n_clear = max(n_expert + 1, 4 * maxc);
    const int n_pad = int(align16(size_t(rows) * 4) / 4) - rows;      // 0..3
    hipLaunchKernelGGL(plan_clear_kernel, dim3(blocks_for(n_clear)), dim3(kPlanThreads), 0, stream,
                       counts, n_expert + 1, chunks, 4 * maxc, perm + rows, inv + rows, n_pad);
    if (rows > 0)
        hipLaunchKernelGGL(plan_count_kernel, dim3(blocks_for((rows + 7) / 8)), dim3(kPlanThreads), 0,
                           stream, ids, rows, n_expert, counts);
    hipLaunchKernelGGL(plan_schedule_kernel, dim3(1), dim3(kPlanThreads), 0, stream, counts, n_expert,
                       chunk_rows, small_gu, small_dn, offsets, aux, xcd);
    if (rows > 0)
        hipLaunchKernelGGL(plan_scatter_kernel, dim3(n_expert + 1), dim3(kPlanThreads), 0, stream, ids,
                           rows, n_expert, counts, offsets, perm, inv);
    hipLaunchKernelGGL(plan_chunks_kernel, dim3(blocks_for(n_expert)), dim3(kPlanThreads), 0, stream,
                       counts, offsets, aux, xcd, n_expert, chunk_rows, chunks, maxc);
    return hipGetLastError();
}

}  // namespace moe
