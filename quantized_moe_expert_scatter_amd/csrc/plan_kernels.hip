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
//             (ties by id), dealt largest first to the XCD with the fewest
//             rows so far, and each XCD's list start and length;
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

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(const int32_t *ids, int rows,
                                                                  int n_expert, int32_t *counts) {
    const int i = blockIdx.x * kPlanThreads + threadIdx.x;
    if (i >= rows) return;
    int e = ids[i];
    if (e < 0 || e >= n_expert) e = n_expert;
    atomicAdd(&counts[e], 1);
}

// One workgroup.  Thread 0 does the two sequential passes (the prefix over
// E + 1 buckets and the greedy dealing, E steps each); the O(E^2) ranking is
// spread over the threads.
__global__ __launch_bounds__(kPlanThreads) void plan_schedule_kernel(const int32_t *counts,
                                                                     int n_expert, int chunk_rows,
                                                                     int32_t *offsets, int32_t *aux,
                                                                     int32_t *xcd_tab) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        int32_t run = 0;
        for (int b = 0; b <= n_expert; ++b) {
            offsets[b] = run;
            run += counts[b];
        }
        offsets[n_expert + 1] = run;
        aux[PlanAux::status(n_expert)] = counts[n_expert];
    }
    // rank of expert e: experts with more rows, or as many rows and a lower id
    for (int e = tid; e < n_expert; e += kPlanThreads) {
        const int32_t c = counts[e];
        int rank = 0;
        for (int f = 0; f < n_expert; ++f) {
            const int32_t cf = counts[f];
            rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
        }
        aux[PlanAux::order(rank)] = e;
    }
    __syncthreads();
    if (tid == 0) {
        long long load[kXcds] = {};
        int32_t listed[kXcds] = {};
        for (int r = 0; r < n_expert; ++r) {
            const int e = aux[PlanAux::order(r)];
            const int32_t c = counts[e];
            if (c == 0) {
                aux[PlanAux::xcd_of(n_expert, e)] = -1;
                aux[PlanAux::base_of(n_expert, e)] = 0;
                continue;
            }
            int x = 0;
            for (int k = 1; k < kXcds; ++k)
                if (load[k] < load[x]) x = k;
            load[x] += c;
            aux[PlanAux::xcd_of(n_expert, e)] = x;
            aux[PlanAux::base_of(n_expert, e)] = listed[x];
            listed[x] += (c + chunk_rows - 1) / chunk_rows;
        }
        int32_t start = 0;
        for (int x = 0; x < kXcds; ++x) {
            xcd_tab[x] = start;
            xcd_tab[kXcds + x] = listed[x];
            start += listed[x];
        }
    }
}

// Workgroup b collects the rows of bucket b (expert b, or the out-of-range ids
// for b == E) in ascending index order: each pass over 256 ids ranks the
// matches by a wave ballot and the waves' totals.
__global__ __launch_bounds__(kPlanThreads) void plan_scatter_kernel(const int32_t *ids, int rows,
                                                                    int n_expert,
                                                                    const int32_t *counts,
                                                                    const int32_t *offsets,
                                                                    int32_t *perm, int32_t *inv) {
    __shared__ int32_t wave_total[kPlanThreads / 64];
    const int b = blockIdx.x;
    const int32_t cnt = counts[b];
    if (cnt == 0) return;
    const int32_t base = offsets[b];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int32_t found = 0;
    for (int i0 = 0; i0 < rows && found < cnt; i0 += kPlanThreads) {
        const int i = i0 + tid;
        bool match = false;
        if (i < rows) {
            int e = ids[i];
            if (e < 0 || e >= n_expert) e = n_expert;
            match = e == b;
        }
        const uint64_t mask = __ballot(match);
        if (lane == 0) wave_total[wave] = __popcll(mask);
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kPlanThreads / 64; ++w) {
            before += w < wave ? wave_total[w] : 0;
            total += wave_total[w];
        }
        if (match) {
            const int32_t pos = found + before + __popcll(mask & below);
            if (pos < cnt) {
                perm[base + pos] = i;
                inv[i] = base + pos;
            }
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
                              uint8_t *ws, const PlanLayout &L, hipStream_t stream) {
    auto at = [&](size_t off) { return reinterpret_cast<int32_t *>(ws + off); };
    int32_t *perm = at(L.perm), *inv = at(L.inv), *chunks = at(L.chunks), *xcd = at(L.xcd);
    int32_t *counts = at(L.counts), *offsets = at(L.offsets), *aux = at(L.aux);
    const int maxc = max_chunks(rows, n_expert, chunk_rows);
    const int n_clear = max(n_expert + 1, 4 * maxc);
    const int n_pad = int(align16(size_t(rows) * 4) / 4) - rows;      // 0..3
    hipLaunchKernelGGL(plan_clear_kernel, dim3(blocks_for(n_clear)), dim3(kPlanThreads), 0, stream,
                       counts, n_expert + 1, chunks, 4 * maxc, perm + rows, inv + rows, n_pad);
    if (rows > 0)
        hipLaunchKernelGGL(plan_count_kernel, dim3(blocks_for(rows)), dim3(kPlanThreads), 0, stream,
                           ids, rows, n_expert, counts);
    hipLaunchKernelGGL(plan_schedule_kernel, dim3(1), dim3(kPlanThreads), 0, stream, counts, n_expert,
                       chunk_rows, offsets, aux, xcd);
    if (rows > 0)
        hipLaunchKernelGGL(plan_scatter_kernel, dim3(n_expert + 1), dim3(kPlanThreads), 0, stream, ids,
                           rows, n_expert, counts, offsets, perm, inv);
    hipLaunchKernelGGL(plan_chunks_kernel, dim3(blocks_for(n_expert)), dim3(kPlanThreads), 0, stream,
                       counts, offsets, aux, xcd, n_expert, chunk_rows, chunks, maxc);
    return hipGetLastError();
}

}  // namespace moe
