// moe_prefill.cpp -- host side of the C ABI: argument validation, the plan
// (counting sort, chunk table, XCD work lists), its upload, and the launches.
//
// "Strata" PR #3752 (commit list, Approach): the experts' rows are made
// contiguous by quantize_scatter, the layer's expert offsets and the CTAs'
// chunk table go up to the device together with the group bounds, and each
// product runs as one launch over all experts, chunks taken largest expert
// first, each expert at its own row count.
#include "../../include/moe_prefill.h"
#include "internal.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <vector>

using namespace moe;

struct moe_plan {
    int tokens = 0, topk = 0, n_expert = 0, chunk_rows = 0, rows = 0;
    int hidden = 0, n_ff = 0;
    int max_chunk_rows = 0;      // rows of the largest chunk (a bound for device-built plans)
    moe_weights gu{}, dn{};
    std::vector<uint64_t> gu_off, dn_off;
    int8_t gu_codebook[16] = {}, dn_codebook[16] = {};
    std::vector<int32_t> counts, offsets, perm, inv, chunks, dev_chunks;
    int32_t xcd_tab[kXcdRows * kXcds] = {};
    int n_chunks = 0;
    long long max_xcd_chunks = 0;
    long long max_large[2] = {0, 0}, max_small[2] = {0, 0};   // per product: longest list of each view
    bool device_built = false;   // sorted maps and chunk lists built on the device
    bool in_scratch = false;     // built in the library's per-device workspace: not freed
    hipStream_t stream = nullptr;  // the stream a plan without an upload event was built on
    void *plan_dev = nullptr;
    PlanLayout layout{};
    void *staging = nullptr;     // pinned, from the staging pool
    size_t staging_cap = 0;
    hipEvent_t uploaded = nullptr;
};

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the block format of a weight type, without the layout flags
int base_type(int type) { return type & ~int(MOE_W_TILED | MOE_W_GU_INTERLEAVED); }

int block_values(int type) {
    const int t = base_type(type);
    return t == MOE_W_Q2_0 ? 64 : (t == MOE_W_NL4 ? 32 : 0);
}

size_t weight_bytes(int type, int rows, int cols) {
    const int blk = block_values(type);
    if (blk == 0 || rows <= 0 || cols <= 0 || cols % blk) return 0;
    return size_t(rows) * size_t(cols / blk) * 18u;
}

// Shape, alignment and extent of a weight descriptor.  `tiled`: the layout
// flag the caller must (1) or must not (0) have set.
int check_weights(const moe_weights *w, int n_expert, bool tiled) {
    if (!w || !w->base || !w->offset) return MOE_EINVAL;
    const int t = base_type(w->type);
    if (t != MOE_W_Q2_0 && t != MOE_W_NL4) return MOE_EFORMAT;
    if (((w->type & MOE_W_TILED) != 0) != tiled) return MOE_EFORMAT;
    // alternating gate/up rows are a storage order the pack undoes
    if (tiled && (w->type & MOE_W_GU_INTERLEAVED)) return MOE_EFORMAT;
    if (w->n_expert != n_expert || w->rows <= 0 || w->cols <= 0) return MOE_EINVAL;
    if (w->rows % 64 || w->cols % block_values(t)) return MOE_EFORMAT;
    if (t == MOE_W_NL4 && !w->codebook) return MOE_EINVAL;
    if (!aligned16(w->base)) return MOE_EALIGN;
    const size_t per = weight_bytes(t, w->rows, w->cols);
    // the kernels address inside one expert with 32-bit offsets
    if (per >= (size_t(1) << 31)) return MOE_EINVAL;
    for (int e = 0; e < n_expert; ++e) {
        if (w->offset[e] & 15u) return MOE_EALIGN;
        if (w->offset[e] > w->base_bytes || w->base_bytes - w->offset[e] < per) return MOE_ESIZE;
    }
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace

namespace {

// Argument checks shared by the host- and device-built plans.
int check_plan_args(int tokens, int topk, int n_expert, int chunk_rows, const moe_weights *w_gu,
                    const moe_weights *w_down) {
    if (tokens < 0 || topk <= 0 || n_expert <= 0 || chunk_rows <= 0 || chunk_rows > kMaxChunkRows)
        return MOE_EINVAL;
    if ((long long)tokens * topk > (1LL << 30)) return MOE_EINVAL;
    int st = check_weights(w_gu, n_expert, true);
    if (st) return st;
    st = check_weights(w_down, n_expert, true);
    if (st) return st;
    if (w_gu->rows % 2 || w_down->rows != w_gu->cols || w_down->cols * 2 != w_gu->rows)
        return MOE_EINVAL;
    return MOE_OK;
}

// A plan under construction: destroyed (waiting for its upload) unless released.
struct PlanDeleter {
    void operator()(moe_plan *p) const { moe_plan_destroy(p); }
};
using PlanPtr = std::unique_ptr<moe_plan, PlanDeleter>;

// Host allocations here and below throw std::bad_alloc when memory runs out;
// the exported functions turn that into MOE_ENOMEM (guarded, below).
PlanPtr new_plan(int tokens, int topk, int n_expert, int chunk_rows, const moe_weights *w_gu,
                 const moe_weights *w_down) {
    PlanPtr p(new moe_plan);
    p->tokens = tokens; p->topk = topk; p->n_expert = n_expert; p->chunk_rows = chunk_rows;
    p->max_chunk_rows = chunk_rows;
    p->rows = tokens * topk; p->hidden = w_gu->cols; p->n_ff = w_gu->rows / 2;
    p->gu = *w_gu; p->dn = *w_down;
    p->gu_off.assign(w_gu->offset, w_gu->offset + n_expert);
    p->dn_off.assign(w_down->offset, w_down->offset + n_expert);
    if (base_type(w_gu->type) == MOE_W_NL4) std::memcpy(p->gu_codebook, w_gu->codebook, 16);
    if (base_type(w_down->type) == MOE_W_NL4) std::memcpy(p->dn_codebook, w_down->codebook, 16);
    p->gu.offset = p->gu_off.data();
    p->dn.offset = p->dn_off.data();
    p->gu.codebook = p->gu_codebook;
    p->dn.codebook = p->dn_codebook;
    p->layout = plan_layout(tokens, topk, n_expert, chunk_rows);
    return p;
}

// Every product launch over the plan fits one HIP grid: the longest list of
// each product's two views times that product's N tiles (the fused gate/up
// takes 128-j tiles), kXcds workgroups of kProductThreads threads per item.
bool grids_fit(const moe_plan *p) {
    const long long gu_tiles = std::max<long long>((2LL * p->n_ff + kTileRows - 1) / kTileRows,
                                                   (p->n_ff + kTileRows / 2 - 1) / (kTileRows / 2));
    const long long tiles[2] = {gu_tiles, (p->hidden + kTileRows - 1) / kTileRows};
    for (int q = 0; q < 2; ++q) {
        const long long items = std::max(p->max_large[q], p->max_small[q]) * tiles[q];
        if (items * kXcds * kProductThreads > kMaxLaunchThreads) return false;
    }
    return true;
}

// Experts largest first, ties by lower id.
std::vector<int> expert_order(const std::vector<int32_t> &counts) {
    std::vector<int> order(counts.size());
    for (size_t e = 0; e < counts.size(); ++e) order[e] = int(e);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return counts[a] > counts[b]; });
    return order;
}

// Chunks (expert, first row, rows, 0) of the experts in `order`, each in row order.
std::vector<int32_t> chunk_list(const std::vector<int> &order, const std::vector<int32_t> &counts,
                                const std::vector<int32_t> &offsets, int chunk_rows) {
    std::vector<int32_t> chunks;
    for (int e : order)
        for (int r0 = 0; r0 < counts[e]; r0 += chunk_rows)
            chunks.insert(chunks.end(), {e, offsets[e] + r0, std::min(chunk_rows, counts[e] - r0), 0});
    return chunks;
}

// Pinned host buffers for the plans' uploads, kept for reuse until the
// process ends: hipHostMalloc costs tens of microseconds per plan and
// hipHostFree waits for the whole device, which would stall a caller that
// destroys one layer's plan while later layers run.  A plan takes the
// smallest free buffer that fits, or a new one of the next power of two, and
// gives it back when destroyed, once its copy has completed.
class StagingPool {
  public:
    void *take(size_t n, size_t *cap) {
        {
            std::lock_guard<std::mutex> g(m_);
            size_t best = free_.size();
            for (size_t i = 0; i < free_.size(); ++i)
                if (free_[i].first >= n && (best == free_.size() || free_[i].first < free_[best].first))
                    best = i;
            if (best < free_.size()) {
                void *ptr = free_[best].second;
                *cap = free_[best].first;
                free_.erase(free_.begin() + long(best));
                return ptr;
            }
        }
        size_t c = 4096;
        while (c < n) c <<= 1;
        void *ptr = nullptr;
        // portable: a buffer may serve a plan on another device later
        if (hipHostMalloc(&ptr, c, hipHostMallocPortable) != hipSuccess) return nullptr;
        *cap = c;
        return ptr;
    }
    void give(void *ptr, size_t cap) noexcept {
        std::lock_guard<std::mutex> g(m_);
        try {
            free_.emplace_back(cap, ptr);
        } catch (...) {
            (void)hipHostFree(ptr);        // no room to keep it: free it (waits for the device)
        }
    }

  private:
    std::mutex m_;
    std::vector<std::pair<size_t, void *>> free_;
};

StagingPool &staging_pool() {
    static StagingPool *pool = new StagingPool;     // never destroyed: outlives every plan
    return *pool;
}

// Pinned staging of workspace bytes [begin, end), copied up asynchronously on
// `stream`; p->uploaded is recorded after `then` (further work on the stream).
template <class Fill, class Then>
int upload(moe_plan *p, size_t begin, size_t end, void *stream, Fill fill, Then then) {
    const size_t n = end - begin;
    p->staging = staging_pool().take(n > 0 ? n : 16, &p->staging_cap);
    if (!p->staging) return MOE_EHIP;
    uint8_t *s = static_cast<uint8_t *>(p->staging);
    std::memset(s, 0, n);
    fill(s - begin);                      // fill writes at workspace offsets
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (hipEventCreateWithFlags(&p->uploaded, hipEventDisableTiming) != hipSuccess) {
        p->uploaded = nullptr;
        return MOE_EHIP;
    }
    if (n > 0 && hipMemcpyAsync(static_cast<uint8_t *>(p->plan_dev) + begin, s, n,
                                hipMemcpyHostToDevice, hs) != hipSuccess)
        return MOE_EHIP;
    // the event follows the copy whatever `then` returns: destroying the plan
    // waits for it before the staging buffer is reused
    const hipError_t launched = then(hs);
    if (hipEventRecord(p->uploaded, hs) != hipSuccess) {
        (void)hipStreamSynchronize(hs);
        return MOE_EHIP;
    }
    return launched == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Runs an exported function's body; no exception crosses the C boundary.
template <class F>
int guarded(F &&body) noexcept {
    try {
        return body();
    } catch (...) {
        return MOE_ENOMEM;
    }
}

}  // namespace

extern "C" {

size_t moe_q8_1_bytes(int rows, int cols) {
    if (rows < 0 || cols <= 0 || cols % 32) return 0;
    return size_t(rows) * (size_t(cols) + size_t(cols) / 32 * 8);
}

size_t moe_weight_bytes(int type, int rows, int cols) { return weight_bytes(type, rows, cols); }

static int moe_weights_pack_impl(const moe_weights *w, void *dst, size_t dst_bytes, void *stream) {
    if (!w || !dst) return MOE_EINVAL;
    const int st = check_weights(w, w->n_expert, false);
    if (st) return st;
    if (w->n_expert <= 0) return MOE_EINVAL;
    if (!aligned16(dst)) return MOE_EALIGN;
    const size_t per = weight_bytes(w->type, w->rows, w->cols);
    for (int e = 0; e < w->n_expert; ++e)
        if (w->offset[e] > dst_bytes || dst_bytes - w->offset[e] < per) return MOE_ESIZE;
    // experts either share a matrix (equal offsets) or do not overlap
    std::vector<uint64_t> offs(w->offset, w->offset + w->n_expert);
    std::sort(offs.begin(), offs.end());
    for (size_t i = 1; i < offs.size(); ++i)
        if (offs[i] != offs[i - 1] && offs[i] - offs[i - 1] < per) return MOE_EINVAL;
    // the copy gathers: source and destination must not overlap
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(w->base), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + dst_bytes && d0 < s0 + w->base_bytes) return MOE_EINVAL;
    const auto *src = static_cast<const uint8_t *>(w->base);
    auto *out = static_cast<uint8_t *>(dst);
    const int nb = w->cols / block_values(w->type);
    const int half = (w->type & MOE_W_GU_INTERLEAVED) ? w->rows / 2 : 0;
    const bool q2 = base_type(w->type) == MOE_W_Q2_0;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // experts at a constant stride go in one launch, others one launch each
    bool uniform = w->n_expert <= 65535;
    const uint64_t stride = w->n_expert > 1 ? w->offset[1] - w->offset[0] : 0;
    for (int e = 1; uniform && e < w->n_expert; ++e)
        uniform = w->offset[e] >= w->offset[0] && w->offset[e] - w->offset[0] == uint64_t(e) * stride;
    if (uniform)
        return hip_status(launch_weight_pack(src + w->offset[0], out + w->offset[0], stride,
                                             stride ? w->n_expert : 1, w->rows, nb, half, q2, s));
    for (int e = 0; e < w->n_expert; ++e) {
        const hipError_t err =
            launch_weight_pack(src + w->offset[e], out + w->offset[e], 0, 1, w->rows, nb, half, q2, s);
        if (err != hipSuccess) return MOE_EHIP;
    }
    return MOE_OK;
}

int moe_weights_pack(const moe_weights *w, void *dst, size_t dst_bytes, void *stream) {
    return guarded([&] { return moe_weights_pack_impl(w, dst, dst_bytes, stream); });
}

size_t moe_plan_device_bytes(int tokens, int topk, int n_expert, int chunk_rows) {
    if (tokens < 0 || topk <= 0 || n_expert <= 0 || chunk_rows <= 0 || chunk_rows > kMaxChunkRows)
        return 0;
    return plan_layout(tokens, topk, n_expert, chunk_rows).total;
}

const char *moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EALIGN: return "pointer or offset not 16-byte aligned";
        case MOE_EFORMAT: return "unsupported weight format or dimension";
        case MOE_ESIZE: return "buffer too small";
        case MOE_ENOMEM: return "host memory exhausted";
        case MOE_EHIP: return "HIP error";
        case MOE_ESTATE: return "plan has no device workspace";
        default: return "unknown status";
    }
}


static int moe_prefill_plan_impl(const int32_t *ids, int tokens, int topk, int n_expert,
                                 int chunk_rows, const moe_weights *w_gu, const moe_weights *w_down,
                                 void *plan_dev, size_t plan_dev_bytes, void *stream,
                                 moe_plan **out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    int st = check_plan_args(tokens, topk, n_expert, chunk_rows, w_gu, w_down);
    if (st) return st;
    if (tokens > 0 && !ids) return MOE_EINVAL;
    const int R = tokens * topk;
    for (int i = 0; i < R; ++i)
        if (ids[i] < 0 || ids[i] >= n_expert) return MOE_EINVAL;
    const PlanLayout L = plan_layout(tokens, topk, n_expert, chunk_rows);
    if (plan_dev) {
        if (!aligned16(plan_dev)) return MOE_EALIGN;
        if (plan_dev_bytes < L.total) return MOE_ESIZE;
    }
    PlanPtr p = new_plan(tokens, topk, n_expert, chunk_rows, w_gu, w_down);

    // counting sort by expert, stable in t*K+k
    p->counts.assign(n_expert, 0);
    for (int i = 0; i < R; ++i) p->counts[ids[i]] += 1;
    p->offsets.assign(n_expert + 1, 0);
    for (int e = 0; e < n_expert; ++e) p->offsets[e + 1] = p->offsets[e] + p->counts[e];
    p->perm.assign(R, 0);
    p->inv.assign(R, 0);
    {
        std::vector<int32_t> fill(p->offsets.begin(), p->offsets.end() - 1);
        for (int i = 0; i < R; ++i) {
            const int r = fill[ids[i]]++;
            p->perm[r] = i;
            p->inv[i] = r;
        }
    }
    const std::vector<int> order = expert_order(p->counts);
    p->chunks = chunk_list(order, p->counts, p->offsets, chunk_rows);
    p->max_chunk_rows = n_expert > 0 ? std::min(chunk_rows, *std::max_element(p->counts.begin(), p->counts.end()))
                                     : 0;
    p->n_chunks = int(p->chunks.size() / 4);

    // XCD work lists: every chunk of an expert goes to one XCD so that its
    // weights and activation rows are re-read from that XCD's L2; experts are
    // dealt largest first to the XCD with the fewest rows so far.
    {
        std::vector<std::vector<int>> members(kXcds);
        long long load[kXcds] = {};
        for (int e : order) {
            if (p->counts[e] == 0) continue;
            int x = 0;
            for (int k = 1; k < kXcds; ++k)
                if (load[k] < load[x]) x = k;
            load[x] += p->counts[e];
            members[x].push_back(e);
        }
        const int small[2] = {small_rows_for(p->hidden), small_rows_for(p->n_ff)};
        int cnt[kXcds], large[2][kXcds], tot_small[2] = {0, 0}, tot_large[2] = {0, 0};
        std::vector<std::vector<int32_t>> lists(kXcds);
        for (int x = 0; x < kXcds; ++x) {
            lists[x] = chunk_list(members[x], p->counts, p->offsets, chunk_rows);
            cnt[x] = int(lists[x].size() / 4);
            for (int q = 0; q < 2; ++q) {
                // members come largest first: the experts above the small
                // kernel's row limit are a prefix of the list
                large[q][x] = 0;
                for (int e : members[x])
                    if (p->counts[e] > small[q]) large[q][x] += (p->counts[e] + chunk_rows - 1) / chunk_rows;
                tot_large[q] += large[q][x];
                tot_small[q] += cnt[x] - large[q][x];
            }
        }
        // a few small experts beside large ones join the product kernel's view
        for (int q = 0; q < 2; ++q)
            if (tot_small[q] < kSmallMinChunks && tot_large[q] > 0)
                for (int x = 0; x < kXcds; ++x) large[q][x] = cnt[x];
        int start = 0;
        for (int x = 0; x < kXcds; ++x) {
            p->xcd_tab[kXcdStart * kXcds + x] = start;
            p->xcd_tab[kXcdCount * kXcds + x] = cnt[x];
            for (int q = 0; q < 2; ++q) {
                p->xcd_tab[(kXcdLarge + 4 * q) * kXcds + x] = start;
                p->xcd_tab[(kXcdLarge + 4 * q + 1) * kXcds + x] = large[q][x];
                p->xcd_tab[(kXcdSmall + 4 * q) * kXcds + x] = start + large[q][x];
                p->xcd_tab[(kXcdSmall + 4 * q + 1) * kXcds + x] = cnt[x] - large[q][x];
                p->max_large[q] = std::max<long long>(p->max_large[q], large[q][x]);
                p->max_small[q] = std::max<long long>(p->max_small[q], cnt[x] - large[q][x]);
            }
            start += cnt[x];
            p->max_xcd_chunks = std::max<long long>(p->max_xcd_chunks, cnt[x]);
            p->dev_chunks.insert(p->dev_chunks.end(), lists[x].begin(), lists[x].end());
        }
    }

    if (!grids_fit(p.get())) return MOE_EINVAL;
    if (plan_dev) {
        p->plan_dev = plan_dev;
        // the sections after dn_off are the device-built plan's own
        st = upload(p.get(), 0, L.counts, stream,
                    [&](uint8_t *s) {
                        std::memcpy(s + L.perm, p->perm.data(), size_t(R) * 4);
                        std::memcpy(s + L.inv, p->inv.data(), size_t(R) * 4);
                        std::memcpy(s + L.chunks, p->dev_chunks.data(), p->dev_chunks.size() * 4);
                        std::memcpy(s + L.xcd, p->xcd_tab, sizeof(p->xcd_tab));
                        std::memcpy(s + L.gu_off, p->gu_off.data(), size_t(n_expert) * 8);
                        std::memcpy(s + L.dn_off, p->dn_off.data(), size_t(n_expert) * 8);
                    },
                    [](hipStream_t) { return hipSuccess; });
        if (st) return st;
    }
    *out = p.release();
    return MOE_OK;
}

int moe_prefill_plan(const int32_t *ids, int tokens, int topk, int n_expert, int chunk_rows,
                     const moe_weights *w_gu, const moe_weights *w_down, void *plan_dev,
                     size_t plan_dev_bytes, void *stream, moe_plan **out) {
    return guarded([&] {
        return moe_prefill_plan_impl(ids, tokens, topk, n_expert, chunk_rows, w_gu, w_down, plan_dev,
                                     plan_dev_bytes, stream, out);
    });
}

static int moe_prefill_plan_device_impl(const int32_t *ids_dev, int tokens, int topk,
                                        int n_expert, int chunk_rows, const moe_weights *w_gu,
                                        const moe_weights *w_down, void *plan_dev,
                                        size_t plan_dev_bytes, void *stream, moe_plan **out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    int st = check_plan_args(tokens, topk, n_expert, chunk_rows, w_gu, w_down);
    if (st) return st;
    if ((tokens > 0 && !ids_dev) || !plan_dev || n_expert > kPlanMaxExperts) return MOE_EINVAL;
    // the dealing packs an XCD's rows and its index into 32 bits
    if ((long long)tokens * topk >= (1LL << 29)) return MOE_EINVAL;
    if ((ids_dev && !aligned16(ids_dev)) || !aligned16(plan_dev)) return MOE_EALIGN;
    const PlanLayout L = plan_layout(tokens, topk, n_expert, chunk_rows);
    if (plan_dev_bytes < L.total) return MOE_ESIZE;
    PlanPtr p = new_plan(tokens, topk, n_expert, chunk_rows, w_gu, w_down);
    p->device_built = true;
    p->plan_dev = plan_dev;
    // per-XCD list lengths are known only on the device: launches take the
    // bound every list stays within, and the surplus workgroups exit at once
    p->n_chunks = -1;
    p->max_xcd_chunks = max_chunks(p->rows, n_expert, chunk_rows);
    for (int q = 0; q < 2; ++q) p->max_large[q] = p->max_small[q] = p->max_xcd_chunks;
    if (!grids_fit(p.get())) return MOE_EINVAL;
    // the two weight offset tables go up from the host, the rest is built there
    st = upload(p.get(), L.gu_off, L.counts, stream,
                [&](uint8_t *s) {
                    std::memcpy(s + L.gu_off, p->gu_off.data(), size_t(n_expert) * 8);
                    std::memcpy(s + L.dn_off, p->dn_off.data(), size_t(n_expert) * 8);
                },
                [&](hipStream_t hs) {
                    return launch_device_plan(ids_dev, p->rows, n_expert, chunk_rows,
                                              small_rows_for(p->hidden), small_rows_for(p->n_ff),
                                              static_cast<uint8_t *>(plan_dev), L, hs);
                });
    if (st) return st;
    *out = p.release();
    return MOE_OK;
}

int moe_prefill_plan_device(const int32_t *ids_dev, int tokens, int topk, int n_expert,
                            int chunk_rows, const moe_weights *w_gu, const moe_weights *w_down,
                            void *plan_dev, size_t plan_dev_bytes, void *stream, moe_plan **out) {
    return guarded([&] {
        return moe_prefill_plan_device_impl(ids_dev, tokens, topk, n_expert, chunk_rows, w_gu, w_down,
                                            plan_dev, plan_dev_bytes, stream, out);
    });
}

// The experts of w at a constant stride: offset[e] = offset[0] + e * stride
// (stride 0: one shared matrix).
static bool strided(const moe_weights *w, uint64_t *first, uint64_t *stride) {
    *first = w->offset[0];
    *stride = w->n_expert > 1 ? w->offset[1] - w->offset[0] : 0;
    for (int e = 1; e < w->n_expert; ++e)
        if (w->offset[e] < w->offset[0] || w->offset[e] - w->offset[0] != uint64_t(e) * *stride)
            return false;
    return true;
}

// One plan object per device for plans in the library's workspace (never
// freed; the next such plan on the device takes it over).
static moe_plan g_scratch_plans[64];

static int moe_prefill_plan_device_noalloc_impl(const int32_t *ids_dev, int tokens, int topk,
                                                int n_expert, int chunk_rows,
                                                const moe_weights *w_gu, const moe_weights *w_down,
                                                void *stream, moe_plan **out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    int st = check_plan_args(tokens, topk, n_expert, chunk_rows, w_gu, w_down);
    if (st) return st;
    if ((tokens > 0 && !ids_dev) || n_expert > kPlanMaxExperts) return MOE_EINVAL;
    if ((long long)tokens * topk >= (1LL << 29)) return MOE_EINVAL;
    if (ids_dev && !aligned16(ids_dev)) return MOE_EALIGN;
    uint64_t gu_first, gu_stride, dn_first, dn_stride;
    if (!strided(w_gu, &gu_first, &gu_stride) || !strided(w_down, &dn_first, &dn_stride))
        return MOE_EINVAL;
    const PlanLayout L = plan_layout(tokens, topk, n_expert, chunk_rows);
    if (L.total > kScratchBytes) return MOE_ESIZE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_EHIP;
    void *ws = nullptr;
    if (scratch_workspace(&ws) != hipSuccess) return MOE_EHIP;
    // the device's plan object: its fields are set here, its containers stay empty
    moe_plan *p = &g_scratch_plans[dev];
    p->tokens = tokens; p->topk = topk; p->n_expert = n_expert; p->chunk_rows = chunk_rows;
    p->max_chunk_rows = chunk_rows;
    p->rows = tokens * topk; p->hidden = w_gu->cols; p->n_ff = w_gu->rows / 2;
    p->gu = *w_gu; p->dn = *w_down;
    p->gu.offset = nullptr; p->dn.offset = nullptr;      // on the device only
    if (base_type(w_gu->type) == MOE_W_NL4) std::memcpy(p->gu_codebook, w_gu->codebook, 16);
    if (base_type(w_down->type) == MOE_W_NL4) std::memcpy(p->dn_codebook, w_down->codebook, 16);
    p->gu.codebook = p->gu_codebook; p->dn.codebook = p->dn_codebook;
    p->layout = L;
    p->n_chunks = -1;
    p->max_xcd_chunks = max_chunks(p->rows, n_expert, chunk_rows);
    for (int q = 0; q < 2; ++q) p->max_large[q] = p->max_small[q] = p->max_xcd_chunks;
    p->device_built = true; p->in_scratch = true;
    p->plan_dev = ws; p->stream = static_cast<hipStream_t>(stream);
    p->staging = nullptr; p->staging_cap = 0; p->uploaded = nullptr;
    if (!grids_fit(p)) return MOE_EINVAL;
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (launch_stride_offsets(reinterpret_cast<uint64_t *>(w8 + L.gu_off), gu_first, gu_stride,
                              reinterpret_cast<uint64_t *>(w8 + L.dn_off), dn_first, dn_stride, n_expert,
                              hs) != hipSuccess ||
        launch_device_plan(ids_dev, p->rows, n_expert, chunk_rows, small_rows_for(p->hidden),
                           small_rows_for(p->n_ff), w8, L, hs) != hipSuccess)
        return MOE_EHIP;
    *out = p;
    return MOE_OK;
}

int moe_prefill_plan_device_noalloc(const int32_t *ids_dev, int tokens, int topk, int n_expert,
                                    int chunk_rows, const moe_weights *w_gu,
                                    const moe_weights *w_down, void *stream, moe_plan **out) {
    return guarded([&] {
        return moe_prefill_plan_device_noalloc_impl(ids_dev, tokens, topk, n_expert, chunk_rows, w_gu,
                                                    w_down, stream, out);
    });
}

static int moe_plan_query_impl(const moe_plan *p, int *rows, int *n_chunks, int32_t *counts,
                               int32_t *offsets, int32_t *perm, int32_t *chunks) {
    if (!p) return MOE_EINVAL;
    if (p->device_built) {
        // read the device-built plan back (waits for it)
        const int E = p->n_expert;
        std::vector<int32_t> dc(E + 1), doff(E + 2), dperm(p->rows), status(1);
        const uint8_t *ws = static_cast<const uint8_t *>(p->plan_dev);
        const PlanLayout &L = p->layout;
        const hipError_t built = p->uploaded ? hipEventSynchronize(p->uploaded)
                                             : hipStreamSynchronize(p->stream);
        if (built != hipSuccess ||
            hipMemcpy(dc.data(), ws + L.counts, dc.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(doff.data(), ws + L.offsets, doff.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(status.data(), ws + L.aux + 4 * size_t(PlanAux::status(E)), 4,
                      hipMemcpyDeviceToHost) != hipSuccess ||
            (p->rows > 0 &&
             hipMemcpy(dperm.data(), ws + L.perm, dperm.size() * 4, hipMemcpyDeviceToHost) != hipSuccess))
            return MOE_EHIP;
        if (status[0] != 0) return MOE_EINVAL;          // routing ids out of range
        dc.resize(E);
        doff.resize(E + 1);
        const std::vector<int32_t> ch = chunk_list(expert_order(dc), dc, doff, p->chunk_rows);
        if (rows) *rows = p->rows;
        if (n_chunks) *n_chunks = int(ch.size() / 4);
        if (counts) std::copy(dc.begin(), dc.end(), counts);
        if (offsets) std::copy(doff.begin(), doff.end(), offsets);
        if (perm) std::copy(dperm.begin(), dperm.end(), perm);
        if (chunks) std::copy(ch.begin(), ch.end(), chunks);
        return MOE_OK;
    }
    if (rows) *rows = p->rows;
    if (n_chunks) *n_chunks = p->n_chunks;
    if (counts) std::copy(p->counts.begin(), p->counts.end(), counts);
    if (offsets) std::copy(p->offsets.begin(), p->offsets.end(), offsets);
    if (perm) std::copy(p->perm.begin(), p->perm.end(), perm);
    if (chunks) std::copy(p->chunks.begin(), p->chunks.end(), chunks);
    return MOE_OK;
}

int moe_plan_query(const moe_plan *p, int *rows, int *n_chunks, int32_t *counts, int32_t *offsets,
                   int32_t *perm, int32_t *chunks) {
    return guarded(
        [&] { return moe_plan_query_impl(p, rows, n_chunks, counts, offsets, perm, chunks); });
}

void moe_plan_destroy(moe_plan *p) {
    if (!p || p->in_scratch) return;
    if (p->uploaded) {
        (void)hipEventSynchronize(p->uploaded);
        (void)hipEventDestroy(p->uploaded);
    }
    // the copy from the staging buffer has completed (or never started)
    if (p->staging) staging_pool().give(p->staging, p->staging_cap);
    delete p;
}

static const uint8_t *dev_at(const moe_plan *p, size_t off) {
    return static_cast<const uint8_t *>(p->plan_dev) + off;
}

static int ready(const moe_plan *p) {
    if (!p) return MOE_EINVAL;
    if (!p->plan_dev) return MOE_ESTATE;
    return MOE_OK;
}

int quantize_scatter(const moe_plan *p, const float *x, void *xq, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (p->rows == 0) return MOE_OK;
    if (!x || !xq) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(xq)) return MOE_EALIGN;
    return hip_status(launch_quantize_scatter(
        x, p->tokens, p->hidden, p->topk, reinterpret_cast<const int32_t *>(dev_at(p, p->layout.inv)),
        static_cast<uint8_t *>(xq), static_cast<hipStream_t>(stream)));
}

static ProductArgs product_args(const moe_plan *p, int product, const void *act) {
    ProductArgs a{};
    const moe_weights &w = product == 0 ? p->gu : p->dn;
    a.act = static_cast<const uint8_t *>(act);
    a.w_base = static_cast<const uint8_t *>(w.base);
    a.w_off = reinterpret_cast<const uint64_t *>(dev_at(p, product == 0 ? p->layout.gu_off
                                                                          : p->layout.dn_off));
    a.chunks = reinterpret_cast<const int32_t *>(dev_at(p, p->layout.chunks));
    const int32_t *tab = reinterpret_cast<const int32_t *>(dev_at(p, p->layout.xcd));
    a.xcd = tab + (kXcdLarge + 4 * product) * kXcds;
    a.xcd_small = tab + (kXcdSmall + 4 * product) * kXcds;
    a.perm = product == 0 ? nullptr : reinterpret_cast<const int32_t *>(dev_at(p, p->layout.perm));
    a.wtype = base_type(w.type);
    a.cols = w.cols;
    a.out_rows = w.rows;
    a.n_tiles = (w.rows + kTileRows - 1) / kTileRows;
    a.max_items = int(p->max_xcd_chunks * a.n_tiles);     // fits: grids_fit at plan time
    if (a.wtype == MOE_W_NL4) std::memcpy(a.codebook, product == 0 ? p->gu_codebook : p->dn_codebook, 16);
    a.small_rows = small_rows_for(w.cols);
    return a;
}

// Weight tiles per product-kernel item.  When every chunk has at most 64
// rows, an item of at most kShortStages stages (the down product: 10 at
// n_ff 640) is short and its start (the table reads and first weight loads
// from HBM, about 4 us) is a large part of it: an item then runs up to
// kGroupTiles tiles of its chunk as one stream, the next tile's first loads in
// flight under the current tile's last stages (2,048 tokens: 5-8 % off the
// down product).  The stream needs Q2_0 fp32 outputs, whole N tiles and a
// stage count the prefetch depths divide.  Longer items keep one tile each:
// the gate/up's (40 stages) are four times longer, and fewer, longer items
// balanced worse over the XCDs than the start they save (fused 3-7 %, and the
// four-launch form's gate/up 9 %, slower).
static int tile_group(const ProductArgs &a, const moe_plan *p) {
    constexpr int kGroupTiles = 5;
    constexpr int kShortStages = 16;
    const int n_stages = (a.cols + 63) / 64;
    if (a.wtype != MOE_W_Q2_0 || a.dots || a.hq || p->max_chunk_rows > 64 || n_stages > kShortStages ||
        n_stages % kStreamStages != 0 || a.out_rows % kTileRows != 0 || a.n_tiles < 2)
        return 1;
    return std::min(a.n_tiles, kGroupTiles);
}

// The experts of at most a.small_rows rows go to the small kernel, the others
// to the product kernel, each over its view of the XCD lists (a.n_tiles set);
// a launch with no item is skipped.
static hipError_t launch_products(const moe_plan *p, int product, ProductArgs a, hipStream_t stream) {
    hipError_t e = hipSuccess;
    a.group = 1;
    a.max_items = int(p->max_small[product] * a.n_tiles);
    if (a.max_items > 0) e = launch_expert_small(a, stream);
    a.group = tile_group(a, p);
    a.max_items = int(p->max_large[product] * ((a.n_tiles + a.group - 1) / a.group));
    if (e == hipSuccess && a.max_items > 0) e = launch_expert_product(a, stream);
    return e;
}

int expert_gate_up(const moe_plan *p, const void *xq, float *gu, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (p->rows == 0) return MOE_OK;
    if (!xq || !gu) return MOE_EINVAL;
    if (!aligned16(xq) || !aligned16(gu)) return MOE_EALIGN;
    ProductArgs a = product_args(p, 0, xq);
    a.out = gu;
    return hip_status(launch_products(p, 0, a, static_cast<hipStream_t>(stream)));
}

int expert_gate_up_swiglu_q8(const moe_plan *p, const void *xq, void *hq, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (p->rows == 0) return MOE_OK;
    if (!xq || !hq) return MOE_EINVAL;
    if (!aligned16(xq) || !aligned16(hq)) return MOE_EALIGN;
    ProductArgs a = product_args(p, 0, xq);
    // work items of 128 j's: gate rows j and up rows n_ff + j together
    a.n_tiles = (p->n_ff + kTileRows / 2 - 1) / (kTileRows / 2);
    a.hq = static_cast<uint8_t *>(hq);
    return hip_status(launch_products(p, 0, a, static_cast<hipStream_t>(stream)));
}

int swiglu_q8(const moe_plan *p, const float *gu, void *hq, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (p->rows == 0) return MOE_OK;
    if (!gu || !hq) return MOE_EINVAL;
    if (!aligned16(gu) || !aligned16(hq)) return MOE_EALIGN;
    return hip_status(launch_swiglu_q8(gu, p->rows, p->n_ff, static_cast<uint8_t *>(hq),
                                       static_cast<hipStream_t>(stream)));
}

int expert_down(const moe_plan *p, const void *hq, float *dm, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (p->rows == 0) return MOE_OK;
    if (!hq || !dm) return MOE_EINVAL;
    if (!aligned16(hq) || !aligned16(dm)) return MOE_EALIGN;
    ProductArgs a = product_args(p, 1, hq);
    a.out = dm;
    return hip_status(launch_products(p, 1, a, static_cast<hipStream_t>(stream)));
}

int moe_combine(const moe_plan *p, const float *dm, const float *w, float *out, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (p->rows == 0) return MOE_OK;
    if (!dm || !w || !out) return MOE_EINVAL;
    if (!aligned16(dm) || !aligned16(w) || !aligned16(out)) return MOE_EALIGN;
    // one thread per float4 of the flat (token, float4) range
    const uint64_t threads = uint64_t(p->tokens) * uint64_t(p->hidden / 4);
    if (threads > 0xFFFFFFFFull) return MOE_EINVAL;
    return hip_status(launch_combine(dm, w, p->tokens, p->topk, p->hidden, out,
                                     static_cast<hipStream_t>(stream)));
}

int moe_debug_block_dots(const moe_plan *p, int product, const void *act, int row_begin,
                         int n_rows, int32_t *dots, void *stream) {
    int st = ready(p);
    if (st) return st;
    if (!act || !dots || (product != 0 && product != 1)) return MOE_EINVAL;
    if (row_begin < 0 || n_rows < 0 || (long long)row_begin + n_rows > p->rows) return MOE_EINVAL;
    if (!aligned16(act) || !aligned16(dots)) return MOE_EALIGN;
    if (n_rows == 0) return MOE_OK;
    ProductArgs a = product_args(p, product, act);
    a.dots = dots;
    a.dots_row_begin = row_begin;
    a.dots_n_rows = n_rows;
    return hip_status(launch_products(p, product, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
