// Online precision residency: fixed-block pools, the budget tracker, the
// hysteresis policy and the transition manager.
//
// Page "DynaExq":
//   * 2.2 / 3.2 -- every expert resolves through a stable handle to a complete
//     version; a new version becomes visible only once its data is complete
//     (publish after the copy), and the old one is reclaimed only after the
//     switch (evict after publish).
//   * 2.3 / 3.3 -- expert versions live in pools of fixed-size blocks with
//     constant-time free lists; a budget tracker admits each promotion with
//     an explicit reservation against what is left after the fixed part.
//   * 2.4 / 3.4 -- copies of prepacked high-precision weights from pinned host
//     memory run on a migration stream apart from the compute stream, and a
//     completion event gates the publish; evictions go first; refused
//     promotions wait (backpressure at admission).
//   * 2.5 / 3.5 -- counters of router selections per update interval folded
//     into an EMA score; the high-precision set is the top n_hi by score,
//     changed only across a hysteresis margin.
//
// The pages run the transition manager as a background thread.  Here every
// transition is an event on a HIP stream, so the manager is polled at window
// boundaries (moe_residency_step) from the thread that runs the layer: no
// locks, and the handle table changes only between forward calls.
#include <stdio.h>

#include <atomic>
#include <chrono>
#include <vector>

#include "../../include/moe_residency.h"
#include "internal.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

using moe::fail;
using moe::hip_status;

// ---------------------------------------------------------------------------
// fixed-block pool
// ---------------------------------------------------------------------------
struct moe_pool {
    char* base;
    size_t block;
    int nblocks;
    std::vector<int> free_list;    // stack of free block indices
    std::vector<uint8_t> in_use;
};

MOE_API int moe_pool_create(void* arena, size_t arena_bytes, size_t block_bytes, moe_pool** out) {
    if (!arena || !out) return fail(MOE_EINVAL, "null pointer");
    if (reinterpret_cast<uintptr_t>(arena) % 256) return fail(MOE_EINVAL, "arena must be 256-byte aligned");
    if (block_bytes == 0 || block_bytes % 256) return fail(MOE_EINVAL, "block_bytes must be a positive multiple of 256");
    const size_t n = arena_bytes / block_bytes;
    if (n < 1) return fail(MOE_EINVAL, "the arena holds no block");
    if (n > (1u << 30)) return fail(MOE_EUNSUPPORTED, "too many blocks");
    moe_pool* p = new moe_pool;
    p->base = static_cast<char*>(arena);
    p->block = block_bytes;
    p->nblocks = static_cast<int>(n);
    p->free_list.resize(n);
    for (size_t i = 0; i < n; ++i) p->free_list[i] = static_cast<int>(n - 1 - i);   // block 0 handed out first
    p->in_use.assign(n, 0);
    *out = p;
    return MOE_OK;
}

MOE_API void moe_pool_destroy(moe_pool* p) { delete p; }

MOE_API int moe_pool_alloc(moe_pool* p, void** block) {
    if (!p || !block) return fail(MOE_EINVAL, "null pointer");
    if (p->free_list.empty()) {
        *block = nullptr;
        return MOE_EFULL;
    }
    const int i = p->free_list.back();
    p->free_list.pop_back();
    p->in_use[i] = 1;
    *block = p->base + static_cast<size_t>(i) * p->block;
    return MOE_OK;
}

MOE_API int moe_pool_free(moe_pool* p, void* block) {
    if (!p || !block) return fail(MOE_EINVAL, "null pointer");
    const char* b = static_cast<const char*>(block);
    if (b < p->base) return fail(MOE_EINVAL, "not a block of this pool");
    const size_t off = static_cast<size_t>(b - p->base);
    if (off % p->block || off / p->block >= static_cast<size_t>(p->nblocks))
        return fail(MOE_EINVAL, "not a block of this pool");
    const int i = static_cast<int>(off / p->block);
    if (!p->in_use[i]) return fail(MOE_EINVAL, "block is already free");
    p->in_use[i] = 0;
    p->free_list.push_back(i);
    return MOE_OK;
}

MOE_API int moe_pool_free_blocks(const moe_pool* p) { return p ? static_cast<int>(p->free_list.size()) : MOE_EINVAL; }
MOE_API int moe_pool_total_blocks(const moe_pool* p) { return p ? p->nblocks : MOE_EINVAL; }
MOE_API size_t moe_pool_block_bytes(const moe_pool* p) { return p ? p->block : 0; }

// ---------------------------------------------------------------------------
// budget tracker
// ---------------------------------------------------------------------------
struct moe_budget {
    size_t capacity;
    std::atomic<size_t> used;
};

MOE_API int moe_budget_create(size_t total_bytes, size_t fixed_bytes, moe_budget** out) {
    if (!out) return fail(MOE_EINVAL, "null pointer");
    if (fixed_bytes > total_bytes) return fail(MOE_EINVAL, "fixed part exceeds the total");
    moe_budget* b = new moe_budget;
    b->capacity = total_bytes - fixed_bytes;
    b->used.store(0);
    *out = b;
    return MOE_OK;
}

MOE_API void moe_budget_destroy(moe_budget* b) { delete b; }

MOE_API int moe_budget_try_reserve(moe_budget* b, size_t bytes) {
    if (!b) return fail(MOE_EINVAL, "null pointer");
    size_t cur = b->used.load(std::memory_order_relaxed);
    do {
        if (bytes > b->capacity - cur) return 0;
    } while (!b->used.compare_exchange_weak(cur, cur + bytes, std::memory_order_acq_rel, std::memory_order_relaxed));
    return 1;
}

MOE_API int moe_budget_release(moe_budget* b, size_t bytes) {
    if (!b) return fail(MOE_EINVAL, "null pointer");
    size_t cur = b->used.load(std::memory_order_relaxed);
    do {
        if (bytes > cur) return fail(MOE_EINVAL, "release exceeds the reserved bytes");
    } while (!b->used.compare_exchange_weak(cur, cur - bytes, std::memory_order_acq_rel, std::memory_order_relaxed));
    return MOE_OK;
}

MOE_API size_t moe_budget_used(const moe_budget* b) { return b ? b->used.load() : 0; }
MOE_API size_t moe_budget_capacity(const moe_budget* b) { return b ? b->capacity : 0; }

// ---------------------------------------------------------------------------
// policy
// ---------------------------------------------------------------------------
namespace {

// Rank order: higher score first, ties to the lower index.
struct Hotter {
    const float* S;
    bool operator()(int a, int b) const { return S[a] > S[b] || (S[a] == S[b] && a < b); }
};

void sort_hottest_first(const float* S, std::vector<int>& v) {
    // insertion sort: N <= 128, and it is stable under the total rank order
    const Hotter h{S};
    for (size_t i = 1; i < v.size(); ++i)
        for (size_t j = i; j > 0 && h(v[j], v[j - 1]); --j) std::swap(v[j], v[j - 1]);
}

void select_impl(const float* S, const uint8_t* in_hi, const uint8_t* locked, int N, int n_hi, float margin,
                 std::vector<int>& promote, std::vector<int>& demote, std::vector<uint8_t>& target) {
    promote.clear();
    demote.clear();
    std::vector<int> members, movable, outsiders;
    for (int e = 0; e < N; ++e) {
        const bool lk = locked && locked[e];
        if (in_hi[e]) {
            members.push_back(e);
            if (!lk) movable.push_back(e);
        } else if (!lk && S[e] > 0.0f) {
            outsiders.push_back(e);
        }
    }
    sort_hottest_first(S, movable);
    std::vector<int> cold(movable.rbegin(), movable.rend());   // coldest first
    size_t ci = 0;
    int size = static_cast<int>(members.size());
    while (size > n_hi && ci < cold.size()) {   // capacity shrink
        demote.push_back(cold[ci++]);
        --size;
    }
    sort_hottest_first(S, outsiders);
    size_t oi = 0;
    while (size < n_hi && oi < outsiders.size()) {   // free capacity
        promote.push_back(outsiders[oi++]);
        ++size;
    }
    for (; oi < outsiders.size() && ci < cold.size(); ++oi, ++ci) {   // hysteresis swaps
        const float bar = S[cold[ci]] + margin;                       // rounded to fp32
        if (!(S[outsiders[oi]] > bar)) break;
        promote.push_back(outsiders[oi]);
        demote.push_back(cold[ci]);
    }
    target.assign(in_hi, in_hi + N);
    for (int e : demote) target[e] = 0;
    for (int e : promote) target[e] = 1;
}

}  // namespace

MOE_API int moe_residency_select(const float* S, const uint8_t* in_hi, const uint8_t* locked, int N, int n_hi,
                                 float margin, uint8_t* target, int32_t* promote, int* n_promote, int32_t* demote,
                                 int* n_demote) {
    if (!S || !in_hi || !target || !promote || !n_promote || !demote || !n_demote)
        return fail(MOE_EINVAL, "null pointer");
    if (N < 1 || N > moe::kMaxExperts) return fail(MOE_EINVAL, "N must be in [1, 128]");
    if (n_hi < 0) return fail(MOE_EINVAL, "n_hi must be >= 0");
    if (!(margin >= 0.0f)) return fail(MOE_EINVAL, "margin must be >= 0");
    std::vector<int> pro, dem;
    std::vector<uint8_t> tgt;
    select_impl(S, in_hi, locked, N, n_hi, margin, pro, dem, tgt);
    for (size_t i = 0; i < pro.size(); ++i) promote[i] = pro[i];
    for (size_t i = 0; i < dem.size(); ++i) demote[i] = dem[i];
    *n_promote = static_cast<int>(pro.size());
    *n_demote = static_cast<int>(dem.size());
    for (int e = 0; e < N; ++e) target[e] = tgt[e];
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// transition manager
// ---------------------------------------------------------------------------
struct moe_residency {
    moe_residency_config cfg;
    std::vector<moe_expert_handle> lo;
    std::vector<const void*> hi_src;
    size_t hi_bytes = 0;
    std::vector<int> state;
    std::vector<void*> block;          // device block of a PROMOTING / HI / EVICTING expert
    std::vector<hipEvent_t> ev_copy;   // per expert: its hi copy on the migration stream
    std::vector<hipEvent_t> ev_pub;    // per expert: the publish of its lo version on the compute stream
    hipEvent_t ev_fold = nullptr;      // the EMA fold on the compute stream
    hipEvent_t ev_scores = nullptr;    // the scores' copy to the host
    bool scores_pending = false;
    std::vector<int> pending;          // promotions waiting for admission, hottest first
    std::chrono::steady_clock::time_point last_update;
    moe_residency_stats stats{};
};

namespace {

void destroy_events(moe_residency* r) {
    for (hipEvent_t e : r->ev_copy) if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : r->ev_pub) if (e) (void)hipEventDestroy(e);
    if (r->ev_fold) (void)hipEventDestroy(r->ev_fold);
    if (r->ev_scores) (void)hipEventDestroy(r->ev_scores);
}

// 1: the event has completed; 0: not yet; negative: error.
int event_done(hipEvent_t ev, bool wait) {
    const hipError_t e = wait ? hipEventSynchronize(ev) : hipEventQuery(ev);
    if (e == hipSuccess) return 1;
    if (e == hipErrorNotReady) return 0;
    return hip_status(e, "moe_residency_step: event");
}

moe_expert_handle hi_handle(const moe_residency* r, int e) {
    const size_t m = static_cast<size_t>(r->cfg.H) * r->cfg.I * 2;   // bytes of one bf16 matrix
    char* b = static_cast<char*>(r->block[e]);
    moe_expert_handle h{};
    h.fmt = MOE_W_BF16;
    h.group = 0;
    h.w_gate = b;
    h.w_up = b + m;
    h.w_down = b + 2 * m;
    return h;
}

}  // namespace

MOE_API int moe_residency_create(const moe_residency_config* cfg, moe_residency** out) {
    if (!cfg || !out) return fail(MOE_EINVAL, "null pointer");
    const moe_residency_config& c = *cfg;
    if (c.N < 1 || c.N > moe::kMaxExperts) return fail(MOE_EINVAL, "N must be in [1, 128]");
    if (c.H < 128 || c.H % 128 || c.I < 128 || c.I % 128)
        return fail(MOE_EINVAL, "H and I must be positive multiples of 128");
    if (!c.table || !c.lo || !c.hi_src || !c.pool_hi || !c.budget || !c.S || !c.c || !c.S_host)
        return fail(MOE_EINVAL, "null pointer");
    if (c.n_hi < 0 || c.n_hi > c.N) return fail(MOE_EINVAL, "n_hi must be in [0, N]");
    if (!(c.alpha >= 0.0f && c.alpha < 1.0f)) return fail(MOE_EINVAL, "alpha must be in [0, 1)");
    if (!(c.margin >= 0.0f)) return fail(MOE_EINVAL, "margin must be >= 0");
    if (c.compute_stream == c.mig_stream) return fail(MOE_EINVAL, "the migration stream must differ from the compute stream");
    const size_t hi_bytes = static_cast<size_t>(6) * c.H * c.I;
    if (c.pool_hi->block < hi_bytes) return fail(MOE_EINVAL, "pool blocks are smaller than one bf16 expert");
    for (int e = 0; e < c.N; ++e) {
        if (!c.hi_src[e]) return fail(MOE_EINVAL, "null hi_src entry");
        if (reinterpret_cast<uintptr_t>(c.hi_src[e]) % 16) return fail(MOE_EINVAL, "hi_src buffers must be 16-byte aligned");
        const moe_expert_handle& h = c.lo[e];
        if (!h.w_gate || !h.w_up || !h.w_down) return fail(MOE_EINVAL, "null low-precision weight pointer");
        if (h.fmt != MOE_W_INT4_G128 && h.fmt != MOE_W_BF16 && h.fmt != MOE_W_F32)
            return fail(MOE_EINVAL, "bad low-precision format");
        if (h.fmt == MOE_W_INT4_G128 && (h.group != 128 || !h.s_gate || !h.s_up || !h.s_down))
            return fail(MOE_EINVAL, "INT4 handle needs group 128 and scale pointers");
    }
    moe_residency* r = new moe_residency;
    r->cfg = c;
    r->lo.assign(c.lo, c.lo + c.N);
    r->hi_src.assign(c.hi_src, c.hi_src + c.N);
    r->hi_bytes = hi_bytes;
    r->state.assign(c.N, MOE_RES_LO);
    r->block.assign(c.N, nullptr);
    r->ev_copy.assign(c.N, nullptr);
    r->ev_pub.assign(c.N, nullptr);
    hipError_t err = hipSuccess;
    for (int e = 0; e < c.N && err == hipSuccess; ++e) {
        err = hipEventCreateWithFlags(&r->ev_copy[e], hipEventDisableTiming);
        if (err == hipSuccess) err = hipEventCreateWithFlags(&r->ev_pub[e], hipEventDisableTiming);
    }
    if (err == hipSuccess) err = hipEventCreateWithFlags(&r->ev_fold, hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&r->ev_scores, hipEventDisableTiming);
    if (err != hipSuccess) {
        destroy_events(r);
        delete r;
        return hip_status(err, "moe_residency_create: hipEventCreate");
    }
    r->last_update = std::chrono::steady_clock::now();
    *out = r;
    return MOE_OK;
}

MOE_API int moe_residency_step(moe_residency* r, const int32_t* cnt, int flags) {
    if (!r) return fail(MOE_EINVAL, "null pointer");
    if (flags & ~(MOE_RES_FORCE_UPDATE | MOE_RES_WAIT)) return fail(MOE_EINVAL, "unknown flags");
    const moe_residency_config& c = r->cfg;
    const int N = c.N;
    const bool wait = flags & MOE_RES_WAIT;
    hipStream_t cs = static_cast<hipStream_t>(c.compute_stream);
    hipStream_t ms = static_cast<hipStream_t>(c.mig_stream);
    int st;
    r->stats.steps++;

    // 1. counts, and an update if it is due
    if (cnt) {
        st = hip_status(moe::launch_hotness_accumulate(c.c, cnt, N, cs), "moe_residency_step: counts");
        if (st) return st;
    }
    const auto now = std::chrono::steady_clock::now();
    const double since = std::chrono::duration<double>(now - r->last_update).count();
    const bool due = (flags & MOE_RES_FORCE_UPDATE) || (c.interval_s >= 0.0 && since >= c.interval_s);
    if (due && !r->scores_pending) {
        hipError_t e = moe::launch_hotness_fold(c.S, c.c, N, c.alpha, cs);
        if (e == hipSuccess) e = hipEventRecord(r->ev_fold, cs);
        if (e == hipSuccess) e = hipStreamWaitEvent(ms, r->ev_fold, 0);
        if (e == hipSuccess) e = hipMemcpyAsync(c.S_host, c.S, N * sizeof(float), hipMemcpyDeviceToHost, ms);
        if (e == hipSuccess) e = hipEventRecord(r->ev_scores, ms);
        st = hip_status(e, "moe_residency_step: update");
        if (st) return st;
        r->scores_pending = true;
        r->last_update = now;
        r->stats.updates++;
    }

    // 2. decide on arrived scores; demotions publish the low version now
    if (r->scores_pending) {
        st = event_done(r->ev_scores, wait);
        if (st < 0) return st;
        if (st == 1) {
            r->scores_pending = false;
            std::vector<uint8_t> in_hi(N), locked(N), target;
            for (int e = 0; e < N; ++e) {
                in_hi[e] = r->state[e] == MOE_RES_HI || r->state[e] == MOE_RES_PROMOTING;
                locked[e] = r->state[e] == MOE_RES_PROMOTING || r->state[e] == MOE_RES_EVICTING;
            }
            std::vector<int> promote, demote;
            select_impl(c.S_host, in_hi.data(), locked.data(), N, c.n_hi, c.margin, promote, demote, target);
            r->stats.decisions++;
            for (int e : demote) {   // state HI (PROMOTING experts are locked)
                hipError_t he = moe::launch_handle_publish(c.table, e, r->lo[e], cs);
                if (he == hipSuccess) he = hipEventRecord(r->ev_pub[e], cs);
                st = hip_status(he, "moe_residency_step: demote");
                if (st) return st;
                r->state[e] = MOE_RES_EVICTING;
                r->stats.demotions++;
            }
            r->pending = promote;
        }
    }

    // 3. reclaim blocks whose switch back to the low version has completed
    for (int e = 0; e < N; ++e) {
        if (r->state[e] != MOE_RES_EVICTING) continue;
        st = event_done(r->ev_pub[e], wait);
        if (st < 0) return st;
        if (st == 0) continue;
        st = moe_pool_free(c.pool_hi, r->block[e]);
        if (st) return st;
        st = moe_budget_release(c.budget, c.pool_hi->block);
        if (st) return st;
        r->block[e] = nullptr;
        r->state[e] = MOE_RES_LO;
        r->stats.evictions++;
    }

    // 4. admit pending promotions while the budget and the pool allow
    size_t admitted = 0;
    for (; admitted < r->pending.size(); ++admitted) {
        const int e = r->pending[admitted];
        if (r->state[e] != MOE_RES_LO) continue;   // stale entry
        st = moe_budget_try_reserve(c.budget, c.pool_hi->block);
        if (st < 0) return st;
        if (st == 0) { r->stats.deferred++; break; }
        void* blk = nullptr;
        st = moe_pool_alloc(c.pool_hi, &blk);
        if (st == MOE_EFULL) {
            moe_budget_release(c.budget, c.pool_hi->block);
            r->stats.deferred++;
            break;
        }
        if (st) return st;
        hipError_t he = hipMemcpyAsync(blk, r->hi_src[e], r->hi_bytes, hipMemcpyHostToDevice, ms);
        if (he == hipSuccess) he = hipEventRecord(r->ev_copy[e], ms);
        if (he != hipSuccess) {
            moe_pool_free(c.pool_hi, blk);
            moe_budget_release(c.budget, c.pool_hi->block);
            return hip_status(he, "moe_residency_step: promote");
        }
        r->block[e] = blk;
        r->state[e] = MOE_RES_PROMOTING;
        r->stats.promotions_started++;
        r->stats.bytes_h2d += static_cast<int64_t>(r->hi_bytes);
    }
    r->pending.erase(r->pending.begin(), r->pending.begin() + admitted);

    // 5. publish the promotions whose copy has completed
    for (int e = 0; e < N; ++e) {
        if (r->state[e] != MOE_RES_PROMOTING) continue;
        st = event_done(r->ev_copy[e], wait);
        if (st < 0) return st;
        if (st == 0) continue;
        hipError_t he = hipStreamWaitEvent(cs, r->ev_copy[e], 0);
        if (he == hipSuccess) he = moe::launch_handle_publish(c.table, e, hi_handle(r, e), cs);
        st = hip_status(he, "moe_residency_step: publish");
        if (st) return st;
        r->state[e] = MOE_RES_HI;
        r->stats.promotions_published++;
    }
    return MOE_OK;
}

MOE_API int moe_residency_state(const moe_residency* r, int e) {
    if (!r || e < 0 || e >= r->cfg.N) return MOE_EINVAL;
    return r->state[e];
}

MOE_API int moe_residency_pending(const moe_residency* r) {
    return r ? static_cast<int>(r->pending.size()) : MOE_EINVAL;
}

MOE_API int moe_residency_get_stats(const moe_residency* r, moe_residency_stats* out) {
    if (!r || !out) return fail(MOE_EINVAL, "null pointer");
    *out = r->stats;
    return MOE_OK;
}

MOE_API int moe_residency_destroy(moe_residency* r) {
    if (!r) return MOE_OK;
    const int st = hip_status(hipStreamSynchronize(static_cast<hipStream_t>(r->cfg.mig_stream)),
                              "moe_residency_destroy");
    destroy_events(r);
    delete r;
    return st;
}
