// HBM expert cache: per-layer slot table with LRU eviction, fed from pinned host
// RAM by hipMemcpyAsync on a copy stream and ordered with hipEvents.
//
// LayerStoRm README ("TL;DR"): the full expert set stays pinned in host RAM,
// GPU memory is used as a cache, activated experts are streamed over PCIe and
// the transfers overlap compute; the rebasdaily article ("keep the experts in
// the warehouse") adds that the host only manages the runtime and moves data.
// The replacement rule (least recently used, hits touched before misses,
// ascending expert id, never evict what the same request needs) is this
// library's reading: the pages name the cache but not its policy.
//
// Ordering, per layer:
//   copy stream   : [wait release of victim slot] -> H2D slab copy -> ... ->
//                   record ready
//   compute stream: wait ready -> table update kernel -> FFN kernels ->
//                   moe_cache_release records the release event that the next
//                   copy into those slots waits for.
// The copy half (moe_cache_prefetch_async) and the compute half (moe_cache_wait)
// can be issued apart, so the copies of later layers are queued before the
// kernels of earlier ones.
#include <algorithm>
#include <cstring>
#include <deque>
#include <memory>
#include <utility>
#include <vector>

#include "common.h"

namespace {

constexpr int kTableBatch = 64;
constexpr int kReleaseRing = 8;

struct TableUpdate {
    int n;
    int experts[kTableBatch];
    const void *ptrs[kTableBatch];
};

__global__ void table_update_kernel(const void **table, TableUpdate u) {
    const int i = threadIdx.x;
    if (i < u.n) table[u.experts[i]] = u.ptrs[i];
}

__global__ void table_clear_kernel(const void **table, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) table[i] = nullptr;
}

// ------------------------------------------------------------------ copy engines
struct Engine {
    virtual ~Engine() = default;
    virtual int wait_release(int layer, int slot, long long release_id) = 0;
    virtual int copy(int layer, int expert, int slot, void *dst, const void *src, size_t bytes) = 0;
    // table writes of a prefetch: applied by the layer's next wait()
    virtual int table(int layer, const std::vector<int> &experts, const std::vector<const void *> &ptrs,
                      const std::vector<int> &slots) = 0;
    // table writes that must land now (a prefetch that failed part-way keeps the
    // table equal to what is resident)
    virtual int table_now(int layer, const std::vector<int> &experts, const std::vector<const void *> &ptrs,
                          const std::vector<int> &slots) {
        return table(layer, experts, ptrs, slots);
    }
    virtual int copies_done(int layer) = 0;                // after the layer's copies, on the copy stream
    virtual int wait(int layer, void *compute_stream) = 0;  // compute waits for them, then the table writes
    virtual int release(int layer, long long release_id, int n_slots, void *compute_stream) = 0;
    virtual int sync() = 0;
    virtual int drain() { return sync(); }
    virtual int clear_table() = 0;
    // later copies in two halves, the second on stream2 (nullptr: one stream)
    virtual int split_copies(hipStream_t) { return MOE_OK; }
    // copy timing (see HipEngine)
    virtual int set_timing(bool) { return MOE_OK; }
    virtual int copy_busy(double *busy_ms, double *span_ms, uint64_t *n) {
        *busy_ms = *span_ms = 0.0;
        *n = 0;
        return MOE_OK;
    }
};

struct HipEngine final : Engine {
    int L = 0, E = 0;
    hipStream_t copy_stream = nullptr;
    hipStream_t copy_stream2 = nullptr;  // second halves of split copies, or nullptr
    const void **tbl = nullptr;
    std::vector<hipEvent_t> ready_ev;    // [L]
    std::vector<hipEvent_t> ready_ev2;   // [L], on copy_stream2
    hipEvent_t join_ev = nullptr;        // copy_stream2 -> copy_stream
    std::vector<hipEvent_t> release_ev;  // [L * kReleaseRing]
    // table writes waiting for wait(), per layer; one entry per expert (the latest)
    std::vector<std::vector<int>> pend_exp;
    std::vector<std::vector<const void *>> pend_ptr;

    int init(int layers, int experts, hipStream_t cs, void **table_dev) {
        L = layers;
        E = experts;
        copy_stream = cs;
        tbl = (const void **)table_dev;
        ready_ev.assign(L, nullptr);
        release_ev.assign((size_t)L * kReleaseRing, nullptr);
        pend_exp.assign(L, {});
        pend_ptr.assign(L, {});
        for (auto &e : ready_ev) MOE_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        for (auto &e : release_ev) MOE_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        return MOE_OK;
    }
    ~HipEngine() override {
        if (copy_stream) (void)hipStreamSynchronize(copy_stream);
        if (copy_stream2) (void)hipStreamSynchronize(copy_stream2);
        for (auto &p : ev_pend) {
            (void)hipEventDestroy(p.first);
            (void)hipEventDestroy(p.second);
        }
        for (auto e : ev_pool) (void)hipEventDestroy(e);
        if (t_ref) (void)hipEventDestroy(t_ref);
        for (auto e : ready_ev)
            if (e) (void)hipEventDestroy(e);
        for (auto e : ready_ev2)
            if (e) (void)hipEventDestroy(e);
        if (join_ev) (void)hipEventDestroy(join_ev);
        for (auto e : release_ev)
            if (e) (void)hipEventDestroy(e);
    }
    // A release that has already completed needs no barrier on the copy stream
    // (a barrier ahead of each copy costs the copy engine tens of microseconds).
    // The ring slot may hold a later release of the layer; that one completing
    // implies this one did.
    int wait_release(int layer, int, long long id) override {
        hipEvent_t ev = release_ev[(size_t)layer * kReleaseRing + id % kReleaseRing];
        const hipError_t q = hipEventQuery(ev);
        if (q == hipSuccess) return MOE_OK;
        if (q != hipErrorNotReady) return moe::fail_hip(q, "hipEventQuery(release)");
        MOE_TRY_HIP(hipStreamWaitEvent(copy_stream, ev, 0));
        if (copy_stream2) MOE_TRY_HIP(hipStreamWaitEvent(copy_stream2, ev, 0));
        return MOE_OK;
    }
    // Two streams: the first half (rounded to 4 KiB) on the copy stream, the rest
    // on the second, so two DMA engines share the link (back-to-back slab copies
    // on one stream leave it ~4% below what one large copy reaches).
    int copy(int, int, int, void *dst, const void *src, size_t bytes) override {
        if (!copy_stream2 || bytes < 8192) return timed_copy(dst, src, bytes, copy_stream);
        const size_t h = (bytes / 2) & ~(size_t)4095;
        int rc = timed_copy(dst, src, h, copy_stream);
        if (rc != MOE_OK) return rc;
        return timed_copy((char *)dst + h, (const char *)src + h, bytes - h, copy_stream2);
    }

    // ---- copy timing: with timing on, each copy is bracketed by two timing
    // events on its stream (the first after the copy's release waits), and the
    // completed pairs become intervals relative to a reference event; the busy
    // time of the link is the length of the union of the intervals of both
    // streams.
    bool timing = false;
    hipEvent_t t_ref = nullptr;
    std::vector<hipEvent_t> ev_pool;
    std::deque<std::pair<hipEvent_t, hipEvent_t>> ev_pend;
    std::vector<std::pair<double, double>> spans;  // ms after t_ref

    int take_event(hipEvent_t *e) {
        if (!ev_pool.empty()) {
            *e = ev_pool.back();
            ev_pool.pop_back();
            return MOE_OK;
        }
        MOE_TRY_HIP(hipEventCreate(e));  // timing events
        return MOE_OK;
    }
    // completed pairs -> spans (pairs complete in order per stream; the queue
    // mixes both streams, so stop at the first one not done)
    int harvest(bool all) {
        while (!ev_pend.empty()) {
            auto [a, b] = ev_pend.front();
            if (all) {
                MOE_TRY_HIP(hipEventSynchronize(b));
            } else {
                const hipError_t q = hipEventQuery(b);
                if (q == hipErrorNotReady) break;
                if (q != hipSuccess) return moe::fail_hip(q, "hipEventQuery(copy timing)");
            }
            float t0 = 0.f, t1 = 0.f;
            MOE_TRY_HIP(hipEventElapsedTime(&t0, t_ref, a));
            MOE_TRY_HIP(hipEventElapsedTime(&t1, t_ref, b));
            spans.emplace_back(t0, t1);
            ev_pool.push_back(a);
            ev_pool.push_back(b);
            ev_pend.pop_front();
        }
        return MOE_OK;
    }
    int timed_copy(void *dst, const void *src, size_t bytes, hipStream_t st) {
        if (!timing) {
            MOE_TRY_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st));
            return MOE_OK;
        }
        int rc = ev_pend.size() >= 64 ? harvest(false) : MOE_OK;
        if (rc != MOE_OK) return rc;
        hipEvent_t a = nullptr, b = nullptr;
        rc = take_event(&a);
        if (rc == MOE_OK) rc = take_event(&b);
        if (rc != MOE_OK) return rc;
        MOE_TRY_HIP(hipEventRecord(a, st));
        MOE_TRY_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, st));
        MOE_TRY_HIP(hipEventRecord(b, st));
        ev_pend.emplace_back(a, b);
        return MOE_OK;
    }
    int set_timing(bool on) override {
        int rc = sync();
        if (rc == MOE_OK) rc = harvest(true);
        if (rc != MOE_OK) return rc;
        spans.clear();
        timing = on;
        if (on) {
            if (!t_ref) MOE_TRY_HIP(hipEventCreate(&t_ref));
            MOE_TRY_HIP(hipEventRecord(t_ref, copy_stream));
        }
        return MOE_OK;
    }
    int copy_busy(double *busy_ms, double *span_ms, uint64_t *n) override {
        int rc = sync();
        if (rc == MOE_OK) rc = harvest(true);
        if (rc != MOE_OK) return rc;
        std::vector<std::pair<double, double>> v(spans);
        std::sort(v.begin(), v.end());
        double busy = 0.0, cur0 = 0.0, cur1 = 0.0;
        bool open = false;
        for (const auto &iv : v) {
            if (open && iv.first <= cur1) {
                cur1 = std::max(cur1, iv.second);
                continue;
            }
            if (open) busy += cur1 - cur0;
            cur0 = iv.first;
            cur1 = iv.second;
            open = true;
        }
        if (open) busy += cur1 - cur0;
        *busy_ms = busy;
        *span_ms = v.empty() ? 0.0 : std::max_element(v.begin(), v.end(), [](auto &x, auto &y) {
                                         return x.second < y.second;
                                     })->second - v.front().first;
        *n = v.size();
        return MOE_OK;
    }
    int split_copies(hipStream_t s2) override {
        if (s2 && ready_ev2.empty()) {
            ready_ev2.assign(L, nullptr);
            for (auto &e : ready_ev2) MOE_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
            MOE_TRY_HIP(hipEventCreateWithFlags(&join_ev, hipEventDisableTiming));
        }
        if (copy_stream2) MOE_TRY_HIP(hipStreamSynchronize(copy_stream2));
        copy_stream2 = s2;
        return MOE_OK;
    }
    // Table writes run on the compute stream after it waits for the layer's
    // copies, so the copy stream carries only DMA copies and event records (a
    // kernel between two copies would stall the copy engine).  One launch writes
    // up to 64 entries; an expert appears at most once per launch.
    int launch_updates(int layer, const std::vector<int> &experts, const std::vector<const void *> &ptrs,
                       hipStream_t st) {
        for (size_t i = 0; i < experts.size(); i += kTableBatch) {
            TableUpdate u{};
            u.n = (int)std::min<size_t>(kTableBatch, experts.size() - i);
            for (int j = 0; j < u.n; ++j) {
                u.experts[j] = experts[i + j];
                u.ptrs[j] = ptrs[i + j];
            }
            hipLaunchKernelGGL(table_update_kernel, dim3(1), dim3(kTableBatch), 0, st, tbl + (size_t)layer * E, u);
            MOE_LAUNCH_CHECK("table_update_kernel");
        }
        return MOE_OK;
    }
    int table(int layer, const std::vector<int> &experts, const std::vector<const void *> &ptrs,
              const std::vector<int> &) override {
        auto &pe = pend_exp[layer];
        auto &pp = pend_ptr[layer];
        for (size_t i = 0; i < experts.size(); ++i) {
            const auto it = std::find(pe.begin(), pe.end(), experts[i]);
            if (it != pe.end()) {
                pp[it - pe.begin()] = ptrs[i];
            } else {
                pe.push_back(experts[i]);
                pp.push_back(ptrs[i]);
            }
        }
        return MOE_OK;
    }
    int table_now(int layer, const std::vector<int> &experts, const std::vector<const void *> &ptrs,
                  const std::vector<int> &slots) override {
        // earlier pending writes of the layer land first, in the same stream order
        int rc = table(layer, experts, ptrs, slots);
        if (rc != MOE_OK) return rc;
        if (copy_stream2) {  // the second halves land before the table names them
            MOE_TRY_HIP(hipEventRecord(join_ev, copy_stream2));
            MOE_TRY_HIP(hipStreamWaitEvent(copy_stream, join_ev, 0));
        }
        rc = launch_updates(layer, pend_exp[layer], pend_ptr[layer], copy_stream);
        pend_exp[layer].clear();
        pend_ptr[layer].clear();
        return rc;
    }
    int copies_done(int layer) override {
        MOE_TRY_HIP(hipEventRecord(ready_ev[layer], copy_stream));
        if (copy_stream2) MOE_TRY_HIP(hipEventRecord(ready_ev2[layer], copy_stream2));
        return MOE_OK;
    }
    int wait(int layer, void *compute_stream) override {
        hipStream_t cs = (hipStream_t)compute_stream;
        MOE_TRY_HIP(hipStreamWaitEvent(cs, ready_ev[layer], 0));
        if (copy_stream2) MOE_TRY_HIP(hipStreamWaitEvent(cs, ready_ev2[layer], 0));
        const int rc = launch_updates(layer, pend_exp[layer], pend_ptr[layer], cs);
        pend_exp[layer].clear();
        pend_ptr[layer].clear();
        return rc;
    }
    int release(int layer, long long id, int, void *compute_stream) override {
        MOE_TRY_HIP(hipEventRecord(release_ev[(size_t)layer * kReleaseRing + id % kReleaseRing],
                                   (hipStream_t)compute_stream));
        return MOE_OK;
    }
    int sync() override {
        MOE_TRY_HIP(hipStreamSynchronize(copy_stream));
        if (copy_stream2) MOE_TRY_HIP(hipStreamSynchronize(copy_stream2));
        return MOE_OK;
    }
    // Copies done and every recorded release reached: no kernel enqueued before
    // a moe_cache_release still reads a slot or the table (an event never
    // recorded counts as complete).
    int drain() override {
        int rc = sync();
        if (rc != MOE_OK) return rc;
        for (auto e : release_ev) MOE_TRY_HIP(hipEventSynchronize(e));
        return MOE_OK;
    }
    int clear_table() override {
        for (int l = 0; l < L; ++l) {
            pend_exp[l].clear();
            pend_ptr[l].clear();
        }
        const size_t n = (size_t)L * E;
        hipLaunchKernelGGL(table_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, copy_stream, tbl, n);
        MOE_LAUNCH_CHECK("table_clear_kernel");
        MOE_TRY_HIP(hipStreamSynchronize(copy_stream));
        return MOE_OK;
    }
};

// Records every command instead of issuing it (host-only tests of the policy).
struct RecordingEngine final : Engine {
    std::vector<int64_t> cmds;  // 4 per command
    int fail_copy_at = 0, copies = 0;
    void put(int64_t k, int64_t a, int64_t b, int64_t c) {
        cmds.push_back(k);
        cmds.push_back(a);
        cmds.push_back(b);
        cmds.push_back(c);
    }
    int wait_release(int, int slot, long long id) override {
        put(1, slot, id, -1);
        return MOE_OK;
    }
    int copy(int layer, int expert, int slot, void *, const void *, size_t) override {
        ++copies;
        if (fail_copy_at > 0 && copies == fail_copy_at)
            return moe::fail_hip(hipErrorInvalidValue, "recorded copy (injected failure)");
        put(2, layer, expert, slot);
        return MOE_OK;
    }
    int table(int layer, const std::vector<int> &experts, const std::vector<const void *> &,
              const std::vector<int> &slots) override {
        for (size_t i = 0; i < experts.size(); ++i) put(3, layer, experts[i], slots[i]);
        return MOE_OK;
    }
    int copies_done(int) override { return MOE_OK; }
    int wait(int layer, void *) override {
        put(4, layer, -1, -1);
        return MOE_OK;
    }
    int release(int layer, long long id, int n_slots, void *) override {
        put(5, layer, id, n_slots);
        return MOE_OK;
    }
    int sync() override { return MOE_OK; }
    int clear_table() override { return MOE_OK; }
};

}  // namespace

struct moe_cache {
    moe_cache_desc d{};
    size_t slab_bytes = 0;
    std::vector<const void *> host;  // [L * E]
    uintptr_t pool = 0;
    std::unique_ptr<Engine> engine;
    RecordingEngine *recorder = nullptr;
    // per layer state
    std::vector<int> slot_of;            // [L * E]
    std::vector<int> expert_of;          // [L * C]
    std::vector<unsigned long long> stamp;  // [L * C], 0 = never used
    std::vector<char> held;              // [L * C]
    std::vector<long long> last_release; // [L * C], -1 = never released
    std::vector<long long> next_release; // [L]
    std::vector<char> unwaited;          // [L], copies or table writes not yet waited for
    unsigned long long clock = 0;
    uint64_t hits = 0, misses = 0, bytes = 0;

    int C() const { return d.slots_per_layer; }
    void *slot_ptr(int layer, int slot) const {
        return (void *)(pool + ((size_t)layer * C() + slot) * slab_bytes);
    }
    void clear_state() {
        const size_t L = d.n_layers, E = d.n_experts, Cs = C();
        slot_of.assign(L * E, -1);
        expert_of.assign(L * Cs, -1);
        stamp.assign(L * Cs, 0);
        held.assign(L * Cs, 0);
        last_release.assign(L * Cs, -1);
        next_release.assign(L, 0);
        unwaited.assign(L, 0);
        clock = 0;
        hits = misses = bytes = 0;
    }
};

namespace {

int validate_desc(const moe_cache_desc *d) {
    if (!d) return moe::fail(MOE_E_ARG, "cache: NULL desc");
    if (d->n_layers < 1 || d->n_experts < 1 || d->slots_per_layer < 1)
        return moe::fail(MOE_E_ARG, "cache: layers=%d experts=%d slots=%d", d->n_layers, d->n_experts,
                         d->slots_per_layer);
    if (d->slots_per_layer > d->n_experts)
        return moe::fail(MOE_E_SHAPE, "cache: slots %d > experts %d", d->slots_per_layer, d->n_experts);
    if (d->format < 0 || d->format > 2) return moe::fail(MOE_E_ARG, "cache: format %d", d->format);
    if (d->format == 2 && moe_expert_bytes_sb(d->hidden, d->inter) == 0)
        return moe::fail(MOE_E_SHAPE, "cache: super-block slabs need H, I multiples of 256");
    if (moe_expert_bytes(d->hidden, d->inter) == 0)
        return moe::fail(MOE_E_SHAPE, "cache: hidden=%d inter=%d", d->hidden, d->inter);
    return MOE_OK;
}

int check_request(const moe_cache *c, int layer, const int32_t *experts, int n) {
    if (!c) return moe::fail(MOE_E_ARG, "cache: NULL cache");
    if (layer < 0 || layer >= c->d.n_layers) return moe::fail(MOE_E_ARG, "cache: layer %d", layer);
    if (n < 0 || (n > 0 && !experts)) return moe::fail(MOE_E_ARG, "cache: n=%d", n);
    std::vector<char> seen(c->d.n_experts, 0);
    for (int i = 0; i < n; ++i) {
        const int e = experts[i];
        if (e < 0 || e >= c->d.n_experts) return moe::fail(MOE_E_ARG, "cache: expert %d out of range", e);
        if (seen[e]) return moe::fail(MOE_E_ARG, "cache: expert %d requested twice", e);
        seen[e] = 1;
    }
    return MOE_OK;
}

}  // namespace

static int cache_make(const moe_cache_desc *desc, moe_cache **out) {
    int rc = validate_desc(desc);
    if (rc != MOE_OK) return rc;
    if (!out) return moe::fail(MOE_E_ARG, "cache: NULL out");
    auto *c = new moe_cache();
    c->d = *desc;
    c->slab_bytes = desc->format == 1   ? moe_expert_bytes_mx(desc->hidden, desc->inter)
                    : desc->format == 2 ? moe_expert_bytes_sb(desc->hidden, desc->inter)
                                        : moe_expert_bytes(desc->hidden, desc->inter);
    c->clear_state();
    *out = c;
    return MOE_OK;
}

extern "C" int moe_cache_create(const moe_cache_desc *desc, const void *const *experts_host, void *slot_pool,
                                void **expert_table, void *copy_stream, moe_cache **out) {
    if (!experts_host || !slot_pool || !expert_table || !out) return moe::fail(MOE_E_ARG, "cache_create: NULL");
    int rc = validate_desc(desc);
    if (rc != MOE_OK) return rc;
    const size_t n = (size_t)desc->n_layers * desc->n_experts;
    for (size_t i = 0; i < n; ++i) {
        hipPointerAttribute_t attr;
        hipError_t e = hipPointerGetAttributes(&attr, experts_host[i]);
        if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return moe::fail(MOE_E_NOT_PINNED, "cache_create: host slab %zu (%p) is not pinned", i, experts_host[i]);
        }
    }
    moe_cache *c = nullptr;
    rc = cache_make(desc, &c);
    if (rc != MOE_OK) return rc;
    c->host.assign(experts_host, experts_host + n);
    c->pool = (uintptr_t)slot_pool;
    auto eng = std::make_unique<HipEngine>();
    rc = eng->init(desc->n_layers, desc->n_experts, (hipStream_t)copy_stream, expert_table);
    if (rc == MOE_OK) rc = eng->clear_table();
    if (rc != MOE_OK) {
        delete c;
        return rc;
    }
    c->engine = std::move(eng);
    *out = c;
    return MOE_OK;
}

extern "C" int moe_cache_create_recording(const moe_cache_desc *desc, uintptr_t slot_pool, int fail_copy_at,
                                          moe_cache **out) {
    moe_cache *c = nullptr;
    int rc = cache_make(desc, &c);
    if (rc != MOE_OK) return rc;
    c->host.assign((size_t)desc->n_layers * desc->n_experts, nullptr);
    c->pool = slot_pool;
    auto eng = std::make_unique<RecordingEngine>();
    eng->fail_copy_at = fail_copy_at;
    c->recorder = eng.get();
    c->engine = std::move(eng);
    *out = c;
    return MOE_OK;
}

extern "C" int64_t moe_cache_trace(const moe_cache *c, int64_t *cmds, int64_t max_cmds) {
    if (!c || !c->recorder) return -1;
    const int64_t total = (int64_t)c->recorder->cmds.size() / 4;
    if (cmds && max_cmds > 0) {
        const int64_t n = std::min(total, max_cmds);
        std::memcpy(cmds, c->recorder->cmds.data(), (size_t)n * 4 * sizeof(int64_t));
    }
    return total;
}

extern "C" int moe_cache_lookup(moe_cache *c, int layer, const int32_t *experts, int n, int32_t *slots,
                                int *n_hits) {
    int rc = check_request(c, layer, experts, n);
    if (rc != MOE_OK) return rc;
    if (n > 0 && !slots) return moe::fail(MOE_E_ARG, "cache_lookup: NULL slots");
    int h = 0;
    for (int i = 0; i < n; ++i) {
        slots[i] = c->slot_of[(size_t)layer * c->d.n_experts + experts[i]];
        h += slots[i] >= 0;
    }
    if (n_hits) *n_hits = h;
    return MOE_OK;
}

extern "C" int moe_cache_prefetch_async(moe_cache *c, int layer, const int32_t *experts, int n, int *n_copies) {
    int rc = check_request(c, layer, experts, n);
    if (rc != MOE_OK) return rc;
    const int Cs = c->C(), E = c->d.n_experts;
    if (n > Cs) return moe::fail(MOE_E_CAPACITY, "cache_prefetch: %d experts > %d slots", n, Cs);
    int *slot_of = &c->slot_of[(size_t)layer * E];
    int *expert_of = &c->expert_of[(size_t)layer * Cs];
    unsigned long long *stamp = &c->stamp[(size_t)layer * Cs];
    char *held = &c->held[(size_t)layer * Cs];
    long long *last_rel = &c->last_release[(size_t)layer * Cs];

    std::vector<int> sorted(experts, experts + n);
    std::sort(sorted.begin(), sorted.end());
    std::vector<int> hit_list, miss_list;
    for (int e : sorted) (slot_of[e] >= 0 ? hit_list : miss_list).push_back(e);
    // capacity: misses need slots that are neither held nor needed by this request
    int free_slots = 0;
    std::vector<char> needed(Cs, 0);
    for (int e : hit_list) needed[slot_of[e]] = 1;
    for (int s = 0; s < Cs; ++s) free_slots += (!held[s] && !needed[s]);
    if ((int)miss_list.size() > free_slots)
        return moe::fail(MOE_E_CAPACITY, "cache_prefetch: %zu misses but only %d free slots (layer %d)",
                         miss_list.size(), free_slots, layer);

    std::vector<int> acquired;
    for (int e : hit_list) {
        const int s = slot_of[e];
        stamp[s] = ++c->clock;
        if (!held[s]) acquired.push_back(s);
        held[s] = 1;
    }
    std::vector<int> t_exp, t_slot;
    std::vector<const void *> t_ptr;
    int copies = 0;
    long long last_wait = -2;
    for (int e : miss_list) {
        int victim = -1;
        for (int s = 0; s < Cs; ++s) {
            if (held[s]) continue;
            if (victim < 0 || stamp[s] < stamp[victim]) victim = s;  // ties keep the lower slot
        }
        const int old = expert_of[victim];
        if (old >= 0) {
            slot_of[old] = -1;
            t_exp.push_back(old);
            t_ptr.push_back(nullptr);
            t_slot.push_back(-1);
        }
        expert_of[victim] = -1;
        stamp[victim] = 0;
        if (last_rel[victim] >= 0 && last_rel[victim] != last_wait) {
            rc = c->engine->wait_release(layer, victim, last_rel[victim]);
            if (rc != MOE_OK) break;
            last_wait = last_rel[victim];
        }
        void *dst = c->slot_ptr(layer, victim);
        rc = c->engine->copy(layer, e, victim, dst, c->host[(size_t)layer * E + e], c->slab_bytes);
        if (rc != MOE_OK) break;
        ++copies;
        expert_of[victim] = e;
        slot_of[e] = victim;
        stamp[victim] = ++c->clock;
        held[victim] = 1;
        acquired.push_back(victim);
        t_exp.push_back(e);
        t_ptr.push_back(dst);
        t_slot.push_back(victim);
    }
    if (rc != MOE_OK) {
        // keep the table consistent with what is resident, then un-hold this request
        (void)c->engine->table_now(layer, t_exp, t_ptr, t_slot);
        for (int s : acquired) held[s] = 0;
        return rc;
    }
    if (!t_exp.empty()) {
        rc = c->engine->table(layer, t_exp, t_ptr, t_slot);
        if (rc != MOE_OK) return rc;
    }
    if (copies > 0 || !t_exp.empty()) {
        rc = c->engine->copies_done(layer);
        if (rc != MOE_OK) return rc;
        c->unwaited[layer] = 1;
    }
    c->hits += hit_list.size();
    c->misses += miss_list.size();
    c->bytes += (uint64_t)copies * c->slab_bytes;
    if (n_copies) *n_copies = copies;
    return MOE_OK;
}

extern "C" int moe_cache_plan(const moe_cache *c, int layer, const int32_t *ids_host, int n_ids,
                              int32_t *wave_experts_host, int32_t *wave_start_host, int max_waves,
                              uint8_t *masks_host, int *n_waves) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_plan: NULL cache");
    if (layer < 0 || layer >= c->d.n_layers) return moe::fail(MOE_E_ARG, "cache_plan: layer %d", layer);
    if (n_ids < 0 || (n_ids > 0 && !ids_host) || !wave_start_host || !n_waves || max_waves < 1 ||
        (n_ids > 0 && !wave_experts_host))
        return moe::fail(MOE_E_ARG, "cache_plan: n_ids=%d max_waves=%d or a NULL pointer", n_ids, max_waves);
    const int E = c->d.n_experts, Cs = c->C();
    std::vector<char> seen(E, 0);
    for (int i = 0; i < n_ids; ++i) {
        const int e = ids_host[i];
        if (e < 0 || e >= E) return moe::fail(MOE_E_ARG, "cache_plan: expert %d out of range", e);
        seen[e] = 1;
    }
    // distinct experts, hits first then misses, each in ascending id
    const int *slot_of = &c->slot_of[(size_t)layer * E];
    std::vector<int> order;
    for (int e = 0; e < E; ++e)
        if (seen[e] && slot_of[e] >= 0) order.push_back(e);
    for (int e = 0; e < E; ++e)
        if (seen[e] && slot_of[e] < 0) order.push_back(e);
    const int n = (int)order.size();
    // one wave if they fit.  Otherwise a small first wave and a small last wave
    // of `edge` experts each, and between them the fewest waves of at most half
    // the slots, sizes differing by at most one (the first ones larger).  The
    // small first wave (resident experts) computes and frees slots soon after the
    // layer starts, so the copy stream, idle since the previous layer's last
    // copy, resumes early; the small last wave leaves little compute after the
    // layer's last copy.
    const int half = std::max(1, Cs / 2);
    std::vector<int> sizes;
    if (n > 0 && n <= Cs) {
        sizes.push_back(n);
    } else if (n > Cs) {
        const int edge = std::max(1, half / 8);
        const int mid = n - 2 * edge;  // >= 0: n > Cs >= 1 and edge <= max(1, Cs / 16)
        const int nm = (mid + half - 1) / half;
        sizes.push_back(edge);
        for (int v = 0; v < nm; ++v) sizes.push_back(mid / nm + (v < mid % nm ? 1 : 0));
        sizes.push_back(edge);
    }
    const int waves = (int)sizes.size();
    if (waves > max_waves) return moe::fail(MOE_E_CAPACITY, "cache_plan: %d waves > max_waves %d", waves, max_waves);
    if (masks_host) std::memset(masks_host, 0, (size_t)max_waves * E);
    wave_start_host[0] = 0;
    int b = 0;
    for (int v = 0; v < waves; ++v) {
        const int e_ = b + sizes[v];
        std::sort(order.begin() + b, order.begin() + e_);
        for (int i = b; i < e_; ++i) {
            wave_experts_host[i] = order[i];
            if (masks_host) masks_host[(size_t)v * E + order[i]] = 1;
        }
        wave_start_host[v + 1] = e_;
        b = e_;
    }
    *n_waves = waves;
    return MOE_OK;
}

extern "C" int moe_cache_plan_step(moe_cache *c, const int32_t *ids_host, int ids_per_layer,
                                   int32_t *wave_experts_host, int32_t *wave_start_host, int max_waves,
                                   uint8_t *masks_host, int32_t *n_waves_host, int issue_single, int *n_copies) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_plan_step: NULL cache");
    if (ids_per_layer < 0 || (ids_per_layer > 0 && !ids_host) || !wave_experts_host || !wave_start_host ||
        !n_waves_host || max_waves < 1)
        return moe::fail(MOE_E_ARG, "cache_plan_step: ids_per_layer=%d max_waves=%d or a NULL pointer", ids_per_layer,
                         max_waves);
    const int Ln = c->d.n_layers, E = c->d.n_experts;
    const size_t per = (size_t)std::max(ids_per_layer, 1);
    int copies = 0;
    for (int l = 0; l < Ln; ++l) {
        int32_t *we = wave_experts_host + (size_t)l * per;
        int32_t *ws = wave_start_host + (size_t)l * (max_waves + 1);
        int nw = 0;
        int rc = moe_cache_plan(c, l, ids_host + (size_t)l * ids_per_layer, ids_per_layer, we, ws, max_waves,
                                masks_host ? masks_host + (size_t)l * max_waves * E : nullptr, &nw);
        if (rc != MOE_OK) return rc;
        n_waves_host[l] = nw;
        if (issue_single && nw == 1) {
            int nc = 0;
            rc = moe_cache_prefetch_async(c, l, we, ws[1], &nc);
            if (rc != MOE_OK) return rc;
            copies += nc;
        }
    }
    if (n_copies) *n_copies = copies;
    return MOE_OK;
}

extern "C" int moe_cache_copy_timing(moe_cache *c, int enable) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_copy_timing: NULL cache");
    return c->engine->set_timing(enable != 0);
}

extern "C" int moe_cache_copy_busy(moe_cache *c, double *busy_ms, double *span_ms, uint64_t *n_copies) {
    if (!c || !busy_ms || !span_ms || !n_copies) return moe::fail(MOE_E_ARG, "cache_copy_busy: NULL pointer");
    return c->engine->copy_busy(busy_ms, span_ms, n_copies);
}

extern "C" int moe_cache_split_copies(moe_cache *c, void *second_copy_stream) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_split_copies: NULL cache");
    for (int l = 0; l < c->d.n_layers; ++l)
        if (c->unwaited[l])
            return moe::fail(MOE_E_STATE, "cache_split_copies: layer %d has copies not yet waited for", l);
    return c->engine->split_copies((hipStream_t)second_copy_stream);
}

extern "C" int moe_cache_wait(moe_cache *c, int layer, void *compute_stream) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_wait: NULL cache");
    if (layer < 0 || layer >= c->d.n_layers) return moe::fail(MOE_E_ARG, "cache_wait: layer %d", layer);
    if (!c->unwaited[layer]) return MOE_OK;
    const int rc = c->engine->wait(layer, compute_stream);
    if (rc != MOE_OK) return rc;
    c->unwaited[layer] = 0;
    return MOE_OK;
}

extern "C" int moe_cache_prefetch(moe_cache *c, int layer, const int32_t *experts, int n, void *compute_stream,
                                  int *n_copies) {
    const int rc = moe_cache_prefetch_async(c, layer, experts, n, n_copies);
    if (rc != MOE_OK) return rc;
    return moe_cache_wait(c, layer, compute_stream);
}

extern "C" int moe_cache_release(moe_cache *c, int layer, void *compute_stream) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_release: NULL cache");
    if (layer < 0 || layer >= c->d.n_layers) return moe::fail(MOE_E_ARG, "cache_release: layer %d", layer);
    if (c->unwaited[layer])
        return moe::fail(MOE_E_STATE, "cache_release: layer %d has copies not yet waited for (moe_cache_wait)", layer);
    const int Cs = c->C();
    char *held = &c->held[(size_t)layer * Cs];
    int n_held = 0;
    for (int s = 0; s < Cs; ++s) n_held += held[s] != 0;
    if (n_held == 0) return MOE_OK;
    const long long id = c->next_release[layer]++;
    int rc = c->engine->release(layer, id, n_held, compute_stream);
    if (rc != MOE_OK) return rc;
    long long *last_rel = &c->last_release[(size_t)layer * Cs];
    for (int s = 0; s < Cs; ++s)
        if (held[s]) {
            held[s] = 0;
            last_rel[s] = id;
        }
    return MOE_OK;
}

extern "C" int moe_cache_stats(const moe_cache *c, uint64_t *hits, uint64_t *misses, uint64_t *h2d_bytes) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_stats: NULL cache");
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (h2d_bytes) *h2d_bytes = c->bytes;
    return MOE_OK;
}

extern "C" int moe_cache_reset(moe_cache *c) {
    if (!c) return moe::fail(MOE_E_ARG, "cache_reset: NULL cache");
    // wait for the copies and for every kernel ordered before a release, so that
    // nothing still reads a slot or table entry when the table is cleared
    int rc = c->engine->drain();
    if (rc != MOE_OK) return rc;
    rc = c->engine->clear_table();
    if (rc != MOE_OK) return rc;
    c->clear_state();
    return MOE_OK;
}

extern "C" void moe_cache_destroy(moe_cache *c) {
    if (c && c->engine) (void)c->engine->drain();
    delete c;
}
