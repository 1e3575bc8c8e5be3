// HBM expert cache in front of a pinned host store (one LRU per layer over a
// fixed set of slots), as colibri's per-layer LRU expert cache
// (fr.news.hada.io topic 31297, "Execution d'un MoE basee sur le streaming
// disque") and LargerLM's routed expert slots ("What It Proves"), with the
// disk tier replaced by pinned host RAM and the read by an asynchronous
// host-to-device copy on a side stream.
//
// Ordering rules (all on the GPU, the host never waits for a copy):
//  - a copy into a slot waits (hipStreamWaitEvent on the copy stream) for the
//    last kernel that read the slot's previous expert;
//  - the compute stream waits for the slot's copy event before a kernel
//    reads it.
// The one host wait per token is for the token's routing (a small
// device-to-host copy of the expert ids, with the next layer's predicted ids
// beside them when a next layer is linked).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe.h"
#include "moe_cache.h"
#include "moe_cache_policy.h"
#include "moe_internal.h"
#include "moe_kernels.h"
#include "moe_layout.h"

namespace moe {

// Which event covers a slot's last read: none yet, the slot's own (a batched
// group), or the layer's end-of-call event (a one-token call).
enum : char { kUseNone = 0, kUseSlotEvent = 1, kUseCallEvent = 2 };

struct LayerSlots {
    explicit LayerSlots(int n_experts, int n_slots) : policy(n_experts, n_slots) {}
    SlotPolicy policy;
    std::vector<const void*> host_blob;    // [E] registered pinned blobs
    std::vector<hipEvent_t> copy_done;     // [slots]
    std::vector<hipEvent_t> last_use;      // [slots] last batched read of the slot
    std::vector<char> use_kind;            // [slots] kUse*: the event that covers the slot's last read
    std::vector<char> copy_recorded;       // [slots] a copy was queued and not yet seen complete
    hipEvent_t last_call = nullptr;        // end of the layer's latest call (after all of its reads)
    hipStream_t call_stream = nullptr;     // the stream last_call was recorded on
    bool call_recorded = false;
    std::vector<uint64_t> usage;           // [E] routed uses (the learning cache's counts)
    std::vector<char> fresh;               // [E] brought in by a prefetch and not used since
    std::vector<int> prediction;           // experts predicted for this layer's next call
    bool has_prediction = false;
    moe_cache_stats_t stats{};
};

}  // namespace moe

struct moe_cache {
    moe_config_t cfg{};
    int n_layers = 0;
    int slots = 0;
    uint8_t* pool = nullptr;
    size_t expert_bytes = 0;
    hipStream_t copy_stream = nullptr;
    std::vector<moe::LayerSlots*> layers;
    int32_t* pinned_ids = nullptr;   // host-pinned staging of one token's ids [0, 16) and prediction [16, 32)
    int32_t* pinned_batch = nullptr; // host-pinned staging of a launch sequence's ids (kMaxDispatchEntries)
    hipEvent_t ids_ready = nullptr;
    std::vector<int> pending_slots;  // slots read by the token being enqueued
    int pending_layer = -1;
    // copy/compute timeline (expert_cache_timeline): a pool of timing events
    // and the recorded intervals (kind 0 copy, 1 kernel; index of the begin
    // event, the end event follows it)
    bool timeline = false;
    int max_marks = 0;
    int truncated = 0;
    std::vector<hipEvent_t> tl_events;
    size_t tl_used = 0;
    std::vector<std::pair<int, int>> tl_marks;

    uint8_t* slot_ptr(int layer, int s) const {
        return pool + ((size_t)layer * slots + (size_t)s) * expert_bytes;
    }
};

namespace moe {

static void destroy_cache(moe_cache* c) {
    if (!c) return;
    for (LayerSlots* L : c->layers) {
        if (!L) continue;
        for (hipEvent_t e : L->copy_done)
            if (e) (void)hipEventDestroy(e);
        for (hipEvent_t e : L->last_use)
            if (e) (void)hipEventDestroy(e);
        if (L->last_call) (void)hipEventDestroy(L->last_call);
        delete L;
    }
    for (hipEvent_t e : c->tl_events) (void)hipEventDestroy(e);
    if (c->ids_ready) (void)hipEventDestroy(c->ids_ready);
    if (c->pinned_ids) (void)hipHostFree(c->pinned_ids);
    if (c->pinned_batch) (void)hipHostFree(c->pinned_batch);
    delete c;
}

// Two timing events for one interval of the timeline (kind 0 copy, 1
// kernel), or false when the timeline is off or full.
static bool timeline_pair(moe_cache* c, int kind, hipEvent_t* begin, hipEvent_t* end) {
    if (!c->timeline) return false;
    if ((int)c->tl_marks.size() >= c->max_marks) {
        c->truncated = 1;
        return false;
    }
    while (c->tl_events.size() < c->tl_used + 2) {
        hipEvent_t ev;
        if (hipEventCreate(&ev) != hipSuccess) {
            (void)hipGetLastError();
            c->truncated = 1;
            return false;
        }
        c->tl_events.push_back(ev);
    }
    *begin = c->tl_events[c->tl_used];
    *end = c->tl_events[c->tl_used + 1];
    c->tl_marks.emplace_back(kind, (int)c->tl_used);
    c->tl_used += 2;
    return true;
}

LaunchTiming cache_kernel_timing(moe_cache* c) {
    LaunchTiming t;
    hipEvent_t b, e;
    if (c && timeline_pair(c, 1, &b, &e)) {
        t.start = b;
        t.stop = e;
    }
    return t;
}

// Makes expert e of layer l resident; `protect` lists experts that must not
// be evicted.  Sets *slot and *missed.
// A layer's end-of-call event is re-recorded by every call, so it has to
// cover the reads of all earlier calls.  Calls on one stream do by stream
// order; a call on another stream first waits for the previous call's event.
static hipError_t join_layer_stream(LayerSlots& L, hipStream_t st) {
    if (!L.call_recorded || L.call_stream == st) return hipSuccess;
    return hipStreamWaitEvent(st, L.last_call, 0);
}

static hipError_t record_layer_call(LayerSlots& L, hipStream_t st) {
    const hipError_t err = hipEventRecord(L.last_call, st);
    if (err == hipSuccess) {
        L.call_recorded = true;
        L.call_stream = st;
    }
    return err;
}

// Whether the copy into slot s may still be running.  A copy seen complete
// is forgotten, so that later reads of the slot need neither a query nor a
// wait.
static hipError_t copy_pending(LayerSlots& L, int s, bool* pending) {
    *pending = false;
    if (!L.copy_recorded[s]) return hipSuccess;
    const hipError_t q = hipEventQuery(L.copy_done[s]);
    if (q == hipErrorNotReady) {
        (void)hipGetLastError();
        *pending = true;
        return hipSuccess;
    }
    if (q == hipSuccess) L.copy_recorded[s] = 0;
    return q;
}

static moe_status_t make_resident(moe_cache* c, int l, int e, const std::vector<int>& protect, int* slot,
                                  bool* missed) {
    LayerSlots& L = *c->layers[l];
    int s = L.policy.slot_of(e);
    if (s >= 0) {
        L.policy.touch(e);
        *slot = s;
        *missed = false;
        return MOE_OK;
    }
    if (!L.host_blob[e]) return fail(MOE_EINVAL, "expert cache: layer %d expert %d is not registered", l, e);
    int evicted = -1;
    s = L.policy.assign(e, protect, &evicted);
    if (s < 0) return fail(MOE_ENOSLOT, "expert cache: no slot of layer %d can be freed", l);
    if (evicted >= 0) {
        ++L.stats.evictions;
        L.fresh[evicted] = 0;
    }
    hipEvent_t tb = nullptr, te = nullptr;
    const bool stamp = timeline_pair(c, 0, &tb, &te);
    hipError_t err = hipSuccess;
    if (L.use_kind[s] == kUseSlotEvent) err = hipStreamWaitEvent(c->copy_stream, L.last_use[s], 0);
    if (L.use_kind[s] == kUseCallEvent) err = hipStreamWaitEvent(c->copy_stream, L.last_call, 0);
    if (err == hipSuccess && stamp) err = hipEventRecord(tb, c->copy_stream);
    if (err == hipSuccess)
        err = hipMemcpyAsync(c->slot_ptr(l, s), L.host_blob[e], c->expert_bytes, hipMemcpyHostToDevice,
                             c->copy_stream);
    if (err == hipSuccess && stamp) err = hipEventRecord(te, c->copy_stream);
    if (err == hipSuccess) err = hipEventRecord(L.copy_done[s], c->copy_stream);
    if (err != hipSuccess) {
        L.policy.release(e);
        return hip_fail(err, "expert cache copy");
    }
    L.copy_recorded[s] = 1;
    L.stats.h2d_bytes += c->expert_bytes;
    *slot = s;
    *missed = true;
    return MOE_OK;
}

// Brings in the experts of `want` (ids -1 skipped) that are not resident, in
// order, at most max_copies of them (< 0: no limit); the slot of each is
// chosen as for a miss with the whole list protected, so no expert of the
// list is evicted for another.  Each copy counts as a prefetch and the
// expert is marked fresh until its first use or its eviction.
static moe_status_t prefetch_experts(moe_cache* c, int l, const std::vector<int>& want, int max_copies) {
    LayerSlots& L = *c->layers[l];
    int copies = 0;
    for (int e : want) {
        if (e < 0 || L.policy.slot_of(e) >= 0) continue;
        if (max_copies >= 0 && copies >= max_copies) break;
        int s = -1;
        bool missed = false;
        moe_status_t r = make_resident(c, l, e, want, &s, &missed);
        if (r != MOE_OK) return r;
        ++L.stats.prefetches;
        L.fresh[e] = 1;
        ++copies;
    }
    return MOE_OK;
}

moe_status_t cache_prepare_token(moe_layer* layer, DecodeArgs& a, hipStream_t st, const int32_t* d_pred) {
    moe_cache* c = layer->cache;
    const int l = layer->cache_layer;
    LayerSlots& L = *c->layers[l];
    const int K = a.K;
    hipError_t err = join_layer_stream(L, st);
    if (err == hipSuccess)
        err = hipMemcpyAsync(c->pinned_ids, a.ids, sizeof(int32_t) * K, hipMemcpyDeviceToHost, st);
    if (err == hipSuccess && d_pred)
        err = hipMemcpyAsync(c->pinned_ids + 16, d_pred, sizeof(int32_t) * K, hipMemcpyDeviceToHost, st);
    if (err == hipSuccess) err = hipEventRecord(c->ids_ready, st);
    if (err == hipSuccess) err = hipEventSynchronize(c->ids_ready);
    if (err != hipSuccess) return hip_fail(err, "expert cache: reading the routing");
    std::vector<int> ids(c->pinned_ids, c->pinned_ids + K);
    // id -1: a choice that the top-p cut dropped (weight 0, never read)
    for (int e : ids)
        if (e < -1 || e >= c->cfg.n_experts || (e == -1 && !(layer->cfg.top_p < 1.0f)))
            return fail(MOE_EINVAL, "expert cache: routed id %d out of range", e);
    std::vector<int> guess;
    if (d_pred) {
        for (int j = 0; j < K; ++j) {
            const int e = c->pinned_ids[16 + j];
            if (e < -1 || e >= c->cfg.n_experts) return fail(MOE_EINVAL, "expert cache: predicted id %d out of range", e);
            if (e >= 0) guess.push_back(e);
        }
    }
    std::vector<int> needed;
    for (int e : ids)
        if (e >= 0) {
            ++L.usage[e];
            needed.push_back(e);
        }
    // how well the previous layer predicted this token's experts
    if (L.has_prediction) {
        for (int e : needed) {
            ++L.stats.predicted_uses;
            if (std::find(L.prediction.begin(), L.prediction.end(), e) != L.prediction.end()) ++L.stats.predicted_hits;
        }
        L.has_prediction = false;
    }
    std::vector<int> hit_slots, miss_slots, slot_of_j(K, -1);
    for (int j = 0; j < K; ++j) {
        a.blobs[j] = nullptr;
        if (ids[j] < 0) continue;
        int s = -1;
        bool missed = false;
        moe_status_t r = make_resident(c, l, ids[j], needed, &s, &missed);
        if (r != MOE_OK) return r;
        slot_of_j[j] = s;
        a.blobs[j] = c->slot_ptr(l, s);
        if (missed) {
            ++L.stats.misses;
            miss_slots.push_back(j);
            continue;
        }
        ++L.stats.hits;
        if (L.fresh[ids[j]]) {
            ++L.stats.prefetch_hits;
            L.fresh[ids[j]] = 0;
        }
        // a hit whose (prefetch) copy is still running goes with the misses,
        // so that it does not hold back the hits that are ready
        bool copying = false;
        err = copy_pending(L, s, &copying);
        if (err != hipSuccess) return hip_fail(err, "expert cache: copy event query");
        (copying ? miss_slots : hit_slots).push_back(j);
    }
    a.direct = 1;
    // gate/up of the hit experts first, then of the misses once copied (the
    // shared expert's ran in the router launch)
    for (int pass = 0; pass < 2; ++pass) {
        const std::vector<int>& js = pass == 0 ? hit_slots : miss_slots;
        if (js.empty()) continue;
        for (int j : js) {
            const int s = slot_of_j[j];
            if (L.copy_recorded[s]) {
                err = hipStreamWaitEvent(st, L.copy_done[s], 0);
                if (err != hipSuccess) return hip_fail(err, "expert cache: stream wait");
            }
        }
        a.use_slot_list = 1;
        a.n_slot_list = (int)js.size();
        for (size_t i = 0; i < js.size(); ++i) a.slot_list[i] = js[i];
        err = decode_routed_gateup(a, st, cache_kernel_timing(c));
        if (err != hipSuccess) return hip_fail(err, "gate/up kernel launch");
    }
    a.use_slot_list = 0;
    a.n_slot_list = 0;
    c->pending_slots.clear();
    for (int s : slot_of_j)
        if (s >= 0) c->pending_slots.push_back(s);
    c->pending_layer = l;
    // the next layer's predicted experts, queued behind this token's misses
    if (d_pred) {
        const int nl = layer->next->cache_layer;
        LayerSlots& N = *c->layers[nl];
        N.prediction = guess;
        N.has_prediction = true;
        const int limit = layer->max_prefetch > 0 ? layer->max_prefetch : K;
        moe_status_t r = prefetch_experts(c, nl, guess, limit);
        if (r != MOE_OK) return r;
    }
    return MOE_OK;
}

// One group of a batched call: tokens [g0, g1) of the launch sequence b,
// whose experts (routed ids in ids) are made resident first.
static moe_status_t run_group(moe_layer* layer, const BatchArgs& b, const int32_t* ids, int g0, int g1,
                              hipStream_t st) {
    moe_cache* c = layer->cache;
    const int l = layer->cache_layer;
    LayerSlots& L = *c->layers[l];
    const int K = b.K, E = b.E;
    std::vector<char> in(E, 0);
    for (int i = g0 * K; i < g1 * K; ++i)
        if (ids[i] >= 0) in[ids[i]] = 1;
    std::vector<int> distinct;
    for (int e = 0; e < E; ++e)
        if (in[e]) distinct.push_back(e);
    ExpertTable table;
    std::memset(&table, 0, sizeof table);
    std::vector<int> slots;
    for (int e : distinct) {
        int s = -1;
        bool missed = false;
        moe_status_t r = make_resident(c, l, e, distinct, &s, &missed);
        if (r != MOE_OK) return r;
        if (missed) {
            ++L.stats.misses;
        } else {
            ++L.stats.hits;
            if (L.fresh[e]) ++L.stats.prefetch_hits;
        }
        L.fresh[e] = 0;
        table.p[e] = c->slot_ptr(l, s);
        slots.push_back(s);
        bool copying = false;
        hipError_t err = copy_pending(L, s, &copying);
        if (err == hipSuccess && copying) err = hipStreamWaitEvent(st, L.copy_done[s], 0);
        if (err != hipSuccess) return hip_fail(err, "expert cache: stream wait");
    }
    BatchArgs g = b;
    const int n = g1 - g0;
    g.x = b.x + (size_t)g0 * b.H;
    g.xa = b.xa + (size_t)g0 * b.H;
    g.kx = b.kx + g0;
    g.ids = b.ids + (size_t)g0 * K;
    g.w = b.w + (size_t)g0 * K;
    g.y = b.y + (size_t)g0 * b.H;
    g.T = n;
    g.tile_tokens = batch_tile_tokens(b.codec, n, K, E);
    g.single_max = batch_single_max(g.tile_tokens);
    hipError_t err = batch_set_table(table, E, const_cast<const uint8_t**>(b.table), st);
    if (err == hipSuccess) err = batch_dispatch(g, st);
    if (err == hipSuccess) err = batch_gateup(g, st);
    if (err == hipSuccess && g.single_max > 0) err = batch_pair_gateup(g, st);
    if (err == hipSuccess) err = batch_hprep(g, st);
    if (err == hipSuccess) err = batch_down(g, st);
    if (err == hipSuccess && g.single_max > 0) err = batch_pair_down(g, st);
    if (err == hipSuccess) err = batch_combine(g, st);
    if (err != hipSuccess) return hip_fail(err, "batched launch behind the expert cache");
    for (int s : slots) {
        err = hipEventRecord(L.last_use[s], st);
        if (err != hipSuccess) return hip_fail(err, "expert cache: last-use event");
        L.use_kind[s] = kUseSlotEvent;
    }
    return MOE_OK;
}

moe_status_t cache_batch_forward(moe_layer* layer, const uint16_t* d_x, int T, float* d_y, int32_t* ids_base,
                                 float* w_base, hipStream_t st) {
    moe_cache* c = layer->cache;
    LayerSlots& L = *c->layers[layer->cache_layer];
    const moe_config_t& cfg = layer->cfg;
    const int K = cfg.top_k, E = cfg.n_experts, H = cfg.hidden;
    const int tb = layer->W.batch_tokens;
    L.has_prediction = false;  // a one-token prediction does not carry over to a batched call
    hipError_t jerr = join_layer_stream(L, st);
    if (jerr != hipSuccess) return hip_fail(jerr, "expert cache: stream wait");
    for (int t0 = 0; t0 < T; t0 += tb) {
        const int n = T - t0 < tb ? T - t0 : tb;
        BatchArgs b = batch_args(layer, d_x + (size_t)t0 * H, n, ids_base + (size_t)t0 * K, w_base + (size_t)t0 * K,
                                 d_y + (size_t)t0 * H);
        hipError_t err = batch_router(b, st);
        if (err == hipSuccess) err = batch_topk(b, true, st);
        if (err == hipSuccess)
            err = hipMemcpyAsync(c->pinned_batch, b.ids, sizeof(int32_t) * n * K, hipMemcpyDeviceToHost, st);
        if (err == hipSuccess) err = hipEventRecord(c->ids_ready, st);
        if (err == hipSuccess) err = hipEventSynchronize(c->ids_ready);
        if (err != hipSuccess) return hip_fail(err, "expert cache: batched routing");
        const int32_t* ids = c->pinned_batch;
        for (int i = 0; i < n * K; ++i) {
            const int e = ids[i];
            if (e < -1 || e >= E || (e == -1 && !(cfg.top_p < 1.0f)))
                return fail(MOE_EINVAL, "expert cache: routed id %d out of range", e);
            if (e >= 0) ++L.usage[e];
        }
        // consecutive groups of tokens whose unpinned experts fit the
        // unpinned slots together (one token always fits: pins leave top_k)
        const int room = c->slots - L.policy.n_pinned();
        std::vector<char> in(E);
        for (int g0 = 0; g0 < n;) {
            std::fill(in.begin(), in.end(), 0);
            int used = 0, t = g0;
            for (; t < n; ++t) {
                int add = 0;
                for (int j = 0; j < K; ++j) {
                    const int e = ids[t * K + j];
                    if (e >= 0 && !in[e] && !L.policy.is_pinned(e)) ++add;
                }
                if (t > g0 && used + add > room) break;
                used += add;
                for (int j = 0; j < K; ++j)
                    if (ids[t * K + j] >= 0) in[ids[t * K + j]] = 1;
            }
            moe_status_t r = run_group(layer, b, ids, g0, t, st);
            if (r != MOE_OK) return r;
            g0 = t;
        }
    }
    // the slots read here carry their own events; this one keeps the layer's
    // end-of-call event on the stream of its latest call
    jerr = record_layer_call(L, st);
    if (jerr != hipSuccess) return hip_fail(jerr, "expert cache: end-of-call event");
    return MOE_OK;
}

moe_status_t cache_finish_token(moe_layer* layer, hipStream_t st) {
    moe_cache* c = layer->cache;
    LayerSlots& L = *c->layers[c->pending_layer];
    // one event after the token's reads covers every slot it read
    hipError_t err = record_layer_call(L, st);
    if (err != hipSuccess) return hip_fail(err, "expert cache: end-of-call event");
    for (int s : c->pending_slots) L.use_kind[s] = kUseCallEvent;
    c->pending_slots.clear();
    c->pending_layer = -1;
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t expert_cache_create(const moe_config_t* cfg, int n_layers, int slots_per_layer, void* d_slot_pool,
                                 size_t pool_bytes, void* copy_stream, moe_cache_t** out) {
    if (!out) return fail(MOE_EINVAL, "expert_cache_create: out is NULL");
    *out = nullptr;
    moe_status_t st = validate_config(cfg);
    if (st != MOE_OK) return st;
    if (n_layers < 1 || slots_per_layer < cfg->top_k)
        return fail(MOE_EINVAL, "expert_cache_create: need n_layers >= 1 and slots_per_layer >= top_k (%d)",
                    cfg->top_k);
    if (slots_per_layer > cfg->n_experts)
        return fail(MOE_EINVAL, "expert_cache_create: more slots than experts");
    const size_t eb = blob_layout(cfg->hidden, cfg->inter, cfg->codec).total;
    const size_t need = eb * (size_t)n_layers * (size_t)slots_per_layer;
    if (!d_slot_pool || pool_bytes < need)
        return fail(MOE_EINVAL, "expert_cache_create: slot pool of %zu bytes is smaller than %zu", pool_bytes, need);
    if (reinterpret_cast<uintptr_t>(d_slot_pool) % 256) return fail(MOE_EINVAL, "slot pool must be 256-byte aligned");
    moe_cache* c = new (std::nothrow) moe_cache();
    if (!c) return fail(MOE_EINVAL, "expert_cache_create: out of host memory");
    c->cfg = *cfg;
    c->n_layers = n_layers;
    c->slots = slots_per_layer;
    c->pool = static_cast<uint8_t*>(d_slot_pool);
    c->expert_bytes = eb;
    c->copy_stream = static_cast<hipStream_t>(copy_stream);
    hipError_t err = hipHostMalloc(reinterpret_cast<void**>(&c->pinned_ids), sizeof(int32_t) * 32);
    if (err == hipSuccess)
        err = hipHostMalloc(reinterpret_cast<void**>(&c->pinned_batch), sizeof(int32_t) * kMaxDispatchEntries);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&c->ids_ready, hipEventDisableTiming);
    for (int l = 0; l < n_layers && err == hipSuccess; ++l) {
        LayerSlots* L = new (std::nothrow) LayerSlots(cfg->n_experts, slots_per_layer);
        if (!L) {
            destroy_cache(c);
            return fail(MOE_EINVAL, "expert_cache_create: out of host memory");
        }
        c->layers.push_back(L);
        L->host_blob.assign(cfg->n_experts, nullptr);
        L->copy_done.assign(slots_per_layer, nullptr);
        L->last_use.assign(slots_per_layer, nullptr);
        L->use_kind.assign(slots_per_layer, kUseNone);
        L->copy_recorded.assign(slots_per_layer, 0);
        L->usage.assign(cfg->n_experts, 0);
        L->fresh.assign(cfg->n_experts, 0);
        err = hipEventCreateWithFlags(&L->last_call, hipEventDisableTiming);
        for (int s = 0; s < slots_per_layer && err == hipSuccess; ++s) {
            err = hipEventCreateWithFlags(&L->copy_done[s], hipEventDisableTiming);
            if (err == hipSuccess) err = hipEventCreateWithFlags(&L->last_use[s], hipEventDisableTiming);
        }
    }
    if (err != hipSuccess) {
        destroy_cache(c);
        return hip_fail(err, "expert_cache_create");
    }
    *out = c;
    return MOE_OK;
}

moe_status_t expert_cache_register(moe_cache_t* cache, int layer, int expert, const void* h_pinned_blob,
                                   size_t bytes) {
    if (!cache || !h_pinned_blob) return fail(MOE_EINVAL, "expert_cache_register: NULL argument");
    if (layer < 0 || layer >= cache->n_layers || expert < 0 || expert >= cache->cfg.n_experts)
        return fail(MOE_EINVAL, "expert_cache_register: layer %d / expert %d out of range", layer, expert);
    if (bytes != cache->expert_bytes)
        return fail(MOE_EINVAL, "expert_cache_register: blob has %zu bytes, expected %zu", bytes, cache->expert_bytes);
    LayerSlots& L = *cache->layers[layer];
    if (L.host_blob[expert]) return fail(MOE_EINVAL, "expert_cache_register: layer %d expert %d registered twice",
                                         layer, expert);
    L.host_blob[expert] = h_pinned_blob;
    return MOE_OK;
}

moe_status_t expert_cache_prefetch(moe_cache_t* cache, int layer, const int32_t* h_experts, int n) {
    if (!cache || (n > 0 && !h_experts)) return fail(MOE_EINVAL, "expert_cache_prefetch: NULL argument");
    if (layer < 0 || layer >= cache->n_layers) return fail(MOE_EINVAL, "expert_cache_prefetch: bad layer %d", layer);
    if (n < 0 || n > cache->slots)
        return fail(MOE_ENOSLOT, "expert_cache_prefetch: %d experts do not fit in %d slots", n, cache->slots);
    std::vector<int> want(h_experts, h_experts + n);
    for (int e : want)
        if (e < 0 || e >= cache->cfg.n_experts) return fail(MOE_EINVAL, "expert_cache_prefetch: expert %d", e);
    return prefetch_experts(cache, layer, want, -1);
}

moe_status_t expert_cache_evict(moe_cache_t* cache, int layer, int expert) {
    if (!cache) return fail(MOE_EINVAL, "expert_cache_evict: cache is NULL");
    if (layer < 0 || layer >= cache->n_layers || expert < 0 || expert >= cache->cfg.n_experts)
        return fail(MOE_EINVAL, "expert_cache_evict: layer %d / expert %d out of range", layer, expert);
    LayerSlots& L = *cache->layers[layer];
    // The slot's next copy waits on the event that covers its last read, so freeing it now is safe.
    if (L.policy.release(expert) >= 0) ++L.stats.evictions;
    L.fresh[expert] = 0;
    return MOE_OK;
}

moe_status_t expert_cache_stats(const moe_cache_t* cache, int layer, moe_cache_stats_t* out) {
    if (!cache || !out) return fail(MOE_EINVAL, "expert_cache_stats: NULL argument");
    if (layer < 0 || layer >= cache->n_layers) return fail(MOE_EINVAL, "expert_cache_stats: bad layer %d", layer);
    *out = cache->layers[layer]->stats;
    out->pinned = (uint64_t)cache->layers[layer]->policy.n_pinned();
    return MOE_OK;
}

moe_status_t expert_cache_usage(const moe_cache_t* cache, int layer, uint64_t* h_counts) {
    if (!cache || !h_counts) return fail(MOE_EINVAL, "expert_cache_usage: NULL argument");
    if (layer < 0 || layer >= cache->n_layers) return fail(MOE_EINVAL, "expert_cache_usage: bad layer %d", layer);
    const std::vector<uint64_t>& u = cache->layers[layer]->usage;
    std::copy(u.begin(), u.end(), h_counts);
    return MOE_OK;
}

moe_status_t expert_cache_pin(moe_cache_t* cache, int layer, const int32_t* h_experts, int n) {
    if (!cache || (n > 0 && !h_experts)) return fail(MOE_EINVAL, "expert_cache_pin: NULL argument");
    if (layer < 0 || layer >= cache->n_layers) return fail(MOE_EINVAL, "expert_cache_pin: bad layer %d", layer);
    if (n < 0) return fail(MOE_EINVAL, "expert_cache_pin: n < 0");
    std::vector<int> want(h_experts, h_experts + n);
    LayerSlots& L = *cache->layers[layer];
    int fresh = 0;
    for (size_t i = 0; i < want.size(); ++i) {
        const int e = want[i];
        if (e < 0 || e >= cache->cfg.n_experts) return fail(MOE_EINVAL, "expert_cache_pin: expert %d", e);
        bool dup = false;
        for (size_t j = 0; j < i; ++j) dup = dup || want[j] == e;
        if (!dup && !L.policy.is_pinned(e)) ++fresh;
    }
    // a token's top_k experts must always find unpinned slots
    if (L.policy.n_pinned() + fresh > cache->slots - cache->cfg.top_k)
        return fail(MOE_ENOSLOT, "expert_cache_pin: %d pinned experts leave fewer than top_k (%d) of %d slots",
                    L.policy.n_pinned() + fresh, cache->cfg.top_k, cache->slots);
    for (int e : want) {
        if (L.policy.slot_of(e) < 0) {
            int s = -1;
            bool missed = false;
            moe_status_t r = make_resident(cache, layer, e, want, &s, &missed);
            if (r != MOE_OK) return r;
            ++L.stats.prefetches;
        }
        L.policy.pin(e);
    }
    return MOE_OK;
}

moe_status_t expert_cache_unpin(moe_cache_t* cache, int layer, const int32_t* h_experts, int n) {
    if (!cache || (n > 0 && !h_experts)) return fail(MOE_EINVAL, "expert_cache_unpin: NULL argument");
    if (layer < 0 || layer >= cache->n_layers) return fail(MOE_EINVAL, "expert_cache_unpin: bad layer %d", layer);
    if (n < 0) return fail(MOE_EINVAL, "expert_cache_unpin: n < 0");
    for (int i = 0; i < n; ++i)
        if (h_experts[i] < 0 || h_experts[i] >= cache->cfg.n_experts)
            return fail(MOE_EINVAL, "expert_cache_unpin: expert %d", h_experts[i]);
    for (int i = 0; i < n; ++i) cache->layers[layer]->policy.unpin(h_experts[i]);
    return MOE_OK;
}

moe_status_t expert_cache_autopin(moe_cache_t* cache, int layer, int n) {
    if (!cache) return fail(MOE_EINVAL, "expert_cache_autopin: cache is NULL");
    if (layer < 0 || layer >= cache->n_layers) return fail(MOE_EINVAL, "expert_cache_autopin: bad layer %d", layer);
    if (n < 0 || n > cache->slots - cache->cfg.top_k)
        return fail(MOE_ENOSLOT, "expert_cache_autopin: %d pinned experts leave fewer than top_k (%d) of %d slots", n,
                    cache->cfg.top_k, cache->slots);
    LayerSlots& L = *cache->layers[layer];
    const int E = cache->cfg.n_experts;
    for (int e = 0; e < E; ++e) L.policy.unpin(e);
    std::vector<int32_t> order(E);
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return L.usage[x] > L.usage[y]; });
    return expert_cache_pin(cache, layer, order.data(), n);
}

void expert_cache_destroy(moe_cache_t* cache) { destroy_cache(cache); }

moe_status_t moe_layer_attach_cache(moe_layer_t* layer, moe_cache_t* cache, int layer_id) {
    if (!layer || !cache) return fail(MOE_EINVAL, "moe_layer_attach_cache: NULL argument");
    if (layer_id < 0 || layer_id >= cache->n_layers)
        return fail(MOE_EINVAL, "moe_layer_attach_cache: layer_id %d out of range", layer_id);
    const moe_config_t &a = layer->cfg, &b = cache->cfg;
    if (a.hidden != b.hidden || a.inter != b.inter || a.n_experts != b.n_experts || a.top_k != b.top_k ||
        a.codec != b.codec)
        return fail(MOE_EINVAL, "moe_layer_attach_cache: cache and layer shapes differ");
    layer->cache = cache;
    layer->cache_layer = layer_id;
    return MOE_OK;
}

// Host-only replay of the slot policy on a routing trace (no GPU needed):
// trace [n_tokens][top_k] expert ids; returns hits/misses/evictions.
moe_status_t expert_cache_replay(int n_experts, int slots, int top_k, const int32_t* trace, int n_tokens,
                                 const int32_t* pinned, int n_pinned, uint64_t* hits, uint64_t* misses,
                                 uint64_t* evictions) {
    if (n_experts < 1 || slots < top_k || top_k < 1 || n_tokens < 0 || (n_tokens > 0 && !trace) || !hits ||
        !misses || !evictions || n_pinned < 0 || (n_pinned > 0 && !pinned) || n_pinned > slots - top_k)
        return fail(MOE_EINVAL, "expert_cache_replay: bad arguments");
    SlotPolicy p(n_experts, slots);
    for (int i = 0; i < n_pinned; ++i) {
        const int e = pinned[i];
        if (e < 0 || e >= n_experts) return fail(MOE_EINVAL, "expert_cache_replay: pinned id %d out of range", e);
        if (p.slot_of(e) < 0) {
            int ev = -1;
            if (p.assign(e, {}, &ev) < 0) return fail(MOE_ENOSLOT, "expert_cache_replay: no slot to pin");
        }
        p.pin(e);
    }
    *hits = *misses = *evictions = 0;
    for (int t = 0; t < n_tokens; ++t) {
        // id -1: a choice the top-p cut dropped (no lookup, as in the cache)
        std::vector<int> ids;
        for (int j = 0; j < top_k; ++j) {
            const int e = trace[(size_t)t * top_k + j];
            if (e < -1 || e >= n_experts) return fail(MOE_EINVAL, "expert_cache_replay: id %d out of range", e);
            if (e >= 0) ids.push_back(e);
        }
        for (int e : ids) {
            if (p.slot_of(e) >= 0) {
                p.touch(e);
                ++*hits;
            } else {
                int ev = -1;
                if (p.assign(e, ids, &ev) < 0) return fail(MOE_ENOSLOT, "expert_cache_replay: no slot");
                ++*misses;
                if (ev >= 0) ++*evictions;
            }
        }
    }
    return MOE_OK;
}

moe_status_t expert_cache_replay_prefetch(int n_experts, int slots, int top_k, const int32_t* trace,
                                          const int32_t* predicted, int n_tokens, int max_prefetch,
                                          const int32_t* pinned, int n_pinned, uint64_t* counts) {
    if (n_experts < 1 || slots < top_k || top_k < 1 || n_tokens < 0 || (n_tokens > 0 && (!trace || !predicted)) ||
        !counts || n_pinned < 0 || (n_pinned > 0 && !pinned) || n_pinned > slots - top_k || max_prefetch < 0)
        return fail(MOE_EINVAL, "expert_cache_replay_prefetch: bad arguments");
    SlotPolicy p(n_experts, slots);
    for (int i = 0; i < n_pinned; ++i) {
        const int e = pinned[i];
        if (e < 0 || e >= n_experts)
            return fail(MOE_EINVAL, "expert_cache_replay_prefetch: pinned id %d out of range", e);
        if (p.slot_of(e) < 0) {
            int ev = -1;
            if (p.assign(e, {}, &ev) < 0) return fail(MOE_ENOSLOT, "expert_cache_replay_prefetch: no slot to pin");
        }
        p.pin(e);
    }
    uint64_t hits = 0, misses = 0, evictions = 0, prefetches = 0, prefetch_hits = 0, pred_uses = 0, pred_hits = 0;
    std::vector<char> fresh(n_experts, 0);
    const int limit = max_prefetch > 0 ? max_prefetch : top_k;
    for (int t = 0; t < n_tokens; ++t) {
        std::vector<int> ids, guess;
        bool any = false;
        for (int j = 0; j < top_k; ++j) {
            const int e = trace[(size_t)t * top_k + j];
            const int g = predicted[(size_t)t * top_k + j];
            if (e < -1 || e >= n_experts || g < -1 || g >= n_experts)
                return fail(MOE_EINVAL, "expert_cache_replay_prefetch: id out of range at token %d", t);
            if (e >= 0) ids.push_back(e);
            if (g >= 0) guess.push_back(g);
            any = any || g != -1;
        }
        if (any) {
            // the prefetch the previous layer's call makes before this lookup
            int copies = 0;
            for (int e : guess) {
                if (p.slot_of(e) >= 0) continue;
                if (copies >= limit) break;
                int ev = -1;
                if (p.assign(e, guess, &ev) < 0) return fail(MOE_ENOSLOT, "expert_cache_replay_prefetch: no slot");
                if (ev >= 0) {
                    ++evictions;
                    fresh[ev] = 0;
                }
                fresh[e] = 1;
                ++prefetches;
                ++copies;
            }
            for (int e : ids) {
                ++pred_uses;
                if (std::find(guess.begin(), guess.end(), e) != guess.end()) ++pred_hits;
            }
        }
        for (int e : ids) {
            if (p.slot_of(e) >= 0) {
                p.touch(e);
                ++hits;
                if (fresh[e]) {
                    ++prefetch_hits;
                    fresh[e] = 0;
                }
            } else {
                int ev = -1;
                if (p.assign(e, ids, &ev) < 0) return fail(MOE_ENOSLOT, "expert_cache_replay_prefetch: no slot");
                ++misses;
                if (ev >= 0) {
                    ++evictions;
                    fresh[ev] = 0;
                }
            }
        }
    }
    counts[0] = hits;
    counts[1] = misses;
    counts[2] = evictions;
    counts[3] = prefetches;
    counts[4] = prefetch_hits;
    counts[5] = pred_uses;
    counts[6] = pred_hits;
    return MOE_OK;
}

moe_status_t moe_layer_set_next(moe_layer_t* layer, moe_layer_t* next, int max_prefetch) {
    if (!layer) return fail(MOE_EINVAL, "moe_layer_set_next: layer is NULL");
    if (max_prefetch < 0) return fail(MOE_EINVAL, "moe_layer_set_next: max_prefetch < 0");
    if (!next) {
        layer->next = nullptr;
        layer->max_prefetch = 0;
        return MOE_OK;
    }
    if (!layer->cache || !next->cache || layer->cache != next->cache)
        return fail(MOE_EINVAL, "moe_layer_set_next: both layers must be attached to the same expert cache");
    if (next == layer || next->cache_layer == layer->cache_layer)
        return fail(MOE_EINVAL, "moe_layer_set_next: the next layer must be another cache layer");
    if (!next->ws) return fail(MOE_EINVAL, "moe_layer_set_next: the next layer has no workspace");
    if (layer->ws && next->ws < layer->ws + layer->W.total && layer->ws < next->ws + next->W.total)
        return fail(MOE_EINVAL, "moe_layer_set_next: the layers' workspaces overlap");
    const moe_config_t &a = layer->cfg, &b = next->cfg;
    if (a.hidden != b.hidden || a.top_k != b.top_k)
        return fail(MOE_EINVAL, "moe_layer_set_next: the layers' hidden sizes or top_k differ");
    layer->next = next;
    layer->max_prefetch = max_prefetch;
    return MOE_OK;
}

moe_status_t expert_cache_timeline(moe_cache_t* cache, int enable, int max_marks) {
    if (!cache) return fail(MOE_EINVAL, "expert_cache_timeline: cache is NULL");
    if (max_marks < 0) return fail(MOE_EINVAL, "expert_cache_timeline: max_marks < 0");
    cache->timeline = enable != 0;
    cache->max_marks = max_marks > 0 ? max_marks : 65536;
    cache->tl_marks.clear();
    cache->tl_used = 0;
    cache->truncated = 0;
    return MOE_OK;
}

// Total length of a set of intervals' union; sorts and merges them in place.
static double merge_union(std::vector<std::pair<double, double>>& v) {
    std::sort(v.begin(), v.end());
    std::vector<std::pair<double, double>> m;
    for (const auto& iv : v) {
        if (!m.empty() && iv.first <= m.back().second)
            m.back().second = std::max(m.back().second, iv.second);
        else
            m.push_back(iv);
    }
    v.swap(m);
    double t = 0.0;
    for (const auto& iv : v) t += iv.second - iv.first;
    return t;
}

moe_status_t expert_cache_timeline_read(moe_cache_t* cache, moe_cache_timeline_t* out) {
    if (!cache || !out) return fail(MOE_EINVAL, "expert_cache_timeline_read: NULL argument");
    std::memset(out, 0, sizeof *out);
    out->truncated = cache->truncated;
    std::vector<std::pair<double, double>> iv[2];
    if (!cache->tl_marks.empty()) {
        hipEvent_t ref = cache->tl_events[cache->tl_marks[0].second];
        for (const auto& m : cache->tl_marks) {
            hipEvent_t b = cache->tl_events[m.second], e = cache->tl_events[m.second + 1];
            hipError_t err = hipEventSynchronize(e);
            float tb = 0.0f, te = 0.0f;
            if (err == hipSuccess) err = hipEventElapsedTime(&tb, ref, b);
            if (err == hipSuccess) err = hipEventElapsedTime(&te, ref, e);
            if (err != hipSuccess) {
                // an interval whose launch or copy was never enqueued
                (void)hipGetLastError();
                continue;
            }
            iv[m.first].emplace_back(tb, te);
        }
    }
    out->copies = iv[0].size();
    out->kernels = iv[1].size();
    double lo = 0.0, hi = 0.0;
    bool first = true;
    for (int k = 0; k < 2; ++k)
        for (const auto& x : iv[k]) {
            lo = first ? x.first : std::min(lo, x.first);
            hi = first ? x.second : std::max(hi, x.second);
            first = false;
        }
    out->copy_ms = merge_union(iv[0]);
    out->kernel_ms = merge_union(iv[1]);
    out->span_ms = first ? 0.0 : hi - lo;
    // intersection of the two unions (both sorted and disjoint now)
    double both = 0.0;
    size_t i = 0, j = 0;
    while (i < iv[0].size() && j < iv[1].size()) {
        const double a0 = std::max(iv[0][i].first, iv[1][j].first);
        const double a1 = std::min(iv[0][i].second, iv[1][j].second);
        if (a1 > a0) both += a1 - a0;
        if (iv[0][i].second < iv[1][j].second)
            ++i;
        else
            ++j;
    }
    out->overlap_ms = both;
    cache->tl_marks.clear();
    cache->tl_used = 0;
    cache->truncated = 0;
    return MOE_OK;
}

}  // extern "C"
