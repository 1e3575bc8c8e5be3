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
// device-to-host copy of the expert ids).
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

struct LayerSlots {
    explicit LayerSlots(int n_experts, int n_slots) : policy(n_experts, n_slots) {}
    SlotPolicy policy;
    std::vector<const void*> host_blob;    // [E] registered pinned blobs
    std::vector<hipEvent_t> copy_done;     // [slots]
    std::vector<hipEvent_t> last_use;      // [slots]
    std::vector<char> use_recorded;        // [slots]
    std::vector<char> copy_recorded;       // [slots]
    std::vector<uint64_t> usage;           // [E] routed uses (the learning cache's counts)
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
    int32_t* pinned_ids = nullptr;   // host-pinned staging of one token's ids
    hipEvent_t ids_ready = nullptr;
    std::vector<int> pending_slots;  // slots read by the token being enqueued
    int pending_layer = -1;

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
        delete L;
    }
    if (c->ids_ready) (void)hipEventDestroy(c->ids_ready);
    if (c->pinned_ids) (void)hipHostFree(c->pinned_ids);
    delete c;
}

// Makes expert e of layer l resident; `protect` lists experts that must not
// be evicted.  Sets *slot and *missed.
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
    if (evicted >= 0) ++L.stats.evictions;
    hipError_t err = hipSuccess;
    if (L.use_recorded[s]) err = hipStreamWaitEvent(c->copy_stream, L.last_use[s], 0);
    if (err == hipSuccess)
        err = hipMemcpyAsync(c->slot_ptr(l, s), L.host_blob[e], c->expert_bytes, hipMemcpyHostToDevice,
                             c->copy_stream);
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

moe_status_t cache_prepare_token(moe_layer* layer, DecodeArgs& a, hipStream_t st) {
    moe_cache* c = layer->cache;
    const int l = layer->cache_layer;
    LayerSlots& L = *c->layers[l];
    const int K = a.K;
    hipError_t err = hipMemcpyAsync(c->pinned_ids, a.ids, sizeof(int32_t) * K, hipMemcpyDeviceToHost, st);
    if (err == hipSuccess) err = hipEventRecord(c->ids_ready, st);
    if (err == hipSuccess) err = hipEventSynchronize(c->ids_ready);
    if (err != hipSuccess) return hip_fail(err, "expert cache: reading the routing");
    std::vector<int> ids(c->pinned_ids, c->pinned_ids + K);
    // id -1: a choice that the top-p cut dropped (weight 0, never read)
    for (int e : ids)
        if (e < -1 || e >= c->cfg.n_experts || (e == -1 && !(layer->cfg.top_p < 1.0f)))
            return fail(MOE_EINVAL, "expert cache: routed id %d out of range", e);
    std::vector<int> needed;
    for (int e : ids)
        if (e >= 0) {
            ++L.usage[e];
            needed.push_back(e);
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
        // a hit on a slot whose (prefetch) copy may still run also waits
        if (missed) {
            ++L.stats.misses;
            miss_slots.push_back(j);
        } else {
            ++L.stats.hits;
            hit_slots.push_back(j);
        }
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
        err = decode_routed_gateup(a, st);
        if (err != hipSuccess) return hip_fail(err, "gate/up kernel launch");
    }
    a.use_slot_list = 0;
    a.n_slot_list = 0;
    c->pending_slots.clear();
    for (int s : slot_of_j)
        if (s >= 0) c->pending_slots.push_back(s);
    c->pending_layer = l;
    return MOE_OK;
}

moe_status_t cache_finish_token(moe_layer* layer, hipStream_t st) {
    moe_cache* c = layer->cache;
    LayerSlots& L = *c->layers[c->pending_layer];
    for (int s : c->pending_slots) {
        hipError_t err = hipEventRecord(L.last_use[s], st);
        if (err != hipSuccess) return hip_fail(err, "expert cache: last-use event");
        L.use_recorded[s] = 1;
    }
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
    hipError_t err = hipHostMalloc(reinterpret_cast<void**>(&c->pinned_ids), sizeof(int32_t) * 16);
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
        L->use_recorded.assign(slots_per_layer, 0);
        L->copy_recorded.assign(slots_per_layer, 0);
        L->usage.assign(cfg->n_experts, 0);
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
    LayerSlots& L = *cache->layers[layer];
    for (int e : want) {
        if (L.policy.slot_of(e) >= 0) continue;
        int s = -1;
        bool missed = false;
        moe_status_t r = make_resident(cache, layer, e, want, &s, &missed);
        if (r != MOE_OK) return r;
        ++L.stats.prefetches;
    }
    return MOE_OK;
}

moe_status_t expert_cache_evict(moe_cache_t* cache, int layer, int expert) {
    if (!cache) return fail(MOE_EINVAL, "expert_cache_evict: cache is NULL");
    if (layer < 0 || layer >= cache->n_layers || expert < 0 || expert >= cache->cfg.n_experts)
        return fail(MOE_EINVAL, "expert_cache_evict: layer %d / expert %d out of range", layer, expert);
    LayerSlots& L = *cache->layers[layer];
    // The slot's next copy waits on its last-use event, so freeing it now is safe.
    if (L.policy.release(expert) >= 0) ++L.stats.evictions;
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

}  // extern "C"
