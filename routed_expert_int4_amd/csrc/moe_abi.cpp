// Host side of the C ABI declared in include/moe.h: argument validation,
// expert packing, workspace carving and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_cache.h"
#include "moe_internal.h"
#include "moe_kernels.h"
#include "moe_layout.h"

namespace moe {

static thread_local std::string g_last_error;

moe_status_t fail(moe_status_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

moe_status_t hip_fail(hipError_t e, const char* what) {
    return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

moe_status_t validate_config(const moe_config_t* c) {
    if (!c) return fail(MOE_EINVAL, "config is NULL");
    if (c->hidden <= 0 || c->inter <= 0 || c->hidden % 32 || c->inter % 32)
        return fail(MOE_EINVAL, "hidden (%d) and inter (%d) must be positive multiples of 32", c->hidden, c->inter);
    if (c->n_experts <= 0 || c->n_groups <= 0 || c->n_experts % c->n_groups)
        return fail(MOE_EINVAL, "n_experts (%d) must be a positive multiple of n_groups (%d)", c->n_experts,
                    c->n_groups);
    const int gsize = c->n_experts / c->n_groups;
    if (gsize < 2) return fail(MOE_EINVAL, "groups need at least two experts (group size %d)", gsize);
    if (c->topk_group < 1 || c->topk_group > c->n_groups)
        return fail(MOE_EINVAL, "topk_group (%d) must be in [1, n_groups=%d]", c->topk_group, c->n_groups);
    if (c->top_k < 1 || c->top_k > c->topk_group * gsize)
        return fail(MOE_EINVAL, "top_k (%d) must be in [1, topk_group * group size = %d]", c->top_k,
                    c->topk_group * gsize);
    if (c->n_shared < 0) return fail(MOE_EINVAL, "n_shared must be >= 0");
    if (!(c->routed_scaling_factor == c->routed_scaling_factor))
        return fail(MOE_EINVAL, "routed_scaling_factor is NaN");
    if (!(c->top_p > 0.0f && c->top_p <= 1.0f)) return fail(MOE_EINVAL, "top_p must be in (0, 1]");
    if (c->codec != kCodecInt4 && c->codec != kCodecMxfp4 && c->codec != kCodecInt8 && c->codec != kCodecInt2)
        return fail(MOE_EINVAL, "unknown codec %d", c->codec);
    return MOE_OK;
}

moe_status_t validate_supported(const moe_config_t* c) {
    moe_status_t st = validate_config(c);
    if (st != MOE_OK) return st;
    if (c->top_k > 8) return fail(MOE_EUNSUPPORTED, "top_k must be at most 8 (got %d)", c->top_k);
    if (!decode_shape_supported(c->hidden, c->inter, c->top_k, c->n_shared) ||
        !batch_shape_supported(c->hidden, c->inter))
        return fail(MOE_EUNSUPPORTED, "no kernel for hidden=%d inter=%d", c->hidden, c->inter);
    if (c->n_experts > 256) return fail(MOE_EUNSUPPORTED, "n_experts > 256");
    if (c->n_experts % 16) return fail(MOE_EUNSUPPORTED, "n_experts must be a multiple of 16");
    const int epl = c->n_experts <= 64 ? 1 : (c->n_experts <= 128 ? 2 : 4);
    const int gsize = c->n_experts / c->n_groups;
    const int lpg = gsize / epl;
    if (gsize % epl || lpg < 1 || (lpg & (lpg - 1)) || lpg > 64)
        return fail(MOE_EUNSUPPORTED, "group size %d does not map onto lanes", gsize);
    if (c->n_shared > 1) return fail(MOE_EUNSUPPORTED, "at most one shared expert");
    return MOE_OK;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(const moe_config_t* c, int max_T) {
    WorkspaceLayout W;
    size_t o = 0;
    const int slots = c->top_k + c->n_shared;
    W.table = o;
    o = align256(o + sizeof(void*) * (size_t)c->n_experts);
    W.control = o;
    o = align256(o + 256);
    W.control_bytes = 256;
    W.sync = o;
    o = align256(o + kSyncBytes);
    W.s = o;
    o = align256(o + sizeof(float) * (size_t)c->n_experts);
    W.sb = o;
    o = align256(o + sizeof(float) * (size_t)c->n_experts);
    W.xq = o;  // 16 byte dwords + (corr, factor) per lane and chunk column
    o = align256(o + (size_t)chunks_per_lane(c->hidden / 32) * kWave * 18 * sizeof(unsigned));
    W.slot_blobs = o;
    o = align256(o + sizeof(void*) * 16);
    W.kept = o;
    o = align256(o + sizeof(int) * 17);
    W.ids = o;
    o = align256(o + sizeof(int32_t) * (size_t)max_T * c->top_k);
    W.w = o;
    o = align256(o + sizeof(float) * (size_t)max_T * c->top_k);
    W.h = o;
    o = align256(o + sizeof(float) * (size_t)slots * c->inter);
    if (max_T > 1) {
        const int tb = max_T < kMaxDispatchEntries / c->top_k ? max_T : kMaxDispatchEntries / c->top_k;
        const size_t E = (size_t)c->n_experts, H = (size_t)c->hidden, I = (size_t)c->inter;
        const size_t n = (size_t)tb * c->top_k, P = (size_t)tb * slots;
        W.batch_tokens = tb;
        auto take = [&](size_t& field, size_t bytes) {
            field = o;
            o = align256(o + bytes);
        };
        take(W.b_logit_part, sizeof(float) * (size_t)batch_router_splits(c->hidden) * tb * E);
        take(W.b_xa, 2 * tb * H);
        take(W.b_kx, sizeof(int) * tb);
        take(W.b_counts, sizeof(int32_t) * E);
        take(W.b_offsets, sizeof(int32_t) * (E + 1));
        take(W.b_perm, sizeof(int32_t) * n);
        take(W.b_inv, sizeof(int32_t) * n);
        take(W.b_distinct, sizeof(int32_t) * E);
        take(W.b_n_distinct, sizeof(int32_t));
        take(W.b_tiles, sizeof(Tile) * (size_t)batch_max_tiles(tb, c->top_k, c->n_experts, c->n_shared));
        take(W.b_n_tiles, sizeof(int32_t));
        take(W.b_singles, sizeof(Tile) * (n < E ? n : E));
        take(W.b_n_singles, sizeof(int32_t));
        take(W.b_h, sizeof(float) * P * I);
        take(W.b_ha_hi, 2 * P * I);
        take(W.b_ha_lo, 2 * P * I);
        take(W.b_kh, sizeof(int) * P);
        take(W.b_d, sizeof(float) * P * H);
    }
    W.total = o;
    return W;
}

// Scale arrays of one expert, permuted into the per-lane packs the kernels
// read (T = uint16_t fp16 bits or uint8_t E8M0 bytes).
template <typename T>
void pack_scale_arrays(uint8_t* dst, const BlobLayout& L, int H, int I, int codec, const T* gate_s, const T* up_s,
                       const T* down_s) {
    const int kh = H / 32, ki = I / 32, rp = row_pack(codec);
    const int p = gateup_rows(kh), pd = down_rows(H, ki, codec);
    // stored row v of half `half` is matrix row rp * v + half (int2: even
    // rows, then odd rows, each in its own arrays)
    for (int half = 0; half < rp; ++half) {
        T* gu = reinterpret_cast<T*>(dst + (half ? L.gu_s2 : L.gu_s));
        for (int v = 0; v < I / rp; ++v) {
            const size_t r = (size_t)rp * v + half;
            for (int g = 0; g < kh; ++g) {
                gu[gateup_scale_index(v, g, 0, kh, p)] = gate_s[r * kh + g];
                gu[gateup_scale_index(v, g, 1, kh, p)] = up_s[r * kh + g];
            }
        }
        T* dn = reinterpret_cast<T*>(dst + (half ? L.down_s2 : L.down_s));
        for (int v = 0; v < H / rp; ++v) {
            const size_t r = (size_t)rp * v + half;
            for (int g = 0; g < ki; ++g) dn[scale_index(v, g, ki, pd)] = down_s[r * ki + g];
        }
    }
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_expert_bytes(const moe_config_t* cfg) {
    if (validate_config(cfg) != MOE_OK) return 0;
    return blob_layout(cfg->hidden, cfg->inter, cfg->codec).total;
}

moe_status_t moe_expert_pack(const moe_config_t* cfg, const uint8_t* gate_q, const void* gate_s,
                             const uint8_t* up_q, const void* up_s, const uint8_t* down_q, const void* down_s,
                             void* dst_blob) {
    moe_status_t st = validate_config(cfg);
    if (st != MOE_OK) return st;
    if (!gate_q || !gate_s || !up_q || !up_s || !down_q || !down_s || !dst_blob)
        return fail(MOE_EINVAL, "moe_expert_pack: NULL pointer");
    const int H = cfg->hidden, I = cfg->inter;
    const BlobLayout L = blob_layout(H, I, cfg->codec);
    uint8_t* dst = static_cast<uint8_t*>(dst_blob);
    const size_t codes = (size_t)H * I / 2;
    const int kh = H / 32, ki = I / 32;
    const int rp = row_pack(cfg->codec);
    if ((I / rp) % gateup_rows(kh) || (H / rp) % down_rows(H, ki, cfg->codec))
        return fail(MOE_EUNSUPPORTED, "moe_expert_pack: rows not a multiple of the scale pack");
    const uint8_t* src_q[3] = {gate_q, up_q, down_q};
    const size_t dst_q[3] = {L.gate_q, L.up_q, L.down_q};
    if (cfg->codec == kCodecMxfp4) {
        // E8M0 byte 255 is NaN: refused rather than carried into the kernels
        const uint8_t* src_s[3] = {static_cast<const uint8_t*>(gate_s), static_cast<const uint8_t*>(up_s),
                                   static_cast<const uint8_t*>(down_s)};
        const size_t n_s = (size_t)H * I / 32;
        for (int m = 0; m < 3; ++m)
            for (size_t i = 0; i < n_s; ++i)
                if (src_s[m][i] == 255) return fail(MOE_EINVAL, "moe_expert_pack: E8M0 scale 255 (NaN)");
        // codes: E2M1 nibbles as they are
        for (int m = 0; m < 3; ++m) std::memcpy(dst + dst_q[m], src_q[m], codes);
        pack_scale_arrays(dst, L, H, I, cfg->codec, src_s[0], src_s[1], src_s[2]);
    } else if (cfg->codec == kCodecInt8) {
        // q = 16 hi + lo: high nibbles (signed, stored + 8) in the int4
        // planes, low nibbles (unsigned) in the low planes
        const size_t dst_lo[3] = {L.gate_lo, L.up_lo, L.down_lo};
        for (int m = 0; m < 3; ++m)
            for (size_t i = 0; i < codes; ++i) {
                const uint8_t a = src_q[m][2 * i], b = src_q[m][2 * i + 1];
                dst[dst_q[m] + i] = (uint8_t)((((a >> 4) ^ 8u) & 15u) | ((((b >> 4) ^ 8u) & 15u) << 4));
                dst[dst_lo[m] + i] = (uint8_t)((a & 15u) | ((b & 15u) << 4));
            }
        pack_scale_arrays(dst, L, H, I, cfg->codec, static_cast<const uint16_t*>(gate_s),
                          static_cast<const uint16_t*>(up_s), static_cast<const uint16_t*>(down_s));
    } else if (cfg->codec == kCodecInt2) {
        // stored row v, column c: nibble (q[2v][c] + 2) | (q[2v + 1][c] + 2) << 2
        // (flipping the sign bit of a two's complement field adds 2)
        const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
        for (int m = 0; m < 3; ++m) {
            const int C = cols[m];
            uint8_t* d = dst + dst_q[m];
            std::memset(d, 0, (size_t)rows[m] / 2 * (C / 2));
            for (int v = 0; v < rows[m] / 2; ++v) {
                const uint8_t* r0 = src_q[m] + (size_t)(2 * v) * (C / 4);
                const uint8_t* r1 = r0 + C / 4;
                for (int c = 0; c < C; ++c) {
                    const unsigned f0 = ((r0[c >> 2] >> (2 * (c & 3))) & 3u) ^ 2u;
                    const unsigned f1 = ((r1[c >> 2] >> (2 * (c & 3))) & 3u) ^ 2u;
                    d[(size_t)v * (C / 2) + (c >> 1)] |= (uint8_t)((f0 | (f1 << 2)) << (4 * (c & 1)));
                }
            }
        }
        pack_scale_arrays(dst, L, H, I, cfg->codec, static_cast<const uint16_t*>(gate_s),
                          static_cast<const uint16_t*>(up_s), static_cast<const uint16_t*>(down_s));
    } else {
        // codes: stored as q + 8 (flip bit 3 of every two's complement nibble)
        for (int m = 0; m < 3; ++m)
            for (size_t i = 0; i < codes; ++i) dst[dst_q[m] + i] = src_q[m][i] ^ 0x88u;
        pack_scale_arrays(dst, L, H, I, cfg->codec, static_cast<const uint16_t*>(gate_s),
                          static_cast<const uint16_t*>(up_s), static_cast<const uint16_t*>(down_s));
    }
    return MOE_OK;
}

size_t moe_workspace_bytes(const moe_config_t* cfg, int max_T) {
    if (validate_config(cfg) != MOE_OK || max_T < 1) return 0;
    return workspace_layout(cfg, max_T).total;
}

moe_status_t moe_layer_create(const moe_config_t* cfg, const float* d_router_w, const float* d_bias,
                              const void* const* d_shared_blobs, moe_layer_t** out) {
    if (!out) return fail(MOE_EINVAL, "moe_layer_create: out is NULL");
    *out = nullptr;
    moe_status_t st = validate_supported(cfg);
    if (st != MOE_OK) return st;
    if (!d_router_w || !d_bias) return fail(MOE_EINVAL, "moe_layer_create: NULL router weight or bias");
    if (cfg->n_shared > 0 && !d_shared_blobs) return fail(MOE_EINVAL, "moe_layer_create: NULL shared blobs");
    moe_layer* L = new (std::nothrow) moe_layer();
    if (!L) return fail(MOE_EINVAL, "moe_layer_create: out of host memory");
    L->cfg = *cfg;
    L->router_w = d_router_w;
    L->bias = d_bias;
    for (int s = 0; s < cfg->n_shared; ++s) {
        if (!d_shared_blobs[s]) {
            delete L;
            return fail(MOE_EINVAL, "moe_layer_create: shared blob %d is NULL", s);
        }
        L->shared.push_back(static_cast<const uint8_t*>(d_shared_blobs[s]));
    }
    L->host_table.assign((size_t)cfg->n_experts, nullptr);
    // host-visible status word of the fused decode launch (pinned, mapped)
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&L->status), 64, hipHostMallocDefault);
    if (e != hipSuccess) {
        delete L;
        return hip_fail(e, "moe_layer_create: hipHostMalloc(status word)");
    }
    *L->status = 0u;
    *out = L;
    return MOE_OK;
}

moe_status_t moe_layer_set_workspace(moe_layer_t* layer, void* d_ws, size_t bytes, int max_T) {
    if (!layer || !d_ws) return fail(MOE_EINVAL, "moe_layer_set_workspace: NULL argument");
    if (max_T < 1) return fail(MOE_EINVAL, "moe_layer_set_workspace: max_T must be >= 1");
    if (reinterpret_cast<uintptr_t>(d_ws) % 256) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
    const WorkspaceLayout W = workspace_layout(&layer->cfg, max_T);
    if (bytes < W.total)
        return fail(MOE_EINVAL, "workspace too small: %zu bytes given, %zu needed for max_T=%d", bytes, W.total,
                    max_T);
    hipError_t e = hipMemset(static_cast<uint8_t*>(d_ws) + W.control, 0, W.control_bytes);
    if (e == hipSuccess) e = hipMemset(static_cast<uint8_t*>(d_ws) + W.sync, 0, kSyncBytes);
    if (e != hipSuccess) return hip_fail(e, "hipMemset(workspace control)");
    layer->ws = static_cast<uint8_t*>(d_ws);
    layer->ws_bytes = bytes;
    layer->max_T = max_T;
    layer->W = W;
    layer->seq = DecodeSeq();  // the control words were just cleared
    *layer->status = 0u;
    if (layer->experts_set) {
        e = hipMemcpy(layer->ws + W.table, layer->host_table.data(), sizeof(void*) * layer->host_table.size(),
                      hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpy(expert table)");
    }
    return MOE_OK;
}

moe_status_t moe_layer_set_experts(moe_layer_t* layer, const void* const* d_blobs) {
    if (!layer || !d_blobs) return fail(MOE_EINVAL, "moe_layer_set_experts: NULL argument");
    if (layer->cache) return fail(MOE_EINVAL, "moe_layer_set_experts: layer uses an expert cache");
    for (int e = 0; e < layer->cfg.n_experts; ++e)
        if (!d_blobs[e]) return fail(MOE_EINVAL, "moe_layer_set_experts: blob %d is NULL", e);
    for (int e = 0; e < layer->cfg.n_experts; ++e) layer->host_table[e] = static_cast<const uint8_t*>(d_blobs[e]);
    // without a workspace the table is copied when one is bound (the
    // allocation-free entry point carries it in its own launch instead)
    if (layer->ws) {
        hipError_t e = hipMemcpy(layer->ws + layer->W.table, layer->host_table.data(),
                                 sizeof(void*) * layer->host_table.size(), hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpy(expert table)");
    }
    layer->experts_set = true;
    return MOE_OK;
}

void moe_layer_destroy(moe_layer_t* layer) {
    if (!layer) return;
    for (hipEvent_t e : layer->prof_events) (void)hipEventDestroy(e);
    if (layer->status) (void)hipHostFree(layer->status);
    delete layer;
}

moe_status_t moe_layer_profile(moe_layer_t* layer, int enable) {
    if (!layer) return fail(MOE_EINVAL, "moe_layer_profile: layer is NULL");
    layer->profiling = enable != 0;
    layer->prof_marks.clear();
    layer->prof_used = 0;
    return MOE_OK;
}

moe_status_t moe_layer_profile_read(moe_layer_t* layer, double* total_ms, uint64_t* launches) {
    if (!layer || !total_ms || !launches) return fail(MOE_EINVAL, "moe_layer_profile_read: NULL argument");
    for (int k = 0; k < kProfileKinds; ++k) {
        total_ms[k] = 0.0;
        launches[k] = 0;
    }
    for (const auto& m : layer->prof_marks) {
        hipEvent_t a = layer->prof_events[m.second], b = layer->prof_events[m.second + 1];
        hipError_t e = hipEventSynchronize(b);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
        if (e != hipSuccess) return hip_fail(e, "moe_layer_profile_read");
        total_ms[m.first] += ms;
        launches[m.first] += 1;
    }
    return check_layer_status(layer, "moe_layer_profile_read");
}

moe_status_t moe_layer_set_decode(moe_layer_t* layer, int launches, unsigned spin_limit) {
    if (!layer) return fail(MOE_EINVAL, "moe_layer_set_decode: layer is NULL");
    if (launches < 1 || launches > 3) return fail(MOE_EINVAL, "moe_layer_set_decode: launches must be 1, 2 or 3");
    layer->decode_launches = launches;
    layer->spin_limit = spin_limit ? spin_limit : kDefaultSpinLimit;
    return MOE_OK;
}

}  // extern "C"

namespace moe {

DecodeArgs decode_args(moe_layer_t* L, uint8_t* ws, const WorkspaceLayout& W, const uint16_t* x, int32_t* ids,
                       float* w, float* y) {
    DecodeArgs a;
    const moe_config_t& c = L->cfg;
    a.x = x;
    a.router_w = L->router_w;
    a.bias = L->bias;
    a.table = L->cache ? nullptr : reinterpret_cast<const uint8_t* const*>(ws + W.table);
    a.counter = reinterpret_cast<unsigned*>(ws + W.control);
    a.shared_blob = c.n_shared > 0 ? L->shared[0] : nullptr;
    a.s = reinterpret_cast<float*>(ws + W.s);
    a.sb = reinterpret_cast<float*>(ws + W.sb);
    a.xq = reinterpret_cast<unsigned*>(ws + W.xq);
    a.slot_blobs = reinterpret_cast<const uint8_t**>(ws + W.slot_blobs);
    a.kept = !L->cache && c.top_p < 1.0f ? reinterpret_cast<int*>(ws + W.kept) : nullptr;
    a.ids = ids;
    a.w = w;
    a.h = reinterpret_cast<float*>(ws + W.h);
    a.y = y;
    a.H = c.hidden;
    a.I = c.inter;
    a.E = c.n_experts;
    a.G = c.n_groups;
    a.TG = c.topk_group;
    a.K = c.top_k;
    a.S = c.n_shared;
    a.rsf = c.routed_scaling_factor;
    a.top_p = c.top_p;
    a.codec = c.codec;
    a.direct = 0;
    a.use_slot_list = 0;
    a.n_slot_list = 0;
    for (int j = 0; j < 16; ++j) {
        a.blobs[j] = nullptr;
        a.slot_list[j] = 0;
    }
    return a;
}

// Per-launch timing when profiling is on.  In kernel mode the two events are
// handed to the launch (stamped with the kernel's own begin and end); in
// span mode they are recorded around whatever is enqueued between the
// constructor and end().  Events come from a pool that grows on demand and is
// reused after moe_layer_profile resets the marks.
class ProfileScope {
public:
    enum Mode { kKernel, kSpan };
    ProfileScope(moe_layer* L, int kind, hipStream_t s, Mode mode) : L_(L), s_(s), mode_(mode) {
        if (!L_->profiling) return;
        while (L_->prof_events.size() < L_->prof_used + 2) {
            hipEvent_t ev;
            if (hipEventCreate(&ev) != hipSuccess) return;
            L_->prof_events.push_back(ev);
        }
        idx_ = (int)L_->prof_used;
        L_->prof_used += 2;
        if (mode_ == kSpan) (void)hipEventRecord(L_->prof_events[idx_], s_);
        L_->prof_marks.emplace_back(kind, idx_);
    }
    LaunchTiming timing() const {
        LaunchTiming t;
        if (idx_ >= 0 && mode_ == kKernel) {
            t.start = L_->prof_events[idx_];
            t.stop = L_->prof_events[idx_ + 1];
        }
        return t;
    }
    void end() {
        if (idx_ >= 0 && mode_ == kSpan) (void)hipEventRecord(L_->prof_events[idx_ + 1], s_);
        idx_ = -1;
    }
    ~ProfileScope() { end(); }

private:
    moe_layer* L_;
    hipStream_t s_;
    Mode mode_;
    int idx_ = -1;
};

// Arguments of one batched launch sequence over n tokens (n <= batch_tokens)
// starting at x, with outputs at ids/w/y (any may be null for the router-only
// or dispatch-only uses).
BatchArgs batch_args(moe_layer_t* L, const uint16_t* x, int n, int32_t* ids, float* w, float* y) {
    BatchArgs b;
    const moe_config_t& c = L->cfg;
    const WorkspaceLayout& W = L->W;
    uint8_t* ws = L->ws;
    b.x = x;
    b.router_w = L->router_w;
    b.bias = L->bias;
    b.table = reinterpret_cast<const uint8_t* const*>(ws + W.table);
    b.shared_blob = c.n_shared > 0 ? L->shared[0] : nullptr;
    b.logit_part = reinterpret_cast<float*>(ws + W.b_logit_part);
    b.xa = reinterpret_cast<uint16_t*>(ws + W.b_xa);
    b.kx = reinterpret_cast<int*>(ws + W.b_kx);
    b.ids = ids;
    b.w = w;
    b.counts = reinterpret_cast<int32_t*>(ws + W.b_counts);
    b.offsets = reinterpret_cast<int32_t*>(ws + W.b_offsets);
    b.perm = reinterpret_cast<int32_t*>(ws + W.b_perm);
    b.inv = reinterpret_cast<int32_t*>(ws + W.b_inv);
    b.distinct = reinterpret_cast<int32_t*>(ws + W.b_distinct);
    b.n_distinct = reinterpret_cast<int32_t*>(ws + W.b_n_distinct);
    b.tiles = reinterpret_cast<Tile*>(ws + W.b_tiles);
    b.n_tiles = reinterpret_cast<int32_t*>(ws + W.b_n_tiles);
    b.singles = reinterpret_cast<Tile*>(ws + W.b_singles);
    b.n_singles = reinterpret_cast<int32_t*>(ws + W.b_n_singles);
    b.h = reinterpret_cast<float*>(ws + W.b_h);
    b.ha_hi = reinterpret_cast<uint16_t*>(ws + W.b_ha_hi);
    b.ha_lo = reinterpret_cast<uint16_t*>(ws + W.b_ha_lo);
    b.kh = reinterpret_cast<int*>(ws + W.b_kh);
    b.d = reinterpret_cast<float*>(ws + W.b_d);
    b.y = y;
    b.T = n;
    b.H = c.hidden;
    b.I = c.inter;
    b.E = c.n_experts;
    b.G = c.n_groups;
    b.TG = c.topk_group;
    b.K = c.top_k;
    b.S = c.n_shared;
    b.down_p = down_rows(c.hidden, c.inter / 32, c.codec);
    b.router_splits = batch_router_splits(c.hidden);
    b.rsf = c.routed_scaling_factor;
    b.top_p = c.top_p;
    b.codec = c.codec;
    b.tile_tokens = batch_tile_tokens(c.codec, n, c.top_k, c.n_experts);
    b.single_max = batch_single_max(b.tile_tokens);
    return b;
}

static moe_status_t check_call(moe_layer_t* L, const uint16_t* d_x, int T, const char* who) {
    if (!L) return fail(MOE_EINVAL, "%s: layer is NULL", who);
    if (T < 0) return fail(MOE_EINVAL, "%s: T < 0", who);
    if (!L->ws) return fail(MOE_EINVAL, "%s: no workspace bound", who);
    if (T > L->max_T) return fail(MOE_EINVAL, "%s: T=%d exceeds the workspace's max_T=%d", who, T, L->max_T);
    if (T > 0 && !d_x) return fail(MOE_EINVAL, "%s: x is NULL", who);
    return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status_t moe_router_topk(moe_layer_t* layer, const uint16_t* d_x, int T, int32_t* d_ids, float* d_w,
                             void* stream) {
    moe_status_t st = check_call(layer, d_x, T, "moe_router_topk");
    if (st != MOE_OK) return st;
    if (T > 0 && (!d_ids || !d_w)) return fail(MOE_EINVAL, "moe_router_topk: NULL ids or w");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const moe_config_t& c = layer->cfg;
    if (T > 1) {
        const int tb = layer->W.batch_tokens;
        for (int t0 = 0; t0 < T; t0 += tb) {
            const int n = T - t0 < tb ? T - t0 : tb;
            BatchArgs b = batch_args(layer, d_x + (size_t)t0 * c.hidden, n, d_ids + (size_t)t0 * c.top_k,
                                     d_w + (size_t)t0 * c.top_k, nullptr);
            hipError_t e = batch_router(b, s);
            if (e == hipSuccess) e = batch_topk(b, false, s);
            if (e != hipSuccess) return hip_fail(e, "batched router/top-k launch");
        }
        return MOE_OK;
    }
    for (int t = 0; t < T; ++t) {
        DecodeArgs a = decode_args(layer, layer->ws, layer->W, d_x + (size_t)t * c.hidden, d_ids + (size_t)t * c.top_k,
                                   d_w + (size_t)t * c.top_k, nullptr);
        hipError_t e = decode_router(a, s);
        if (e != hipSuccess) return hip_fail(e, "router kernel launch");
    }
    return MOE_OK;
}

moe_status_t moe_layer_forward(moe_layer_t* layer, const uint16_t* d_x, int T, float* d_y, int32_t* d_ids,
                               float* d_w, void* stream) {
    moe_status_t st = check_call(layer, d_x, T, "moe_layer_forward");
    if (st != MOE_OK) return st;
    st = check_layer_status(layer, "moe_layer_forward");
    if (st != MOE_OK) return st;
    if (T > 0 && !d_y) return fail(MOE_EINVAL, "moe_layer_forward: y is NULL");
    if (!layer->cache && !layer->experts_set)
        return fail(MOE_EINVAL, "moe_layer_forward: no experts set and no cache attached");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const moe_config_t& c = layer->cfg;
    int32_t* ids_base = d_ids ? d_ids : reinterpret_cast<int32_t*>(layer->ws + layer->W.ids);
    float* w_base = d_w ? d_w : reinterpret_cast<float*>(layer->ws + layer->W.w);
    // The batched kernels cover every codec (with or without the top-p cut;
    // int2 where hidden is a multiple of 512 and inter of 256), behind an
    // expert cache too; other T > 1 calls run as T one-token passes below.
    if (T > 1 && layer->cache && batch_codec_supported(c.codec, c.hidden, c.inter))
        return cache_batch_forward(layer, d_x, T, d_y, ids_base, w_base, s);
    if (T > 1 && !layer->cache && batch_codec_supported(c.codec, c.hidden, c.inter)) {
        // batch union: every distinct expert of a launch sequence is read once
        const int tb = layer->W.batch_tokens;
        for (int t0 = 0; t0 < T; t0 += tb) {
            const int n = T - t0 < tb ? T - t0 : tb;
            BatchArgs b = batch_args(layer, d_x + (size_t)t0 * c.hidden, n, ids_base + (size_t)t0 * c.top_k,
                                     w_base + (size_t)t0 * c.top_k, d_y + (size_t)t0 * c.hidden);
            ProfileScope p0(layer, 0, s, ProfileScope::kSpan);
            hipError_t e = batch_router(b, s);
            if (e == hipSuccess) e = batch_topk(b, true, s);
            if (e == hipSuccess) e = batch_dispatch(b, s);
            if (e != hipSuccess) return hip_fail(e, "batched routing launch");
            p0.end();
            ProfileScope p1(layer, 1, s, ProfileScope::kSpan);
            {
                ProfileScope k4(layer, 4, s, ProfileScope::kKernel);
                e = batch_gateup(b, s, k4.timing());
            }
            if (e == hipSuccess && b.single_max > 0) {
                ProfileScope k6(layer, 6, s, ProfileScope::kKernel);
                e = batch_pair_gateup(b, s, k6.timing());
            }
            if (e == hipSuccess) e = batch_hprep(b, s);
            if (e != hipSuccess) return hip_fail(e, "batched gate/up launch");
            p1.end();
            ProfileScope p2(layer, 2, s, ProfileScope::kSpan);
            {
                ProfileScope k5(layer, 5, s, ProfileScope::kKernel);
                e = batch_down(b, s, k5.timing());
            }
            if (e == hipSuccess && b.single_max > 0) {
                ProfileScope k7(layer, 7, s, ProfileScope::kKernel);
                e = batch_pair_down(b, s, k7.timing());
            }
            if (e == hipSuccess) e = batch_combine(b, s);
            if (e != hipSuccess) return hip_fail(e, "batched down/combine launch");
            p2.end();
        }
        return MOE_OK;
    }
    return decode_tokens(layer, layer->ws, layer->W, d_x, T, d_y, ids_base, c.top_k, w_base, c.top_k,
                         &layer->seq, s);
}

}  // extern "C"

namespace moe {

moe_status_t check_layer_status(const moe_layer* L, const char* who) {
    if (L->status && __atomic_load_n(L->status, __ATOMIC_ACQUIRE) != 0u)
        return fail(MOE_EHIP, "%s: a wait inside the fused decode launch gave up (its workgroups were not all "
                    "resident at once); outputs since then are not valid; bind the workspace again to reset", who);
    return MOE_OK;
}

// Whether the fused one-token launch serves this layer: not behind an expert
// cache (the host must see each token's routing), an instance for the shape
// and codec, and every workgroup resident at once (occupancy per CU times
// the CU count covers the grid; checked once per layer).
static bool use_fused(moe_layer_t* L, const DecodeArgs& a) {
    if (L->cache || L->decode_launches != 1) return false;
    if (L->fused_fits < 0) {
        L->fused_fits = 0;
        int threads = 0, per_cu = 0, dev = 0, cus = 0;
        const int grid = fused_grid(a, &threads);
        const void* fn = fused_kernel_function(a);
        if (grid > 0 && fn && hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) == hipSuccess)
            L->fused_fits = (long long)per_cu * cus >= grid ? 1 : 0;
        (void)hipGetLastError();
    }
    return L->fused_fits == 1;
}

// Whether the gate/up + down launch serves this layer (after the router
// launch): as for the fused launch, not behind an expert cache, an instance
// for the shape and codec, and every workgroup resident at once.
static bool use_gateup_down(moe_layer_t* L, const DecodeArgs& a) {
    if (L->cache || L->decode_launches != 2) return false;
    if (L->gateup_down_fits < 0) {
        L->gateup_down_fits = 0;
        int threads = 0, per_cu = 0, dev = 0, cus = 0;
        const int grid = gateup_down_grid(a, &threads);
        const void* fn = gateup_down_kernel_function(a);
        if (grid > 0 && fn && hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) == hipSuccess)
            L->gateup_down_fits = (long long)per_cu * cus >= grid ? 1 : 0;
        (void)hipGetLastError();
    }
    return L->gateup_down_fits == 1;
}

moe_status_t decode_tokens(moe_layer_t* layer, uint8_t* ws, const WorkspaceLayout& W, const uint16_t* d_x, int T,
                           float* d_y, int32_t* ids_base, int ids_stride, float* w_base, int w_stride,
                           DecodeSeq* seq, hipStream_t s) {
    const moe_config_t& c = layer->cfg;
    moe_status_t st = MOE_OK;
    if (layer->cache && layer->next) {
        // the prediction runs on the next layer's workspace, which must not
        // hold this call's state
        const moe_layer* nx = layer->next;
        if (!nx->ws || (nx->ws < ws + W.total && ws < nx->ws + nx->W.total))
            return fail(MOE_EINVAL, "moe_layer_forward: the linked next layer needs a workspace of its own");
    }
    for (int t = 0; t < T; ++t) {
        DecodeArgs a = decode_args(layer, ws, W, d_x + (size_t)t * c.hidden, ids_base + (size_t)t * ids_stride,
                                   w_base + (size_t)t * w_stride, d_y + (size_t)t * c.hidden);
        if (use_fused(layer, a)) {
            FusedArgs f;
            f.h_done = reinterpret_cast<unsigned*>(ws + W.sync + kSyncHDone);
            f.shared_done = reinterpret_cast<unsigned*>(ws + W.sync + kSyncSharedDone);
            f.s_rec = reinterpret_cast<unsigned long long*>(ws + W.sync + kSyncScoreRecords);
            f.sb_rec = f.s_rec + kSyncMaxExperts;
            f.status = layer->status;
            f.seq = ++seq->fused;
            f.spin_limit = layer->spin_limit;
            ProfileScope pf(layer, 3, s, ProfileScope::kKernel);
            hipError_t e = decode_fused(a, f, s, pf.timing());
            if (e != hipSuccess) return hip_fail(e, "fused decode launch");
            continue;
        }
        // a kernel that moe_layer_profile does not time is stamped for the
        // cache's copy/compute timeline when that is on
        auto stamp = [&](const ProfileScope& p) {
            LaunchTiming t = p.timing();
            return t.start || !layer->cache ? t : cache_kernel_timing(layer->cache);
        };
        ProfileScope p0(layer, 0, s, ProfileScope::kKernel);
        hipError_t e = decode_router(a, s, stamp(p0));
        if (e != hipSuccess) return hip_fail(e, "router kernel launch");
        p0.end();
        // speculative prefetch: the linked next layer's router and top-k on
        // this token's input (no shared expert work), into that layer's
        // one-token routing slots
        const int32_t* d_pred = nullptr;
        if (layer->cache && layer->next) {
            moe_layer* nx = layer->next;
            DecodeArgs pa = decode_args(nx, nx->ws, nx->W, a.x, reinterpret_cast<int32_t*>(nx->ws + nx->W.ids),
                                        reinterpret_cast<float*>(nx->ws + nx->W.w), nullptr);
            pa.S = 0;
            e = decode_router(pa, s, cache_kernel_timing(layer->cache));
            if (e != hipSuccess) return hip_fail(e, "next-layer router launch");
            d_pred = pa.ids;
        }
        if (!layer->cache && use_gateup_down(layer, a)) {
            FusedArgs f{};
            f.h_done = reinterpret_cast<unsigned*>(ws + W.sync + kSyncGateUpDownDone);
            f.status = layer->status;
            f.seq = ++seq->gateup_down;
            f.spin_limit = layer->spin_limit;
            ProfileScope p8(layer, 8, s, ProfileScope::kKernel);
            e = decode_gateup_down(a, f, s, p8.timing());
            if (e != hipSuccess) return hip_fail(e, "gate/up + down kernel launch");
            continue;
        }
        ProfileScope p1(layer, 1, s, layer->cache ? ProfileScope::kSpan : ProfileScope::kKernel);
        if (layer->cache) {
            // the host needs the routing: the cache reads it back, resolves
            // it, copies missing experts and enqueues the routed gate/up
            // (hits first)
            st = cache_prepare_token(layer, a, s, d_pred);
            if (st != MOE_OK) return st;
        } else {
            e = decode_routed_gateup(a, s, p1.timing());
            if (e != hipSuccess) return hip_fail(e, "gate/up kernel launch");
        }
        p1.end();
        ProfileScope p2(layer, 2, s, ProfileScope::kKernel);
        e = decode_down_combine(a, s, stamp(p2));
        if (e != hipSuccess) return hip_fail(e, "down/combine kernel launch");
        p2.end();
        if (layer->cache) {
            st = cache_finish_token(layer, s);
            if (st != MOE_OK) return st;
        }
    }
    return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status_t moe_dispatch(moe_layer_t* layer, const int32_t* d_ids, int T, int32_t* d_counts, int32_t* d_offsets,
                          int32_t* d_perm, int32_t* d_distinct, int32_t* d_n_distinct, void* stream) {
    if (!layer) return fail(MOE_EINVAL, "moe_dispatch: layer is NULL");
    if (T < 0) return fail(MOE_EINVAL, "moe_dispatch: T < 0");
    if (T == 0) return MOE_OK;
    if (!d_ids || !d_counts || !d_offsets || !d_perm || !d_distinct || !d_n_distinct)
        return fail(MOE_EINVAL, "moe_dispatch: NULL argument");
    if (!layer->ws) return fail(MOE_EINVAL, "moe_dispatch: no workspace bound");
    if (T > layer->W.batch_tokens)
        return fail(MOE_EINVAL, "moe_dispatch: T=%d exceeds the workspace's batch of %d tokens", T,
                    layer->W.batch_tokens);
    BatchArgs b = batch_args(layer, nullptr, T, const_cast<int32_t*>(d_ids), nullptr, nullptr);
    b.counts = d_counts;
    b.offsets = d_offsets;
    b.perm = d_perm;
    b.distinct = d_distinct;
    b.n_distinct = d_n_distinct;
    hipError_t e = batch_dispatch(b, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dispatch kernel launch");
    return MOE_OK;
}

}  // extern "C"
