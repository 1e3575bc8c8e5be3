// Host-side state of a layer and helpers shared by the ABI translation units.
#pragma once

#include <cstddef>
#include <cstdint>
#include <utility>
#include <vector>

#include "../../include/moe.h"
#include "moe_kernels.h"
#include "moe_layout.h"

namespace moe {

struct WorkspaceLayout {
    size_t table = 0;          // [E] device blob pointers of the routed experts
    size_t control = 0;        // control words (cleared when bound)
    size_t control_bytes = 0;
    size_t sync = 0;           // counters of the fused launch (kSyncBytes, cleared when bound)
    size_t s = 0;              // [E] router affinities of the token in flight
    size_t sb = 0;             // [E] biased scores
    size_t xq = 0;             // activation operands of the token in flight
    size_t slot_blobs = 0;     // [16] blobs of the routed slots of the token in flight
    size_t kept = 0;           // [17] routed slots kept by the top-p cut (count first)
    size_t ids = 0;            // [max_T][K] when the caller passes no ids buffer
    size_t w = 0;              // [max_T][K]
    size_t h = 0;              // [K + S][I]
    // batched path (max_T > 1), sized for batch_tokens tokens per launch sequence
    int batch_tokens = 0;
    size_t b_logit_part = 0;   // [splits][Tb][E] partial router logits
    size_t b_xa = 0;           // [Tb][H] fp16
    size_t b_kx = 0;           // [Tb]
    size_t b_counts = 0, b_offsets = 0, b_perm = 0, b_inv = 0, b_distinct = 0, b_n_distinct = 0;
    size_t b_tiles = 0, b_n_tiles = 0, b_singles = 0, b_n_singles = 0;
    size_t b_h = 0;            // [P][I] fp32, P = Tb * (K + S)
    size_t b_ha_hi = 0, b_ha_lo = 0;  // [P][I] fp16
    size_t b_kh = 0;           // [P]
    size_t b_d = 0;            // [P][H] fp32
    size_t total = 0;
};

WorkspaceLayout workspace_layout(const moe_config_t* c, int max_T);
moe_status_t fail(moe_status_t code, const char* fmt, ...);
moe_status_t hip_fail(hipError_t e, const char* what);
moe_status_t validate_config(const moe_config_t* c);
moe_status_t validate_supported(const moe_config_t* c);

// The one-token decode path over T tokens with the per-call state at ws
// (laid out as W): token t reads x[t], writes y[t] and its routing to
// ids_base + t * ids_stride and w_base + t * w_stride.
// seq counts, per kernel, the launches made on ws since its control words
// were cleared (the in-kernel counters of the fused launch and of the
// gate/up + down launch count up across calls).
struct DecodeSeq {
    unsigned fused = 0;        // fused one-token launches
    unsigned gateup_down = 0;  // gate/up + down launches
};
moe_status_t decode_tokens(moe_layer* L, uint8_t* ws, const WorkspaceLayout& W, const uint16_t* d_x, int T,
                           float* d_y, int32_t* ids_base, int ids_stride, float* w_base, int w_stride,
                           DecodeSeq* seq, hipStream_t s);
// Kernel arguments of one token's decode launches, and of one batched launch
// sequence over n tokens starting at x (outputs at ids / w / y).
DecodeArgs decode_args(moe_layer* L, uint8_t* ws, const WorkspaceLayout& W, const uint16_t* x, int32_t* ids,
                       float* w, float* y);
BatchArgs batch_args(moe_layer* L, const uint16_t* x, int n, int32_t* ids, float* w, float* y);
// MOE_EHIP if a fused launch of this layer reported a wait that gave up.
moe_status_t check_layer_status(const moe_layer* L, const char* who);

constexpr unsigned kDefaultSpinLimit = 1u << 20;  // polls, about a second
// moe_layer_profile kinds: router, gate/up, down + combine, fused one-token
// launch, the batched path's grouped gate/up and down kernels alone, the
// batched GEMVs of single-entry experts, and the gate/up + down launch
constexpr int kProfileKinds = 9;

}  // namespace moe

struct moe_layer {
    moe_config_t cfg{};
    const float* router_w = nullptr;
    const float* bias = nullptr;
    std::vector<const uint8_t*> shared;
    std::vector<const uint8_t*> host_table;  // mirror of the device table
    bool experts_set = false;
    uint8_t* ws = nullptr;
    size_t ws_bytes = 0;
    int max_T = 0;
    moe::WorkspaceLayout W;
    moe_cache* cache = nullptr;
    int cache_layer = -1;
    // speculative next-layer prefetch (moe_layer_set_next): the linked layer
    // whose experts one-token calls predict and prefetch, and the copy limit
    moe_layer* next = nullptr;
    int max_prefetch = 0;
    // one-token calls: 3 = three launches (the default), 2 = the router
    // launch and one gate/up + down launch, 1 = one fused launch; 2 and 1
    // when their workgroups fit on the device at once, else three
    // (moe_layer_set_decode)
    int decode_launches = 3;
    unsigned spin_limit = moe::kDefaultSpinLimit;
    int fused_fits = -1;           // occupancy check of the fused launch (-1: not yet made)
    int gateup_down_fits = -1;     // occupancy check of the gate/up + down launch
    moe::DecodeSeq seq;            // in-kernel counted launches on the bound workspace
    unsigned* status = nullptr;    // host-visible word the fused kernel sets when a wait gives up
    // per-kernel event timing (moe_layer_profile)
    bool profiling = false;
    std::vector<hipEvent_t> prof_events;          // pool
    std::vector<std::pair<int, int>> prof_marks;  // (kind, index of start event)
    size_t prof_used = 0;
};
