// Launch interface between the host library and the HIP kernels.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace moe {

// Arguments of the one-token decode path.  Every pointer is device memory.
struct DecodeArgs {
    const uint16_t* x;               // [H] bf16 bits
    const float* router_w;           // [E][H]
    const float* bias;               // [E]
    const uint8_t* const* table;     // [E] packed routed expert blobs
    const uint8_t* shared_blob;      // packed shared expert (when S == 1)
    float* s;                        // [E] router affinities sigmoid(logit) (scratch)
    float* sb;                       // [E] biased scores s + bias (scratch)
    unsigned* xpairs;                // activations as scaled fp16 pairs, per lane (scratch)
    int* kx;                         // their power-of-two scaling exponent (scratch)
    int32_t* ids;                    // [K] routing output
    float* w;                        // [K]
    const uint8_t** slot_blobs;      // [16] blobs of the routed slots, resolved once (scratch)
    float* h;                        // [(K + S) * I] scratch
    float* y;                        // [H] output
    int H, I, E, G, TG, K, S;
    float rsf;
    // Expert-cache mode: routed slot j reads blobs[j] instead of
    // table[ids[j]] (the host resolved the routing before the launch).
    int direct;
    const uint8_t* blobs[16];
    // Optional subset of routed slots for the gate/up launch: with
    // use_slot_list the launch covers slot_list[0 .. n_slot_list-1] only
    // (possibly none).
    int use_slot_list;
    int n_slot_list;
    int slot_list[16];
    // Whether this gate/up launch also covers the shared expert (its items
    // come first; they do not depend on the routing).
    int with_shared;
};

// Optional timing of one launch: when start is set the launch stamps start
// and stop with the kernel's own begin and end.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Router logits -> s, sb; activation pairs.
hipError_t decode_router(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
// Group-limited top-k from s, sb on one wave -> ids, w.
hipError_t decode_topk(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
// Gate/up + SwiGLU of the shared expert (with_shared) and the routed
// experts.  In table mode every wave also derives the routing itself from
// s, sb (and the first wave writes ids, w and slot_blobs), so no separate
// top-k launch is needed.
hipError_t decode_routed_gateup(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
// Down projection of every slot and the weighted combine into y.
hipError_t decode_down_combine(const DecodeArgs& a, hipStream_t st, const LaunchTiming& tm = {});
bool decode_shape_supported(int hidden, int inter, int top_k, int n_shared);

}  // namespace moe
