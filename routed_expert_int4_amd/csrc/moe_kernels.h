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
    float* logits;                   // [E] scratch
    unsigned* ticket;                // zero between calls
    int32_t* ids;                    // [K] routing output
    float* w;                        // [K]
    float* h;                        // [(K + S) * I] scratch
    float* y;                        // [H] output
    int H, I, E, G, TG, K, S;
    float rsf;
    // Expert-cache mode: routed slot j reads blobs[j] instead of
    // table[ids[j]] (the host resolved the routing before the launch).
    int direct;
    const uint8_t* blobs[16];
    // Optional subset of routed slots for the gate/up launch (n_slot_list
    // > 0): the launch covers slot_list[0 .. n_slot_list-1] only.
    int n_slot_list;
    int slot_list[16];
};

hipError_t decode_router_and_shared(const DecodeArgs& a, hipStream_t st);
hipError_t decode_routed_gateup(const DecodeArgs& a, hipStream_t st);
hipError_t decode_down_combine(const DecodeArgs& a, hipStream_t st);
bool decode_shape_supported(int hidden, int inter);

}  // namespace moe
