// Expert cache hooks used by moe_layer_forward.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_internal.h"
#include "moe_kernels.h"

namespace moe {

// After the router of one token was enqueued on `st`: waits for its ids,
// makes every selected expert resident (copies on the cache's copy stream),
// fills a.blobs / a.direct and enqueues the routed gate/up work, hits first,
// then misses and hits whose copy is still running, after their copies
// (stream waits on copy events).  With d_pred (device ids [top_k] of the
// linked next layer, predicted on this call's input and enqueued before this
// call), the prediction is read back in the same wait and the predicted
// experts of the next layer that are not resident are copied after this
// token's misses.
moe_status_t cache_prepare_token(moe_layer* L, DecodeArgs& a, hipStream_t st, const int32_t* d_pred);
// T > 1 tokens of a cached layer on the batched kernels: per launch sequence
// the routing is read back once, the tokens are split into consecutive groups
// whose distinct unpinned experts fit the layer's unpinned slots, and each
// group's distinct experts are made resident (ascending ids, one lookup per
// expert and group) before its dispatch, grouped gate/up and down run.
moe_status_t cache_batch_forward(moe_layer* L, const uint16_t* d_x, int T, float* d_y, int32_t* ids_base,
                                 float* w_base, hipStream_t st);
// Begin/end events for one kernel launch when the cache's timeline is on
// (empty otherwise).
LaunchTiming cache_kernel_timing(moe_cache* c);
// After the token's last kernel that reads the slots was enqueued: records
// the slots' last-use events.
moe_status_t cache_finish_token(moe_layer* L, hipStream_t st);

}  // namespace moe
