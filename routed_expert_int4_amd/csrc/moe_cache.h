// Expert cache hooks used by moe_layer_forward.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

// After the router of one token was enqueued on `st`: waits for its ids,
// makes every selected expert resident (copies on the cache's copy stream),
// fills a.blobs / a.direct and enqueues the routed gate/up work, hits first,
// then misses after their copies (stream waits on copy events).
moe_status_t cache_prepare_token(moe_layer* L, DecodeArgs& a, hipStream_t st);
// After the token's last kernel that reads the slots was enqueued: records
// the slots' last-use events.
moe_status_t cache_finish_token(moe_layer* L, hipStream_t st);

}  // namespace moe
