// Allocation-free variant of the layer forward (moe_layer_forward_noalloc):
// the per-call device state that moe_layer_forward keeps in the caller's
// workspace lives here in one file-scope device array instead, so a caller
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc) needs no workspace.
//
// The array is the library's own: each GPU the library runs on holds one
// copy until the process ends.  Host code never uses the array's name as an
// address; it looks up each device's copy once (hipGetSymbolAddress, with
// that device current) and passes that address to the kernels.
//
// Every call on a GPU shares that GPU's array: calls that overlap on one GPU
// (two streams, two host threads) race and must be ordered by the caller.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"
#include "moe_kernels.h"

namespace moe {
namespace {

// Largest per-call state the variant serves: the one-token decode layout of
// the biggest supported shape (hidden 8192, intermediate 4096, 256 experts,
// top-8 + 1 shared) needs about 186 KiB.
constexpr size_t kScratchBytes = 256 * 1024;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// The expert pointer table travels as a kernel argument (2 KiB), so putting
// it in device memory needs no host-to-device copy from pageable memory.
struct TableArg {
    const uint8_t* p[256];
};

// Writes the layer's table into the array and clears the control and sync
// words the decode kernels expect to find at zero.
__global__ void __launch_bounds__(256) noalloc_setup_kernel(TableArg t, int n, const uint8_t** table,
                                                            unsigned* control, int n_control, unsigned* sync,
                                                            int n_sync) {
    const int i = threadIdx.x;
    if (i < n) table[i] = t.p[i];
    if (i < n_control) control[i] = 0u;
    for (int k = i; k < n_sync; k += blockDim.x) sync[k] = 0u;
}

std::mutex g_mutex;
void* g_scratch[kMaxDevices];

// This device's copy of the array (looked up once per device).
moe_status_t scratch_address(uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "moe_layer_forward_noalloc: hipGetSymbolAddress(scratch)");
        g_scratch[dev] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch[dev]);
    return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_layer_forward_noalloc(moe_layer_t* layer, const uint16_t* d_x, int T, float* d_y, int32_t* d_ids,
                                       float* d_w, void* stream) {
    if (!layer) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: layer is NULL");
    if (T < 0) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: T < 0");
    if (T == 0) return MOE_OK;
    if (!d_x || !d_y) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: NULL x or y");
    if (layer->cache) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: the layer uses an expert cache");
    if (!layer->experts_set) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: no experts set");
    moe_status_t st0 = check_layer_status(layer, "moe_layer_forward_noalloc");
    if (st0 != MOE_OK) return st0;
    const moe_config_t& c = layer->cfg;
    if (c.n_experts > 256) return fail(MOE_EINVAL, "moe_layer_forward_noalloc: more than 256 experts");
    const WorkspaceLayout W = workspace_layout(&c, 1);
    if (W.total > kScratchBytes)
        return fail(MOE_EINVAL, "moe_layer_forward_noalloc: the layer needs %zu bytes of per-call state, the static "
                    "scratch holds %zu", W.total, kScratchBytes);
    uint8_t* base = nullptr;
    moe_status_t st = scratch_address(&base);
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    TableArg t;
    std::memset(&t, 0, sizeof t);
    for (int e = 0; e < c.n_experts; ++e) t.p[e] = layer->host_table[e];
    hipLaunchKernelGGL(noalloc_setup_kernel, dim3(1), dim3(256), 0, s, t, c.n_experts,
                       reinterpret_cast<const uint8_t**>(base + W.table), reinterpret_cast<unsigned*>(base + W.control),
                       (int)(W.control_bytes / sizeof(unsigned)), reinterpret_cast<unsigned*>(base + W.sync),
                       (int)(kSyncBytes / sizeof(unsigned)));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "moe_layer_forward_noalloc: setup launch");
    // routing outputs the caller does not want go to the array's one-token
    // slots, overwritten token after token
    int32_t* ids = d_ids ? d_ids : reinterpret_cast<int32_t*>(base + W.ids);
    float* w = d_w ? d_w : reinterpret_cast<float*>(base + W.w);
    // the setup launch cleared the control words: in-kernel counted launches
    // count from 0
    DecodeSeq seq;
    return decode_tokens(layer, base, W, d_x, T, d_y, ids, d_ids ? c.top_k : 0, w, d_w ? c.top_k : 0, &seq, s);
}

}  // extern "C"
