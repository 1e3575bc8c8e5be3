// Read-only HBM streaming probe: the device's read ceiling that the layer's
// streaming kernels are measured against (the analogue of the disk read
// benchmark the colibri repository ships, fr.news.hada.io topic 31297,
// "Structure du depot et licence").  Every lane reads 16-byte chunks with
// non-temporal loads in a grid-stride loop, four chunks in flight, and folds
// them into one word so that no load is dead; one word per workgroup is
// written to the sink.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) hbm_read_kernel(const u32x4* __restrict__ src, size_t n16, unsigned* sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned acc = 0u;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ unsigned part[256];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned r = 0u;
        for (int t = 0; t < (int)blockDim.x; ++t) r ^= part[t];
        sink[blockIdx.x] = r;
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_hbm_read_probe(const void* d_buf, size_t bytes, unsigned* d_sink, int blocks, void* stream) {
    if (!d_buf || !d_sink) return fail(MOE_EINVAL, "moe_hbm_read_probe: NULL buffer or sink");
    if (bytes % 16 || reinterpret_cast<uintptr_t>(d_buf) % 16)
        return fail(MOE_EINVAL, "moe_hbm_read_probe: buffer and size must be multiples of 16 bytes");
    if (blocks < 1) return fail(MOE_EINVAL, "moe_hbm_read_probe: blocks must be >= 1");
    hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(d_buf), bytes / 16, d_sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "moe_hbm_read_probe launch");
    return MOE_OK;
}

}  // extern "C"
