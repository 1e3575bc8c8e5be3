// Read-only HBM streaming probe: the device's read ceiling that the layer's
// streaming kernels are measured against (the analogue of the disk read
// benchmark the colibri repository ships, fr.news.hada.io topic 31297,
// "Structure du depot et licence").  The buffer is cut into tiles of 32 KiB
// (256 threads x 8 chunks of 16 bytes); a workgroup takes tiles b, b + grid,
// ...  and each thread issues all 8 non-temporal loads of a tile before it
// uses any (a wave load covers 1 KiB of contiguous bytes, as in the decode
// kernels), folding them into one word so that no load is dead; one word per
// workgroup is written to the sink.  A grid of one workgroup per tile reads
// the buffer in one pass.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) hbm_read_kernel(const u32x4* __restrict__ src, size_t n16, unsigned* sink) {
    constexpr int U = 8;  // chunks in flight per thread
    const size_t n_tiles = (n16 + 256 * U - 1) / (256 * U);
    unsigned acc = 0u;
    for (size_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const size_t base = t * 256 * U + threadIdx.x;
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const size_t i = base + (size_t)k * 256;
            v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
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
