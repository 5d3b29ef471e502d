// Plain streaming copy used to calibrate memory-traffic counters (see gnnmb_probe.h).
#include "common.hpp"
#include "gnnmb_probe.h"

namespace gnnmb {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy_probe(const u32x4 *src, u32x4 *dst, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

// Hash throughput ceiling: every lane evaluates `per_lane` sampling keys mix64(z), z stepping by
// the key-stream increment exactly as the sampler's candidate loop does (two keys per step), and
// counts the keys <= tau (the count is written so that no key is optimised away).
__global__ __launch_bounds__(256) void k_hash_probe(uint64_t seed, uint64_t tau, int64_t per_lane,
                                                    unsigned long long *out) {
    const uint64_t t = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const uint64_t step = kGamma * 64u;
    uint64_t z = mix64(seed ^ t) + kGamma;
    uint32_t cnt = 0;
    for (int64_t i = 0; i < per_lane; i += 2) {
        const uint64_t k0 = mix64(z);
        const uint64_t k1 = mix64(z + step);
        z += 2 * step;
        cnt += (k0 <= tau) + (k1 <= tau);
    }
    if (cnt) atomicAdd(out, static_cast<unsigned long long>(cnt));
}

}  // namespace gnnmb

extern "C" gnn_status gnn_hash_probe(uint64_t seed, uint64_t tau, int64_t lanes, int64_t per_lane,
                                     unsigned long long *d_count, gnn_stream stream) {
    using namespace gnnmb;
    if (!d_count || lanes < 256 || lanes % 256 != 0 || lanes / 256 > 0x7FFFFFFF || per_lane < 2 ||
        per_lane % 2 != 0)
        return GNN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_hash_probe, dim3(static_cast<unsigned>(lanes / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), seed, tau, per_lane, d_count);
    return hipGetLastError() == hipSuccess ? GNN_OK : GNN_ERR_HIP;
}

extern "C" gnn_status gnn_copy_probe(const void *src, void *dst, size_t bytes, gnn_stream stream) {
    using namespace gnnmb;
    if (!src || !dst || bytes == 0 || bytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
        return GNN_ERR_INVALID_ARG;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    hipLaunchKernelGGL(k_copy_probe, dim3(grid_for(n, 256 * 8, 8192)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? GNN_OK : GNN_ERR_HIP;
}

extern "C" gnn_status gnn_copy_probe_host(const void *host_src, void *dst, size_t bytes,
                                          gnn_stream stream) {
    if (!host_src) return GNN_ERR_INVALID_ARG;
    void *mapped = nullptr;
    if (hipHostGetDevicePointer(&mapped, const_cast<void *>(host_src), 0) != hipSuccess || !mapped)
        return GNN_ERR_HIP;
    return gnn_copy_probe(mapped, dst, bytes, stream);
}
