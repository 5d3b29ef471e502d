// Sort-unique relabel over the id universe (gfx950).
//
// Defines V_l = ascending unique of V_{l-1} and the sampled ids (GARDEN: Efficient GPU-Accelerated
// Billion-Scale GNN Training via Caching-Sampling-Batching Co-Design, Sec. II.B / Fig. 1: the
// destinations of a layer are part of its sources) and the local ids of both lists.  FastGL: A
// GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large Scale (Fused-Map)
// builds the map with atomic hash inserts, whose first-come local ids vary from run to run; here
// the order is ascending global id, so the result is a pure function of the input.
//
// Method: a counting sort with one bucket per id.  A bitmap of id_bound bits marks every id
// (atomicOr; the final bitmap does not depend on the order of the ors), a two-level scan of the
// per-word popcounts gives each word the number of set bits before it, set bits are written out in
// order (this is the sorted unique list), and the rank of id v is
//   prefix[v >> 5] + popcount(word[v >> 5] & ((1 << (v & 31)) - 1)).
// Work is O(id_bound / 32) words plus O(list length); every output position comes from a scan.
#include "common.hpp"

namespace gnnmb {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *p, int64_t n, uint32_t value) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = value;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *p, int64_t n, int32_t value) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = value;
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t value, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 256 * 4, 2048)), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_i32, dim3(grid_for(n, 256 * 4, 2048)), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

// Marks both lists.  With check_dup_keep, a keep id whose bit was already set by another keep id
// is a duplicate (the keep list is marked by its own launch before the add list).
__global__ __launch_bounds__(256) void k_mark(const int32_t *ids, const int64_t *d_n, int64_t cap,
                                             uint32_t *bitmap, int64_t id_bound, int32_t *status,
                                             int32_t check_dup) {
    const int64_t n = load_count(d_n, cap);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int32_t v = ids[i];
        if (v < 0 || v >= id_bound) {
            set_status(status, GNN_ERR_OUT_OF_RANGE);
            continue;
        }
        const uint32_t bit = 1u << (v & 31);
        const uint32_t old = atomicOr(&bitmap[v >> 5], bit);
        if (check_dup && (old & bit)) set_status(status, GNN_ERR_INVALID_ARG);
    }
}

// Per-workgroup popcount of kBitmapTile consecutive words.
__global__ __launch_bounds__(kBitmapThreads) void k_popc_tiles(RelabelArgs a) {
    __shared__ uint32_t red[kBitmapThreads / 64];
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kBitmapTile +
                       static_cast<int64_t>(threadIdx.x) * kBitmapWordsPerThread;
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < kBitmapWordsPerThread; ++q)
        if (w0 + q < a.W) c += __popc(a.bitmap[w0 + q]);
    c = wave_sum(c);
    if (lane_id() == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int i = 0; i < kBitmapThreads / 64; ++i) s += red[i];
        a.bsum[blockIdx.x] = s;
    }
}

// One workgroup: exclusive scan of the tile popcounts in place; |uniq| to *d_uniq.
__global__ __launch_bounds__(1024) void k_popc_scan(RelabelArgs a) {
    __shared__ uint32_t smem[16];
    const int nb = a.nbw;
    const int per = (nb + 1023) / 1024;
    const int b0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int t = 0; t < per; ++t)
        if (b0 + t < nb) local += a.bsum[b0 + t];
    uint32_t total;
    uint32_t run = block_exclusive_scan<uint32_t, 1024>(local, &total, smem);
    for (int t = 0; t < per; ++t) {
        if (b0 + t < nb) {
            const uint32_t x = a.bsum[b0 + t];
            a.bsum[b0 + t] = run;
            run += x;
        }
    }
    if (threadIdx.x == 0) {
        *a.d_uniq = total;
        if (static_cast<int64_t>(total) > a.uniq_cap) set_status(a.status, GNN_ERR_CAPACITY);
    }
}

// Word prefixes and the sorted unique ids.
__global__ __launch_bounds__(kBitmapThreads) void k_emit(RelabelArgs a) {
    __shared__ uint32_t smem[kBitmapThreads / 64];
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kBitmapTile +
                       static_cast<int64_t>(threadIdx.x) * kBitmapWordsPerThread;
    uint32_t words[kBitmapWordsPerThread];
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < kBitmapWordsPerThread; ++q) {
        words[q] = w0 + q < a.W ? a.bitmap[w0 + q] : 0u;
        c += __popc(words[q]);
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<uint32_t, kBitmapThreads>(c, &total, smem);
    run += a.bsum[blockIdx.x];
#pragma unroll
    for (int q = 0; q < kBitmapWordsPerThread; ++q) {
        const int64_t w = w0 + q;
        if (w >= a.W) break;
        a.wprefix[w] = run;
        uint32_t bits = words[q];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            if (static_cast<int64_t>(run) < a.uniq_cap)
                a.uniq[run] = static_cast<int32_t>(w * 32 + b);
            ++run;
        }
    }
}

// Ranks of both lists (keep first, then add) in the unique list.
__global__ __launch_bounds__(256) void k_rank(RelabelArgs a) {
    const int64_t nk = load_count(a.d_keep, a.keep_cap);
    const int64_t na = load_count(a.d_add, a.add_cap);
    const int64_t total = a.keep_cap + a.add_cap;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const bool is_keep = t < a.keep_cap;
        const int64_t i = is_keep ? t : t - a.keep_cap;
        if (i >= (is_keep ? nk : na)) continue;
        const int32_t v = is_keep ? a.keep[i] : a.add[i];
        int32_t r = -1;
        if (v >= 0 && v < a.id_bound) {
            const uint32_t word = a.bitmap[v >> 5];
            r = static_cast<int32_t>(a.wprefix[v >> 5] + __popc(word & ((1u << (v & 31)) - 1u)));
        }
        if (is_keep) a.keep_lid[i] = r;
        else a.add_lid[i] = r;
    }
}

hipError_t launch_relabel(const RelabelArgs &a, hipStream_t s) {
    hipError_t e = launch_fill_u32(a.bitmap, a.W, 0u, s);
    if (e != hipSuccess) return e;
    if (a.keep_cap > 0)
        hipLaunchKernelGGL(k_mark, dim3(grid_for(a.keep_cap, 256, 4096)), dim3(256), 0, s, a.keep,
                           a.d_keep, a.keep_cap, a.bitmap, a.id_bound, a.status,
                           a.check_dup_keep);
    if (a.add_cap > 0)
        hipLaunchKernelGGL(k_mark, dim3(grid_for(a.add_cap, 256, 4096)), dim3(256), 0, s, a.add,
                           a.d_add, a.add_cap, a.bitmap, a.id_bound, a.status, 0);
    hipLaunchKernelGGL(k_popc_tiles, dim3(a.nbw), dim3(kBitmapThreads), 0, s, a);
    hipLaunchKernelGGL(k_popc_scan, dim3(1), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(k_emit, dim3(a.nbw), dim3(kBitmapThreads), 0, s, a);
    if (a.keep_cap + a.add_cap > 0)
        hipLaunchKernelGGL(k_rank, dim3(grid_for(a.keep_cap + a.add_cap, 256, 4096)), dim3(256),
                           0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
