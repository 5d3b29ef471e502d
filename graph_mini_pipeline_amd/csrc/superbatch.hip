// Super-batch distribution (gfx950).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. IV.D with Alg. 1: several mini-batches are stored contiguously with sub-batch
// bounds (BatchPtr), deduplicated across mini-batches and classified once, so that each node
// appears once in the super-batch view while each mini-batch keeps its own logical result.
//
// Here the G sub-batches of a super-batch share one batch seed, so the sample of node v at hop l
// is the same in every sub-batch whose frontier holds v.  The union U of the G frontiers is
// relabelled (bitmap B0), classified and sampled once; then every sub-batch takes, for each of its
// destinations v, the row of v in the union block: c = u_indptr[r+1] - u_indptr[r] with
// r = rank of v in U, an exclusive scan of c within the sub-batch gives its block indptr, and the
// row's ids are copied.  Each sub-batch's result is therefore exactly that of a separate run.
#include "common.hpp"

namespace gnnmb {

__device__ __forceinline__ int find_sub(const DistArgs &a, int t) {
    int g = 0;
    while (g + 1 < a.G && a.sub[g + 1].tile0 <= t) ++g;
    return g;
}

__device__ __forceinline__ int32_t union_rank(const DistArgs &a, int32_t v) {
    const uint32_t w = a.bm0[v >> 5];
    return static_cast<int32_t>(a.wprefix0[v >> 5] + __popc(w & ((1u << (v & 31)) - 1u)));
}

// Destination i of sub-batch g: its union row [lo, hi) (empty if the id is invalid).
__device__ __forceinline__ void union_row(const DistArgs &a, const DistSub &S, int64_t i,
                                          int64_t &lo, int32_t &c) {
    lo = 0;
    c = 0;
    const int32_t v = S.front[i];
    if (v < 0 || v >= a.id_bound) return;  // reported by the union marking
    const int64_t nU = load_count(a.d_U, a.U_cap);
    const int32_t r = union_rank(a, v);
    if (r < 0 || r >= nU) {
        set_status(a.status, GNN_ERR_INTERNAL);
        return;
    }
    int64_t l0 = a.u_indptr[r], l1 = a.u_indptr[r + 1];
    l0 = l0 < 0 ? 0 : (l0 > a.uE_cap ? a.uE_cap : l0);
    l1 = l1 < l0 ? l0 : (l1 > a.uE_cap ? a.uE_cap : l1);
    lo = l0;
    c = static_cast<int32_t>(l1 - l0);
}

__global__ __launch_bounds__(kClassifyThreads) void k_dist_count(DistArgs a) {
    __shared__ uint32_t red[kClassifyThreads / 64];
    const int t = blockIdx.x;
    const int g = find_sub(a, t);
    const DistSub &S = a.sub[g];
    const int64_t F = load_count(S.d_F, S.F_cap);
    const int64_t base = static_cast<int64_t>(t - S.tile0) * kClassifyTile +
                         static_cast<int64_t>(threadIdx.x) * kClassifyItems;
    uint32_t csum = 0;
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        if (base + q < F) {
            int64_t lo;
            int32_t c;
            union_row(a, S, base + q, lo, c);
            csum += static_cast<uint32_t>(c);
        }
    }
    csum = wave_sum(csum);
    if (lane_id() == 0) red[threadIdx.x >> 6] = csum;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int i = 0; i < kClassifyThreads / 64; ++i) s += red[i];
        a.bsum[t] = s;
    }
}

__global__ __launch_bounds__(kClassifyThreads) void k_dist_scatter(DistArgs a) {
    __shared__ uint32_t sm[kClassifyThreads / 64];
    __shared__ uint32_t s_red[2][kClassifyThreads / 64];
    __shared__ uint32_t s_off;
    const int t = blockIdx.x;
    const int g = find_sub(a, t);
    const DistSub &S = a.sub[g];
    const int lt = t - S.tile0;
    const int64_t F = load_count(S.d_F, S.F_cap);
    uint32_t before = 0, all = 0;
    for (int b = threadIdx.x; b < S.ntile; b += blockDim.x) {
        const uint32_t x = a.bsum[S.tile0 + b];
        all += x;
        if (b < lt) before += x;
    }
    before = wave_sum(before);
    all = wave_sum(all);
    if (lane_id() == 0) {
        s_red[0][threadIdx.x >> 6] = before;
        s_red[1][threadIdx.x >> 6] = all;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b0 = 0, tot = 0;
        for (int i = 0; i < kClassifyThreads / 64; ++i) {
            b0 += s_red[0][i];
            tot += s_red[1][i];
        }
        s_off = b0;
        if (lt == 0) {
            S.blk_indptr[F] = static_cast<int32_t>(tot);
            *S.d_E = tot;
            if (static_cast<int64_t>(tot) > S.E_cap) set_status(a.status, GNN_ERR_CAPACITY);
        }
    }
    __syncthreads();
    const int64_t base = static_cast<int64_t>(lt) * kClassifyTile +
                         static_cast<int64_t>(threadIdx.x) * kClassifyItems;
    int64_t lo[kClassifyItems];
    int32_t c[kClassifyItems];
    uint32_t csum = 0;
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        lo[q] = 0;
        c[q] = 0;
        if (base + q < F) union_row(a, S, base + q, lo[q], c[q]);
        csum += static_cast<uint32_t>(c[q]);
    }
    uint32_t tot;
    uint32_t o = block_exclusive_scan<uint32_t, kClassifyThreads>(csum, &tot, sm) + s_off;
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        const int64_t i = base + q;
        if (i >= F) break;
        S.blk_indptr[i] = static_cast<int32_t>(o);
        for (int32_t j = 0; j < c[q]; ++j)
            if (static_cast<int64_t>(o) + j < S.E_cap) S.blk_gid[o + j] = a.u_gid[lo[q] + j];
        o += static_cast<uint32_t>(c[q]);
    }
}

hipError_t launch_dist(const DistArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_dist_count, dim3(a.ntiles), dim3(kClassifyThreads), 0, s, a);
    hipLaunchKernelGGL(k_dist_scatter, dim3(a.ntiles), dim3(kClassifyThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
