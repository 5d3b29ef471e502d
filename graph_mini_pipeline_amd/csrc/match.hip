// Match and Greedy Reorder (gfx950).
//
// FastGL: A GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large Scale,
// "The idea" and "What it costs": consecutive batches share nodes, so a batch's rows that the
// batch still on the GPU already holds are copied from there and only the remainder is read from
// the store (Match, against the immediately previous batch only); and a group of sampled batches
// is put in nearest-overlap-first order from its full pairwise overlap matrix (Greedy Reorder).
//
// Both sets are node lists V_K, strictly ascending, so membership is a binary search and an
// intersection a count of hits.  Match: one lane per row of the new batch searches its id in the
// previous list (the previous list's position p is the row of the previous X that holds it);
// the gather kernels then take the row from there.  Overlap: for each pair a < b, one lane per
// element of L_a searches it in L_b; a workgroup adds its hits with one atomic.
#include "common.hpp"

namespace gnnmb {

// Position of v in the strictly ascending list l[0 .. n), or -1.
__device__ __forceinline__ int64_t find_sorted(const int32_t *l, int64_t n, int32_t v) {
    int64_t lo = 0, hi = n;   // l[lo - 1] < v <= l[hi] (virtually)
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (l[mid] < v) lo = mid + 1;
        else hi = mid;
    }
    return lo < n && l[lo] == v ? lo : -1;
}

__global__ __launch_bounds__(256) void k_match(MatchArgs a) {
    const int64_t n = load_count(a.d_n, a.n_cap);
    const int64_t pn = load_count(a.d_prev_n, a.prev_cap);
    uint32_t hits = 0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t p = find_sorted(a.prev_ids, pn, a.ids[i]);
        a.match[i] = static_cast<int32_t>(p);
        hits += p >= 0;
    }
    if (a.d_matched) {
        hits = wave_sum(hits);
        if (lane_id() == 0 && hits)
            atomicAdd(reinterpret_cast<unsigned long long *>(a.d_matched),
                      static_cast<unsigned long long>(hits));
    }
}

hipError_t launch_match(const MatchArgs &a, hipStream_t s) {
    if (a.n_cap <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_match, dim3(grid_for(a.n_cap, 256, 4096)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// overlap[a B + b] = 0 for a != b, |L_a| on the diagonal.
__global__ __launch_bounds__(256) void k_overlap_init(OverlapArgs a) {
    const int t = static_cast<int>(threadIdx.x);
    if (t < a.B * a.B) {
        const int r = t / a.B, c = t - r * a.B;
        a.out[t] = r == c ? static_cast<unsigned long long>(load_count(a.d_n[r], a.cap[r])) : 0ull;
    }
}

// Workgroup (x, y): chunk x of list pa[y], each element searched in list pb[y].
__global__ __launch_bounds__(256) void k_overlap(OverlapArgs a) {
    __shared__ uint32_t s_sum[4];
    const int y = static_cast<int>(blockIdx.y);
    const int la = a.pa[y], lb = a.pb[y];
    const int64_t na = load_count(a.d_n[la], a.cap[la]);
    const int64_t nb = load_count(a.d_n[lb], a.cap[lb]);
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kOverlapChunk;
    if (i0 >= na) return;   // uniform: the whole workgroup leaves
    uint32_t hits = 0;
    const int64_t i1 = i0 + kOverlapChunk < na ? i0 + kOverlapChunk : na;
    for (int64_t i = i0 + threadIdx.x; i < i1; i += blockDim.x)
        hits += find_sorted(a.ids[lb], nb, a.ids[la][i]) >= 0;
    hits = wave_sum(hits);
    if (lane_id() == 0) s_sum[threadIdx.x >> 6] = hits;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t t = s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
        if (t) atomicAdd(&a.out[la * a.B + lb], static_cast<unsigned long long>(t));
    }
}

// overlap[b B + a] = overlap[a B + b] for a < b.
__global__ __launch_bounds__(256) void k_overlap_mirror(OverlapArgs a) {
    const int t = static_cast<int>(threadIdx.x);
    if (t < a.B * a.B) {
        const int r = t / a.B, c = t - r * a.B;
        if (r > c) a.out[t] = a.out[c * a.B + r];
    }
}

hipError_t launch_overlap(const OverlapArgs &a, hipStream_t s) {
    static_assert(kMaxGroup * kMaxGroup <= 256, "one workgroup covers the matrix");
    hipLaunchKernelGGL(k_overlap_init, dim3(1), dim3(256), 0, s, a);
    if (a.npairs > 0) {
        int64_t cmax = 1;
        for (int l = 0; l < a.B; ++l) {
            const int64_t c = (a.cap[l] + kOverlapChunk - 1) / kOverlapChunk;
            cmax = c > cmax ? c : cmax;
        }
        if (cmax > 0x7FFFFFFFLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_overlap, dim3(static_cast<unsigned>(cmax), static_cast<unsigned>(a.npairs)),
                           dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(k_overlap_mirror, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
