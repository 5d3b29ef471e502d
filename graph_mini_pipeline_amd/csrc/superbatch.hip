// Super-batch distribution (gfx950).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. IV.D with Alg. 1: several mini-batches are stored contiguously with sub-batch
// bounds (BatchPtr), deduplicated across mini-batches and classified once, so that each node
// appears once in the super-batch view while each mini-batch keeps its own logical result.
//
// Here the G sub-batches of a super-batch share one batch seed, so the sample of node v at hop l
// is the same in every sub-batch whose frontier holds v.  The union U_l of the G frontiers is
// classified and sampled once.  (With full-range sub-batch bitmaps, a destination's union row is
// found by its rank in the union bitmap and only the ids are copied; the compact relabel follows.)  Its sampled ids and U_l itself are relabelled into
// U_{l+1} = U_l + sampled ids, which is the union of the G node sets V_l, so every id of every
// sub-batch's block has a position in U_{l+1}.  Each sub-batch then takes, for destination i at
// union position r = upos[i], the union row [u_indptr[r], u_indptr[r+1]): an exclusive scan of
// the row lengths within the sub-batch gives its block indptr, and the row's ids and their
// U_{l+1} positions are copied.  The sub-batch's own relabel then runs on those positions
// (a bitmap of |U_{l+1}| bits instead of one over every node id), and its result is exactly that
// of a separate run.
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

// Destination i of a sub-batch: its union row [lo, lo + c) and (compact relabel) its position in
// U_{l+1} (-1 and an empty row for a destination without a union position: an invalid seed,
// already reported by the union marking).
__device__ __forceinline__ void union_row(const DistArgs &a, const DistSub &S, int64_t i,
                                          int64_t &lo, int32_t &c, int32_t &next_pos,
                                          int32_t &r) {
    lo = 0;
    c = 0;
    next_pos = -1;
    r = -1;
    if (S.upos) {
        r = S.upos[i];
    } else {
        const int32_t v = S.front[i];
        if (v < 0 || v >= a.id_bound) return;  // reported by the union marking
        r = union_rank(a, v);
    }
    if (r < 0) return;
    const int64_t nU = load_count(a.d_U, a.U_cap);
    if (r >= nU) {
        set_status(a.status, GNN_ERR_INTERNAL);
        r = -1;
        return;
    }
    int64_t l0 = a.u_indptr[r], l1 = a.u_indptr[r + 1];
    l0 = l0 < 0 ? 0 : (l0 > a.uE_cap ? a.uE_cap : l0);
    l1 = l1 < l0 ? l0 : (l1 > a.uE_cap ? a.uE_cap : l1);
    lo = l0;
    c = static_cast<int32_t>(l1 - l0);
    if (a.umap) next_pos = a.umap[r];
}

// Tiles of kDistTile destinations: wavefront 0 handles one destination per lane.  The whole grid
// first zeroes the live words of the sub-batch bitmaps that the sub-batch relabel marks next.
// The grid is capped (kDistMaxGrid) and workgroups stride over the tiles, which are sized by the
// frontier bounds: tiles past a sub-batch's actual destinations are skipped, not dispatched.
__global__ __launch_bounds__(256) void k_dist_count(DistArgs a) {
    if (a.clear_ptr) {
        const int64_t n1 = load_count(a.d_U1, a.U1_cap);
        const int64_t words = (n1 + 31) >> 5;
        const int64_t total = words * a.G;
        for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
             t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
            const int64_t g = t / words;
            a.clear_ptr[g * a.clear_stride + (t - g * words)] = 0u;
        }
        if (a.clear_bytes) {   // 8 words of bytes per bitmap word
            const int64_t bw = 8 * words;
            for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < bw * a.G;
                 t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
                const int64_t g = t / bw;
                a.clear_bytes[g * 8 * a.clear_stride + (t - g * bw)] = 0u;
            }
        }
    }
    if (threadIdx.x >= kDistTile) return;
    for (int t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
        const int sg = find_sub(a, t);
        const DistSub &S = a.sub[sg];
        const int64_t F = load_count(S.d_F, S.F_cap);
        const int64_t i0 = static_cast<int64_t>(t - S.tile0) * kDistTile;
        if (i0 >= F) continue;   // past the destinations: k_dist_scatter reads no sum for it
        const int64_t i = i0 + threadIdx.x;
        int64_t lo;
        int32_t c = 0, np, r;
        if (i < F) {
            union_row(a, S, i, lo, c, np, r);
            if (S.f_pos) S.f_pos[i] = np;
            if (a.inv && r >= 0) a.inv[static_cast<int64_t>(r) * a.G + sg] = static_cast<int32_t>(i + 1);
        }
        const uint32_t sum = wave_sum(static_cast<uint32_t>(c));
        if (threadIdx.x == 0) a.bsum[t] = sum;
    }
}

__global__ __launch_bounds__(256) void k_dist_scatter(DistArgs a) {
    __shared__ uint32_t s_red[2][4];
    __shared__ uint32_t s_off, s_tot;
    __shared__ uint32_t s_item_off[kDistTile + 1];
    __shared__ int64_t s_item_lo[kDistTile];
    for (int t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
        const DistSub &S = a.sub[find_sub(a, t)];
        const int lt = t - S.tile0;
        const int64_t F = load_count(S.d_F, S.F_cap);
        // tiles past the actual destinations have nothing to place (tile 0 still writes the totals)
        const int live = static_cast<int>((F + kDistTile - 1) / kDistTile);
        if (lt > 0 && lt >= live) continue;
        // the sums of the earlier tiles (tile 0: of all tiles, for the sub-batch's total)
        uint32_t before = 0, all = 0;
        const int upto = lt == 0 ? live : lt;
        for (int b = threadIdx.x; b < upto; b += blockDim.x) {
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
            const uint32_t b0 = s_red[0][0] + s_red[0][1] + s_red[0][2] + s_red[0][3];
            const uint32_t tot = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
            s_off = b0;
            if (lt == 0) {
                S.blk_indptr[F] = static_cast<int32_t>(tot);
                *S.d_E = tot;
                if (static_cast<int64_t>(tot) > S.E_cap) set_status(a.status, GNN_ERR_CAPACITY);
            }
        }
        __syncthreads();
        if (threadIdx.x < kDistTile) {
            const int64_t i = static_cast<int64_t>(lt) * kDistTile + threadIdx.x;
            int64_t lo = 0;
            int32_t c = 0, np, r;
            if (i < F) union_row(a, S, i, lo, c, np, r);
            const uint32_t inc = wave_inclusive_scan(static_cast<uint32_t>(c));
            const uint32_t o = inc - static_cast<uint32_t>(c);
            s_item_off[threadIdx.x] = o;
            s_item_lo[threadIdx.x] = lo;
            if (threadIdx.x == kDistTile - 1) s_tot = inc;
            if (i < F) S.blk_indptr[i] = static_cast<int32_t>(s_off + o);
        }
        __syncthreads();
        const uint32_t tot = s_tot;
        for (uint32_t p = threadIdx.x; p < tot; p += blockDim.x) {
            int lo_i = 0, hi_i = kDistTile;  // last destination whose offset is <= p
            while (hi_i - lo_i > 1) {
                const int mid = (lo_i + hi_i) >> 1;
                if (s_item_off[mid] <= p) lo_i = mid;
                else hi_i = mid;
            }
            const int64_t dst = static_cast<int64_t>(s_off) + p;
            const int64_t src = s_item_lo[lo_i] + (p - s_item_off[lo_i]);
            if (dst < S.E_cap) {
                S.blk_gid[dst] = a.u_gid[src];
                if (S.e_pos) S.e_pos[dst] = a.u_pos[src];
            }
        }
        __syncthreads();   // the shared arrays are rewritten by the next tile
    }
}

constexpr int kDistMaxGrid = 4096;

hipError_t launch_dist(const DistArgs &a, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(a.ntiles < kDistMaxGrid ? a.ntiles : kDistMaxGrid);
    hipLaunchKernelGGL(k_dist_count, dim3(grid), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_dist_scatter, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
