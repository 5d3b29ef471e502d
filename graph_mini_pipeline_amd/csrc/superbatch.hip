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
// found by its rank in the union bitmap and only the ids are copied; the compact relabel follows.)
// The sampler sets the bits of its sampled ids in the node-id bitmap that already holds U_l, whose
// set bits are then U_{l+1} = U_l + sampled ids, the union of the G node sets V_l, so every id of
// every sub-batch's block has a position in U_{l+1}: its rank in that bitmap.  Each sub-batch
// then takes, for destination i at union position r = upos[i], the union row [u_indptr[r],
// u_indptr[r+1]): an exclusive scan of the row lengths within the sub-batch gives its block
// indptr, the row's ids are copied with their U_{l+1} positions, and those positions are marked
// in the sub-batch's own relabel bitmap (|U_{l+1}| bits instead of one over every node id), whose
// result is exactly that of a separate run.
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

// Position in U_{l+1} of node id v (compact relabel): its rank in U_{l+1}'s node-id bitmap, or -1
// for an id outside the bitmap or not in it (only after an error already reported).
__device__ __forceinline__ int32_t next_rank(const DistArgs &a, int32_t v) {
    if (v < 0 || v >= a.id_bound) return -1;
    const uint32_t w = a.bm1[v >> 5];          // both loads issued together
    const uint32_t pre = a.wprefix1[v >> 5];
    const uint32_t bit = 1u << (v & 31);
    return (w & bit) ? static_cast<int32_t>(pre + __popc(w & (bit - 1u))) : -1;
}

// Position p of sub-batch g's relabel (compact relabel), marked as k_mark marks it: a byte when the
// byte maps exist, else the bitmap bit; with the duplicate check, the bit with the returned word.
__device__ __forceinline__ void mark_sub(const DistArgs &a, int g, int32_t p, bool dup) {
    const uint32_t bit = 1u << (p & 31);
    uint32_t *word = a.mark_words + static_cast<int64_t>(g) * a.mark_stride + (p >> 5);
    if (a.mark_bytes) a.mark_bytes[static_cast<int64_t>(g) * 32 * a.mark_stride + p] = 1;
    if (dup) {
        const uint32_t old = atomicOr(word, bit);
        if (old & bit) set_status(a.status, GNN_ERR_INVALID_ARG);   // a seed given twice
    } else if (!a.mark_bytes) {
        atomicOr(word, bit);   // result unused: posted
    }
}

// Destination i of a sub-batch: its union row [lo, lo + c) and (compact relabel) its position in
// U_{l+1} (-1 and an empty row for a destination without a union position: an invalid seed,
// already reported by the union marking).
__device__ __forceinline__ void union_row(const DistArgs &a, const DistSub &S, int64_t i,
                                          int64_t &lo, int32_t &c, int32_t &next_pos,
                                          int32_t &r, bool want_next = true) {
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
    if (a.Ul && want_next) next_pos = next_rank(a, a.Ul[r]);
}

// Tiles of kDistTile destinations: each wavefront takes a tile, one destination per lane (and,
// with the compact relabel, marks its position in U_{l+1} for the sub-batch relabel).  The grid
// is capped (kDistMaxGrid) and workgroups stride over the tiles, which are sized by the
// frontier bounds: tiles past a sub-batch's actual destinations are skipped, not dispatched.
__global__ __launch_bounds__(256) void k_dist_count(DistArgs a) {
    static_assert(kDistTile == 64, "one destination per lane of a wavefront");
    const int64_t n1 = a.mark_words ? load_count(a.d_U1, a.U1_cap) : 0;   // |U_{l+1}|
    const int wv = static_cast<int>(threadIdx.x >> 6);
    const int lane = lane_id();
    for (int t = blockIdx.x * 4 + wv; t < a.ntiles; t += gridDim.x * 4) {
        const int sg = find_sub(a, t);
        const DistSub &S = a.sub[sg];
        const int64_t F = load_count(S.d_F, S.F_cap);
        const int64_t i0 = static_cast<int64_t>(t - S.tile0) * kDistTile;
        if (i0 >= F) continue;   // past the destinations: k_dist_scatter reads no sum for it
        const int64_t i = i0 + lane;
        int64_t lo;
        int32_t c = 0, np, r;
        if (i < F) {
            union_row(a, S, i, lo, c, np, r);
            if (S.f_pos) S.f_pos[i] = np;
            if (a.mark_words && np >= 0 && np < n1) mark_sub(a, sg, np, a.mark_dup != 0);
            if (a.inv && r >= 0) {
                a.inv[static_cast<int64_t>(r) * a.G + sg] = static_cast<int32_t>(i + 1);
                atomicOr(&a.inv_mask[r], 1u << sg);
            }
        }
        const uint32_t sum = wave_sum(static_cast<uint32_t>(c));
        if (lane == 0) a.bsum[t] = sum;
    }
}

__global__ __launch_bounds__(256) void k_dist_scatter(DistArgs a) {
    __shared__ uint32_t s_red[2][4];
    __shared__ uint32_t s_off, s_tot;
    __shared__ uint32_t s_item_off[kDistTile + 1];
    __shared__ int64_t s_item_lo[kDistTile];
    const int64_t n1 = a.mark_words ? load_count(a.d_U1, a.U1_cap) : 0;   // |U_{l+1}|
    for (int t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
        const int sg = find_sub(a, t);
        const DistSub &S = a.sub[sg];
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
            if (i < F) union_row(a, S, i, lo, c, np, r, false);
            const uint32_t inc = wave_inclusive_scan(static_cast<uint32_t>(c));
            const uint32_t o = inc - static_cast<uint32_t>(c);
            s_item_off[threadIdx.x] = o;
            s_item_lo[threadIdx.x] = lo;
            if (threadIdx.x == kDistTile - 1) s_tot = inc;
            if (i < F) S.blk_indptr[i] = static_cast<int32_t>(s_off + o);
        }
        __syncthreads();
        // The tile's sampled ids, U rounds of one per thread at a time so that each round's
        // dependent loads (the id, then its bitmap word and prefix) are in flight together.
        const uint32_t tot = s_tot;
        constexpr int U = 4;
        for (uint32_t p0 = threadIdx.x; p0 < tot; p0 += U * blockDim.x) {
            int64_t dst[U], src[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t p = p0 + u * blockDim.x;
                int lo_i = 0, hi_i = kDistTile;  // last destination whose offset is <= p
                while (hi_i - lo_i > 1) {
                    const int mid = (lo_i + hi_i) >> 1;
                    if (s_item_off[mid] <= p) lo_i = mid;
                    else hi_i = mid;
                }
                dst[u] = static_cast<int64_t>(s_off) + p;
                src[u] = s_item_lo[lo_i] + (p - s_item_off[lo_i]);
                ok[u] = p < tot && dst[u] < S.E_cap;
            }
            int32_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = ok[u] ? a.u_gid[src[u]] : -1;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) S.blk_gid[dst[u]] = v[u];
            if (S.e_pos) {
                int32_t q[U];
#pragma unroll
                for (int u = 0; u < U; ++u) q[u] = ok[u] ? next_rank(a, v[u]) : -1;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!ok[u]) continue;
                    S.e_pos[dst[u]] = q[u];
                    if (a.mark_words && q[u] >= 0 && q[u] < n1) mark_sub(a, sg, q[u], false);
                }
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
