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
    const uint2 e = a.rdir0[v >> 5];
    return static_cast<int32_t>(e.x + __popc(e.y & ((1u << (v & 31)) - 1u)));
}

// Position in U_{l+1} of node id v (compact relabel): its rank in U_{l+1}'s node-id bitmap, or -1
// for an id outside the bitmap or not in it (only after an error already reported).
__device__ __forceinline__ int32_t next_rank(const DistArgs &a, int32_t v) {
    if (v < 0 || v >= a.id_bound) return -1;
    return rdir_rank(a.rdir1, v);
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

// One pass over the destinations, in tiles of kDistTile (one per thread): each tile finds its
// destinations' union rows (and, with the compact relabel, marks their positions in U_{l+1}), sums
// their lengths, takes the sum of the earlier tiles of its sub-batch by look-back, writes its
// part of the block indptr and copies its rows' ids.  Workgroup b serves the sub-batch whose
// tiles hold b; those past the sub-batch's actual destinations leave before taking a ticket (a
// sub-batch without destinations keeps one tile, which writes the empty block), and the live ones
// take tickets 0 .. live - 1 from the sub-batch's counter, ticket t being tile t, so that a tile
// only waits for tiles already running.  The last live tile writes the block's edge count.
__global__ __launch_bounds__(kDistTile) void k_dist(DistArgs a) {
    constexpr int NW = kDistTile / 64;
    __shared__ uint32_t s_wave[NW];
    __shared__ uint32_t s_ticket, s_base;
    __shared__ uint32_t s_item_off[kDistTile];
    __shared__ int64_t s_item_lo[kDistTile];
    const int b = static_cast<int>(blockIdx.x);
    const int sg = find_sub(a, b);
    const DistSub &S = a.sub[sg];
    const int64_t F = load_count(S.d_F, S.F_cap);
    const int64_t live = (F + kDistTile - 1) / kDistTile;
    if (b - S.tile0 >= (live > 0 ? live : 1)) return;
    const int64_t n1 = a.mark_words ? load_count(a.d_U1, a.U1_cap) : 0;   // |U_{l+1}|
    const int64_t lt = lb_ticket(a.lb.ticket + sg, &s_ticket);
    const int lane = lane_id();
    const int wv = static_cast<int>(threadIdx.x >> 6);
    const int64_t i = lt * kDistTile + threadIdx.x;
    int64_t lo = 0;
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
    // the tile's row lengths: offsets within the tile, then the tile's base by look-back
    const uint32_t inc = wave_inclusive_scan(static_cast<uint32_t>(c));
    if (lane == 63) s_wave[wv] = inc;
    __syncthreads();
    uint32_t wbefore = 0, agg = 0;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
        const uint32_t v = s_wave[q];
        if (q < wv) wbefore += v;
        agg += v;
    }
    if (wv == 0) {
        uint64_t *chain = a.lb.words + S.tile0;
        uint32_t before = 0;
        if (lt == 0) {
            if (lane == 0) lb_publish(&chain[0], kLbInclusive, agg);
        } else {
            if (lane == 0) lb_publish(&chain[lt], kLbAggregate, agg);
            before = lb_exclusive(chain, lt);
            if (lane == 0) lb_publish(&chain[lt], kLbInclusive, before + agg);
        }
        if (lane == 0) {
            s_base = before;
            if (lt == (live > 0 ? live - 1 : 0)) {
                const uint32_t tot = before + agg;
                S.blk_indptr[F] = static_cast<int32_t>(tot);
                *S.d_E = tot;
                if (static_cast<int64_t>(tot) > S.E_cap) set_status(a.status, GNN_ERR_CAPACITY);
            }
        }
    }
    const uint32_t o = wbefore + inc - static_cast<uint32_t>(c);
    s_item_off[threadIdx.x] = o;
    s_item_lo[threadIdx.x] = lo;
    __syncthreads();
    const uint32_t base = s_base;
    if (i < F) S.blk_indptr[i] = static_cast<int32_t>(base + o);
    // The tile's sampled ids, U rounds of one per thread at a time so that each round's dependent
    // loads (the id, then its bitmap word and prefix) are in flight together.
    constexpr int U = 4;
    for (uint32_t p0 = threadIdx.x; p0 < agg; p0 += U * kDistTile) {
        int64_t dst[U], src[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p = p0 + u * kDistTile;
            int lo_i = 0, hi_i = kDistTile;  // last destination whose offset is <= p
            while (hi_i - lo_i > 1) {
                const int mid = (lo_i + hi_i) >> 1;
                if (s_item_off[mid] <= p) lo_i = mid;
                else hi_i = mid;
            }
            dst[u] = static_cast<int64_t>(base) + p;
            src[u] = s_item_lo[lo_i] + (p - s_item_off[lo_i]);
            ok[u] = p < agg && dst[u] < S.E_cap;
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
}

// The first union level U_0 of a compact super-batch, when the sub-batches' seeds fit its bound
// as they are: their concatenation, in sub-batch order, instead of their sorted union.  A seed
// held by several sub-batches appears once per sub-batch, and each copy's row is sampled with
// the same result (the sample depends only on the node and the hop seed), so every sub-batch
// gets exactly the rows a sorted union would give it; from U_1 on, the levels are the ranks of
// the accumulated node-id bitmap as before, into which each seed's bit is set here.  Ids out of
// range are left unmarked (the classification reports them).
__global__ __launch_bounds__(256) void k_seed_concat(SeedConcatArgs a) {
    const int64_t total = a.off[a.G];
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t0 == 0) *a.d_U0 = total;
    for (int64_t t = t0; t < total; t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        int g = 0;
        while (g + 1 < a.G && a.off[g + 1] <= t) ++g;
        const int64_t i = t - a.off[g];
        const int32_t v = a.seeds[g][i];
        a.U0[t] = v;
        a.upos[g * a.P + i] = static_cast<int32_t>(t);
        if (v >= 0 && v < a.num_nodes) atomicOr(&a.bitmap[v >> 5], 1u << (v & 31));
    }
}

hipError_t launch_seed_concat(const SeedConcatArgs &a, hipStream_t s) {
    const int64_t total = a.off[a.G];
    hipLaunchKernelGGL(k_seed_concat, dim3(grid_for(total, 256, 1024)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dist(const DistArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_dist, dim3(a.ntiles), dim3(kDistTile), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
