// Frontier degree classification and degree-grouped k-hop neighbour sampling (gfx950, wave64).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. IV.C: a "full node" (degree <= fanout) keeps its whole neighbour list; other
// nodes draw `fanout` neighbours; lanes are grouped so that the threads of a group run identical
// logic, and high-degree nodes take a separate path.  Sec. IV.D, Alg. 1: classification by a flag
// and an exclusive scan turns placement into index arithmetic, with no atomics.
//
// Here the draw is the bottom-k of per-edge SplitMix64 keys: node v at hop l keeps the k positions
// with the smallest (key, position), key(j) = mix64(s_{l,v} + G*(j+1)).  Keys depend only on
// (seed, hop, node, position), so no adjacency is read to choose; only the k chosen neighbour ids
// are read.  Selection is exact: a threshold tau is chosen so that the expected number of keys
// <= tau is a little above k; the keys <= tau (candidates) are compacted to LDS; if fewer than k or
// more than the LDS capacity survive, tau is bisected and the pass repeated.  Once
// k <= count <= capacity the k smallest candidates are exactly the k smallest keys of the row.
//
// Classes (per hop, per frontier node v of degree deg, fanout k), all in one launch:
//   FULL   deg <= k                one lane per node copies the row
//   GROUP  k < deg <= group_max   16 lanes per node (4 nodes per wavefront)
//   WAVE   group_max < deg <= wave_max   one wavefront per node
//   BLOCK  deg > wave_max          one 512-thread workgroup per node
// Each class walks its work-list with a static stride (no shared work counter); results do not
// depend on the order in which nodes are processed.
#include <math.h>

#include "common.hpp"

namespace gnnmb {

// ---- classification: count, scan, scatter ------------------------------------------------------

// Node v's neighbour ids: its row in the HBM adjacency cache when the cache holds it, else its
// CSR row (HBM, or pinned host memory read in place).
template <bool ADJ>
__device__ __forceinline__ const int32_t *adj_row(const HopArgs &a, int32_t v, int64_t start) {
    if (ADJ && a.adj_off != nullptr) {
        const int64_t o = a.adj_off[v];
        if (o >= 0) return a.adj_rows + o;
    }
    return a.indices + start;
}

// Entry v of a CSR indptr of IB-byte entries (the sampler is compiled for each width).
template <int IB>
__device__ __forceinline__ int64_t row_at(const void *indptr, int64_t v) {
    if constexpr (IB == 8) return static_cast<const int64_t *>(indptr)[v];
    else return static_cast<int64_t>(static_cast<const int32_t *>(indptr)[v]);
}

__device__ __forceinline__ int32_t node_class(int64_t deg, int k, int group_max, int wave_max) {
    if (deg <= k) return kFull;
    if (deg <= group_max && k * 4 <= kGroupCap) return kGroup;
    if (deg <= wave_max && k * 4 <= kWaveCap) return kWave;
    return kBlock;
}

// Classification categories: FULL, GROUP, the WAVE class split into kWaveBuckets degree buckets
// listed largest first (bucket b holds degrees in [2^(13-b), 2^(14-b)), the last also all smaller
// ones and the first all larger ones), BLOCK.  The WAVE list is ordered by bucket, so wavefronts
// that walk it with a snake stride take the largest rows first and balance their loads.
constexpr int kCatBlock = kCats - 1;
static_assert(kCols == 1 + kCats, "edges, then one column per category");
__device__ __forceinline__ int32_t node_cat(int32_t cls, int64_t deg) {
    if (cls == kFull) return 0;
    if (cls == kGroup) return 1;
    if (cls == kBlock) return kCatBlock;
    const int lg = 63 - __clzll(static_cast<unsigned long long>(deg));   // floor(log2 deg)
    int b = 13 - lg;
    b = b < 0 ? 0 : (b >= kWaveBuckets ? kWaveBuckets - 1 : b);
    return 2 + b;
}
// Nodes of a class (totals: edges, then the categories' sizes).
__device__ __forceinline__ int64_t class_total(const uint32_t *totals, int32_t cls) {
    if (cls == kFull) return totals[1];
    if (cls == kGroup) return totals[2];
    if (cls == kBlock) return totals[1 + kCatBlock];
    int64_t n = 0;
    for (int b = 0; b < kWaveBuckets; ++b) n += totals[3 + b];
    return n;
}

// Item `item` of the one-wavefront class, whose nodes sit in one work-list per degree bucket
// (largest degrees first): the bucket holding the item, then the item's place in it.
__device__ __forceinline__ int32_t wave_item(const HopArgs &a, int64_t item) {
    uint32_t off = static_cast<uint32_t>(item);   // list positions are below 2^31
    int b = 0;
#pragma unroll
    for (int q = 0; q < kWaveBuckets - 1; ++q) {
        const uint32_t c = a.totals[3 + q];
        const bool past = b == q && off >= c;
        off -= past ? c : 0u;
        b += past ? 1 : 0;
    }
    return a.lists[static_cast<int64_t>(2 + b) * a.F_cap + off];
}

// Count of category `cat` in counters packed as the classification packs them (categories 0..3
// in 16-bit fields of c0, 4..8 in 12-bit fields of c1).
__device__ __forceinline__ uint32_t cat_count(uint64_t c0, uint64_t c1, int cat) {
    return cat < 4 ? static_cast<uint32_t>((c0 >> (16 * cat)) & 0xFFFF)
                   : static_cast<uint32_t>((c1 >> (12 * (cat - 4))) & 0xFFF);
}

// One pass over the frontier, in tiles of kClassifyTile nodes taken by ticket: each node's c and
// category; the block indptr as an exclusive scan of c (the tile's offset by look-back over the
// earlier tiles; the last tile writes |E_l|); each node appended to its category's work-list
// (one atomic reservation per category per tile: the order inside a list does not matter, since
// every node's outputs are placed by its block indptr).  The grid also zeroes the optional clear
// region and, for a super-batch's last hop, the union positions table.
__global__ __launch_bounds__(kClassifyThreads) void k_classify(HopArgs a) {
    __shared__ uint32_t sm_c[kClassifyThreads / 64];
    __shared__ uint64_t sm_k0[kClassifyThreads / 64];
    __shared__ uint64_t sm_k1[kClassifyThreads / 64];
    __shared__ uint32_t s_ticket, s_prefix;
    __shared__ uint32_t s_base[kCats];
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < a.clear_n;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x)
        a.clear_ptr[t] = 0u;
    const int64_t F = load_count(a.d_F, a.F_cap);
    const int64_t last = F > 0 ? (F - 1) / kClassifyTile : 0;   // last tile holding nodes
    // The grid is sized by the frontier bound: workgroups beyond the live tiles leave before
    // taking a ticket (tickets of one counter are handed out one at a time).  The live ones take
    // tickets 0 .. last, and ticket t is tile t.
    if (static_cast<int64_t>(blockIdx.x) > last) return;
    const int64_t tile = lb_ticket(a.lb.ticket, &s_ticket);
    const int64_t base = tile * kClassifyTile + static_cast<int64_t>(threadIdx.x) * kClassifyItems;
    int32_t cq[kClassifyItems], catq[kClassifyItems];
    uint32_t csum = 0;
    uint64_t kc0 = 0, kc1 = 0;  // categories 0..3 in 16-bit counters, 4..8 in 12-bit counters
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        const int64_t i = base + q;
        catq[q] = -1;
        cq[q] = 0;
        if (i < F) {
            const int32_t v = a.front[i];
            int64_t deg = 0;
            if (v < 0 || v >= a.num_nodes) {
                set_status(a.status, GNN_ERR_OUT_OF_RANGE);
            } else {
                deg = row_ptr(a.indptr, a.ib, v + 1) - row_ptr(a.indptr, a.ib, v);
            }
            const int32_t c = deg <= a.k ? static_cast<int32_t>(deg) : a.k;
            const int32_t cat = node_cat(node_class(deg, a.k, a.group_max, a.wave_max), deg);
            if (a.inv_mask) a.inv_mask[i] = 0u;
            cq[q] = c;
            catq[q] = cat;
            csum += static_cast<uint32_t>(c);
            if (cat < 4) kc0 += 1ull << (16 * cat);
            else kc1 += 1ull << (12 * (cat - 4));
        }
    }
    uint32_t ctot;
    uint64_t ktot0, ktot1;
    uint32_t coff = block_exclusive_scan<uint32_t, kClassifyThreads>(csum, &ctot, sm_c);
    uint64_t koff0 = block_exclusive_scan<uint64_t, kClassifyThreads>(kc0, &ktot0, sm_k0);
    uint64_t koff1 = block_exclusive_scan<uint64_t, kClassifyThreads>(kc1, &ktot1, sm_k1);
    if (threadIdx.x < 64) {
        const int lane = lane_id();
        uint32_t before = 0;
        if (tile == 0) {
            if (lane == 0) lb_publish(&a.lb.words[0], kLbInclusive, ctot);
        } else {
            if (lane == 0) lb_publish(&a.lb.words[tile], kLbAggregate, ctot);
            before = lb_exclusive(a.lb.words, tile);
            if (lane == 0) lb_publish(&a.lb.words[tile], kLbInclusive, before + ctot);
        }
        if (lane < kCats) {
            const uint32_t n = cat_count(ktot0, ktot1, lane);
            s_base[lane] = n ? atomicAdd(&a.totals[1 + lane], n) : 0u;
        }
        if (lane == 0) {
            s_prefix = before;
            if (tile == last) {
                const uint32_t total = before + ctot;
                a.blk_indptr[F] = static_cast<int32_t>(total);
                *a.d_E = total;
                a.totals[0] = total;
                if (static_cast<int64_t>(total) > a.E_cap) set_status(a.status, GNN_ERR_CAPACITY);
            }
        }
    }
    __syncthreads();
    coff += s_prefix;
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        const int32_t cat = catq[q];
        if (cat < 0) continue;
        const int64_t i = base + q;
        a.blk_indptr[i] = static_cast<int32_t>(coff);
        coff += static_cast<uint32_t>(cq[q]);
        uint32_t r;
        if (cat < 4) {
            r = static_cast<uint32_t>((koff0 >> (16 * cat)) & 0xFFFF);
            koff0 += 1ull << (16 * cat);
        } else {
            r = static_cast<uint32_t>((koff1 >> (12 * (cat - 4))) & 0xFFF);
            koff1 += 1ull << (12 * (cat - 4));
        }
        a.lists[static_cast<int64_t>(cat) * a.F_cap + s_base[cat] + r] = static_cast<int32_t>(i);
    }
}

// Longest row the sampler handles (positions are int32).
constexpr int64_t kMaxRowLength = 0x7FFFFFFFLL;

// Output e of the block gets neighbour id `id`; with a union bitmap to accumulate (a super-batch
// relabelled in the union's positions), the id's bit is set too.  The atomic's result is unused,
// so the store is posted and the lane does not wait for it.
template <bool MARK>
__device__ __forceinline__ void emit_id(const HopArgs &a, int64_t e, int32_t id) {
    if (e >= 0 && e < a.E_cap) a.blk_gid[e] = id;
    if (MARK) {
        if (id >= 0 && id < a.num_nodes) atomicOr(&a.mark[id >> 5], 1u << (id & 31));
        else set_status(a.status, GNN_ERR_OUT_OF_RANGE);
    }
}

// ---- threshold selection helpers ----------------------------------------------------------------
//
// Thresholds have the form tau = T * 2^32 + (2^32 - 1), so key <= tau exactly when the key's high
// 32 bits are <= T: the candidate test needs only the high word of each key, and the full key is
// formed for the candidates alone (they are ranked by (key, position)).

// High 32 bits of the product of mix64's second step, and the key's high word from it.
__device__ __forceinline__ uint64_t mix64_pre(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    return (z ^ (z >> 27)) * 0x94D049BB133111EBULL;   // mix64(z) = this ^ (this >> 31)
}
__device__ __forceinline__ uint32_t key_high(uint64_t w) {
    const uint32_t h = static_cast<uint32_t>(w >> 32);
    return h ^ (h >> 31);
}
__device__ __forceinline__ uint64_t key_full(uint64_t w) { return w ^ (w >> 31); }

// T whose expected number of keys <= tau among deg uniform keys is ~ k + 3 sqrt(k) + 6.  Only
// the number of threshold passes depends on T (any T gives the exact selection), so it is taken
// in single precision with a fast reciprocal.
__device__ __forceinline__ uint32_t initial_tau(int64_t deg, int k) {
    const float kf = static_cast<float>(k);
    const float mu = kf + 3.0f * sqrtf(kf) + 6.0f;
    const float p = __fdividef(mu, static_cast<float>(deg));
    if (!(p < 1.0f)) return 0xFFFFFFFFu;
    const float t = p * 4294967296.0f;
    if (!(t < 4294967040.0f)) return 0xFFFFFFFFu;   // the largest float below 2^32
    return static_cast<uint32_t>(t);
}

// Next T after a pass that collected `cnt` keys <= tau.  Returns false when done (k <= cnt <= cap)
// and sets *fail when no threshold can separate the keys (more than cap - k keys sharing one high
// word: never expected).
__device__ __forceinline__ bool next_tau(int cnt, int k, int cap, uint32_t &tau, uint32_t &lo,
                                         uint32_t &hi, bool &has_lo, bool &has_hi, bool &fail) {
    if (cnt < k) {
        has_lo = true;
        lo = tau;
        if (has_hi) tau = lo + (hi - lo) / 2;
        else tau = tau >= 0x3FFFFFFFu ? 0xFFFFFFFFu : ((tau << 2) | 3u);
    } else if (cnt > cap) {
        has_hi = true;
        hi = tau;
        const uint32_t l = has_lo ? lo : 0u;
        tau = l + (hi - l) / 2;
    } else {
        return false;
    }
    if (has_lo && has_hi && hi - lo <= 1) {
        fail = true;
        return false;
    }
    return true;
}

// ---- candidate collection --------------------------------------------------------------------
//
// Set bits of x in the lanes below this one (the lane-mask count instruction pair); with x a
// ballot restricted to this lane's group, the group's lanes below it.
__device__ __forceinline__ int lanes_below(uint64_t x) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(x >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(x), 0u)));
}

// Lanes of this lane's group whose bit is set in the wavefront ballot b, given x = b restricted
// to the group: a scalar count for a whole-wavefront group, else the population count of x (two
// count instructions that also add it to the running total).
template <int G>
__device__ __forceinline__ int group_lanes(uint64_t b, uint64_t x) {
    if constexpr (G == 64) return __popcll(b);
    else return __popcll(x);
}

// A candidate as the lanes' classes keep it while collecting: one 8-byte LDS entry, its key's
// high word above its position (the full key is formed again from the position only when the
// high words cannot decide the selection).  Stored as its two 32-bit halves: one paired LDS
// store, no 64-bit register pair to build.
__device__ __forceinline__ void put_cand(uint64_t *s_cand, int pos, uint32_t hi, int32_t j) {
    uint32_t *w = reinterpret_cast<uint32_t *>(s_cand + pos);
    w[0] = static_cast<uint32_t>(j);
    w[1] = hi;
}
__device__ __forceinline__ int32_t cand_pos(uint64_t e) {
    return static_cast<int32_t>(static_cast<uint32_t>(e));
}

// Keys of positions j = gl, gl + G, ... of a row of length deg (G lanes, lane gl); the ones
// <= tau are appended, in ascending position, to s_cand (first CAP kept) as packed entries.
// Returns the number of keys <= tau.  Four keys per lane per step (positions j0 + q G + gl,
// q = 0..3); the position bound is checked only in the tail.  Rows are shorter than 2^31 (checked
// by the caller).  The step's candidates are placed only when some lane of the wavefront has one
// (a scalar test of the unmasked ballots); each lane's place counts its group's lanes only.
template <int G, int CAP>
__device__ __forceinline__ int collect_lanes(uint64_t ns, int32_t deg, uint32_t tau, int gl,
                                             uint64_t gmask, uint64_t *s_cand) {
    constexpr int U = 4;
    const uint64_t step = kGamma * static_cast<uint64_t>(G);
    uint64_t z = ns + kGamma * static_cast<uint64_t>(gl + 1);
    int cnt = 0;
    const int32_t main_end = deg / (U * G) * (U * G);
    int32_t j0 = 0;
    for (; j0 < main_end; j0 += U * G) {
        uint32_t h[U];
        bool p[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            h[q] = key_high(mix64_pre(z + step * q));
            p[q] = h[q] <= tau;
        }
        z += step * U;
        uint64_t m[U];
#pragma unroll
        for (int q = 0; q < U; ++q) m[q] = __ballot(p[q]);
        if (m[0] | m[1] | m[2] | m[3]) {
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const uint64_t x = G == 64 ? m[q] : (m[q] & gmask);
                if (p[q]) {
                    const int pos = cnt + lanes_below(x);
                    if (pos < CAP) put_cand(s_cand, pos, h[q], j0 + q * G + gl);
                }
                cnt += group_lanes<G>(m[q], x);
            }
        }
    }
    for (; j0 < deg; j0 += G) {
        const int32_t j = j0 + gl;
        const uint32_t h = key_high(mix64_pre(z));
        z += step;
        const bool p = j < deg && h <= tau;
        const uint64_t m = __ballot(p);
        const uint64_t x = G == 64 ? m : (m & gmask);
        if (p) {
            const int pos = cnt + lanes_below(x);
            if (pos < CAP) put_cand(s_cand, pos, h, j);
        }
        cnt += group_lanes<G>(m, x);
    }
    return cnt;
}

// ---- candidate ranking ------------------------------------------------------------------------------
//
// Rank of candidate (kc, jc) among the cnt candidates in s_key / s_pos: how many precede it in
// (key, position) order.  Eight candidates per round, their LDS loads issued together, so one LDS
// round trip serves eight comparisons (one per candidate had left a wavefront waiting on LDS for
// most of its per-node selection).
__device__ __forceinline__ int rank_of(const uint64_t *s_key, const int32_t *s_pos, int cnt,
                                       uint64_t kc, int32_t jc) {
    constexpr int R = 8;
    int r = 0;
    int t = 0;
    for (; t + R <= cnt; t += R) {
        uint64_t kt[R];
        int32_t jt[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            kt[q] = s_key[t + q];
            jt[q] = s_pos[t + q];
        }
#pragma unroll
        for (int q = 0; q < R; ++q) r += (kt[q] < kc) | ((kt[q] == kc) & (jt[q] < jc));
    }
    for (; t < cnt; ++t) {
        const uint64_t kt = s_key[t];
        r += (kt < kc) | ((kt == kc) & (s_pos[t] < jc));
    }
    return r;
}

// Among the cnt positions in s_pos whose sign bit marks them selected, how many selected ones lie
// before position jc; eight per round as above.
__device__ __forceinline__ int selected_before(const int32_t *s_pos, int cnt, int32_t jc) {
    constexpr int R = 8;
    int r = 0;
    int t = 0;
    for (; t + R <= cnt; t += R) {
        int32_t pt[R];
#pragma unroll
        for (int q = 0; q < R; ++q) pt[q] = s_pos[t + q];
#pragma unroll
        for (int q = 0; q < R; ++q) r += (pt[q] < 0) & ((pt[q] & 0x7FFFFFFF) < jc);
    }
    for (; t < cnt; ++t) {
        const int32_t pt = s_pos[t];
        r += (pt < 0) & ((pt & 0x7FFFFFFF) < jc);
    }
    return r;
}

// Rank of high word hc among the high words of the cnt candidates (the odd 32-bit halves of the
// packed entries in s_key): how many are smaller.  Eight per round, as in rank_of.
__device__ __forceinline__ int rank_hi(const uint64_t *s_key, int cnt, uint32_t hc) {
    const uint32_t *s_hi = reinterpret_cast<const uint32_t *>(s_key) + 1;
    constexpr int R = 8;
    int r = 0;
    int t = 0;
    for (; t + R <= cnt; t += R) {
        uint32_t h[R];
#pragma unroll
        for (int q = 0; q < R; ++q) h[q] = s_hi[2 * (t + q)];
#pragma unroll
        for (int q = 0; q < R; ++q) r += h[q] < hc;
    }
    for (; t < cnt; ++t) r += s_hi[2 * t] < hc;
    return r;
}

// ---- one random node on G lanes of a wavefront ---------------------------------------------------
//
// Control flow is uniform across the G lanes of the group; other groups of the same wavefront may
// be elsewhere.  s_key / s_pos are the group's private LDS candidate arrays of CAP entries.
template <int G, int CAP, int IB, bool ADJ, bool MARK>
__device__ __forceinline__ void sample_node_lanes(const HopArgs &a, int32_t i, uint64_t *s_key,
                                                  int32_t *s_pos, int gl, uint64_t gmask) {
    const int k = a.k;
    const int32_t v = a.front[i];
    const int64_t start = row_at<IB>(a.indptr, v);
    const int64_t deg = row_at<IB>(a.indptr, v + 1) - start;
    const int32_t *row = adj_row<ADJ>(a, v, start);
    const int64_t out0 = a.blk_indptr[i];
    const uint64_t ns = mix64(a.hop_seed ^ static_cast<uint64_t>(static_cast<uint32_t>(v)));
    uint32_t tau = initial_tau(deg, k), lo = 0, hi = 0;
    bool has_lo = false, has_hi = false, fail = deg > kMaxRowLength;
    if (fail && gl == 0) set_status(a.status, GNN_ERR_UNSUPPORTED);   // positions are int32
    int cnt = 0;
    for (int it = 0; it < 128 && !fail; ++it) {
        cnt = collect_lanes<G, CAP>(ns, static_cast<int32_t>(deg), tau, gl, gmask, s_key);
        if (!next_tau(cnt, k, CAP, tau, lo, hi, has_lo, has_hi, fail)) break;
    }
    if (fail || cnt < k || cnt > CAP) {
        if (gl == 0) set_status(a.status, GNN_ERR_INTERNAL);
        cnt = 0;
    }
    wave_lds_sync();
    // Candidates sit in ascending position (packed: high word, position); keep those of rank < k
    // among (key, pos).  First by the keys' high words alone: the candidates with fewer than k
    // smaller high words include the k first in (key, pos) order (a candidate of rank < k has
    // fewer than k candidates before it, and every candidate with a smaller high word is before
    // it), so when there are exactly k of them they are those k.  More than k means high words
    // tied at the k-th place: the candidates' full keys are formed again from their positions
    // (into s_key, positions into s_pos) and the node is ranked by (key, pos).  Bit b of sel_bits
    // is this lane's candidate of round b.
    static_assert((CAP + G - 1) / G <= 32, "selection rounds fit one word");
    uint32_t sel_bits = 0;
    int n_sel = k + 1;
    if (!a.exact_rank) {
        n_sel = 0;
        for (int c0 = 0, b = 0; c0 < cnt; c0 += G, ++b) {
            const int c = c0 + gl;
            bool sel = false;
            if (c < cnt) sel = rank_hi(s_key, cnt, static_cast<uint32_t>(s_key[c] >> 32)) < k;
            n_sel += __popcll(__ballot(sel) & gmask);
            sel_bits |= static_cast<uint32_t>(sel) << b;
        }
    }
    const bool exact = n_sel != k;
    if (exact) {
        for (int c0 = 0; c0 < cnt; c0 += G) {   // each lane its own candidates, in place
            const int c = c0 + gl;
            if (c < cnt) {
                const int32_t j = cand_pos(s_key[c]);
                s_key[c] = key_full(mix64_pre(ns + kGamma * static_cast<uint64_t>(j + 1)));
                s_pos[c] = j;
            }
        }
        wave_lds_sync();
        sel_bits = 0;
        for (int c0 = 0, b = 0; c0 < cnt; c0 += G, ++b) {
            const int c = c0 + gl;
            bool sel = false;
            if (c < cnt) sel = rank_of(s_key, s_pos, cnt, s_key[c], s_pos[c]) < k;
            sel_bits |= static_cast<uint32_t>(sel) << b;
        }
    }
    int outc = 0;
    for (int c0 = 0, b = 0; c0 < cnt; c0 += G, ++b) {
        const bool sel = (sel_bits >> b) & 1u;
        const uint64_t m = __ballot(sel) & gmask;
        if (sel) {
            const int64_t o = out0 + outc + lanes_below(m);
            const int c = c0 + gl;
            emit_id<MARK>(a, o, row[exact ? s_pos[c] : cand_pos(s_key[c])]);
        }
        outc += __popcll(m);
    }
    wave_lds_sync();
}

// ---- one giant-row node on a whole workgroup -------------------------------------------------------
template <int IB, bool ADJ, bool MARK>
__device__ __forceinline__ void sample_node_block(const HopArgs &a, int32_t i, uint64_t *s_key,
                                                  int32_t *s_pos, uint32_t *s_cnt) {
    constexpr int NT = kBlockThreads;
    constexpr int CAP = kBlockCap;
    constexpr int U = 4;
    const int lane = lane_id();
    const int k = a.k;
    const int32_t v = a.front[i];
    const int64_t start = row_at<IB>(a.indptr, v);
    const int64_t deg64 = row_at<IB>(a.indptr, v + 1) - start;
    const int32_t *row = adj_row<ADJ>(a, v, start);
    const int64_t out0 = a.blk_indptr[i];
    const uint64_t ns = mix64(a.hop_seed ^ static_cast<uint64_t>(static_cast<uint32_t>(v)));
    uint32_t tau = initial_tau(deg64, k), lo = 0, hi = 0;
    bool has_lo = false, has_hi = false, fail = deg64 > kMaxRowLength;
    if (fail && threadIdx.x == 0) set_status(a.status, GNN_ERR_UNSUPPORTED);   // positions are int32
    const int32_t deg = fail ? 0 : static_cast<int32_t>(deg64);
    int cnt = 0;
    const uint64_t step = kGamma * static_cast<uint64_t>(NT);
    const int32_t main_end = deg / (U * NT) * (U * NT);
    for (int it = 0; it < 128 && !fail; ++it) {
        if (threadIdx.x == 0) *s_cnt = 0;
        __syncthreads();
        uint64_t z = ns + kGamma * static_cast<uint64_t>(threadIdx.x + 1);
        int32_t j0 = 0;
        for (; j0 < main_end; j0 += U * NT) {
            uint64_t w[U];
            bool p[U];
#pragma unroll
            for (int q = 0; q < U; ++q) {
                w[q] = mix64_pre(z + step * q);
                p[q] = key_high(w[q]) <= tau;
            }
            z += step * U;
            uint64_t m[U];
#pragma unroll
            for (int q = 0; q < U; ++q) m[q] = __ballot(p[q]);
            if (m[0] | m[1] | m[2] | m[3]) {
                uint32_t wbase = 0;
                if (lane == 0)
                    wbase = atomicAdd(s_cnt, static_cast<uint32_t>(__popcll(m[0]) + __popcll(m[1]) +
                                                                   __popcll(m[2]) + __popcll(m[3])));
                wbase = __shfl(wbase, 0, 64);
#pragma unroll
                for (int q = 0; q < U; ++q) {
                    if (p[q]) {
                        const uint32_t pos = wbase + static_cast<uint32_t>(lanes_below(m[q]));
                        if (pos < CAP) {
                            s_key[pos] = key_full(w[q]);
                            s_pos[pos] = j0 + q * NT + static_cast<int32_t>(threadIdx.x);
                        }
                    }
                    wbase += __popcll(m[q]);
                }
            }
        }
        for (; j0 < deg; j0 += NT) {
            const int32_t j = j0 + static_cast<int32_t>(threadIdx.x);
            const uint64_t w = mix64_pre(z);
            z += step;
            const bool p = j < deg && key_high(w) <= tau;
            const uint64_t m = __ballot(p);
            if (m) {
                uint32_t wbase = 0;
                if (lane == 0) wbase = atomicAdd(s_cnt, static_cast<uint32_t>(__popcll(m)));
                wbase = __shfl(wbase, 0, 64);
                if (p) {
                    const uint32_t pos = wbase + static_cast<uint32_t>(lanes_below(m));
                    if (pos < CAP) {
                        s_key[pos] = key_full(w);
                        s_pos[pos] = j;
                    }
                }
            }
        }
        __syncthreads();
        cnt = static_cast<int>(*s_cnt);
        __syncthreads();
        if (!next_tau(cnt, k, CAP, tau, lo, hi, has_lo, has_hi, fail)) break;
    }
    if (fail || cnt < k || cnt > CAP) {
        if (threadIdx.x == 0) set_status(a.status, GNN_ERR_INTERNAL);
        cnt = 0;
    }
    // Candidates are in arbitrary order: rank by (key, pos); the selected ones (rank < k) get the
    // sign bit of their position (positions are < 2^31), then each is placed by position.
    static_assert((kBlockCap + NT - 1) / NT <= 32, "selection bits fit one word");
    uint32_t sel = 0;
    for (int c = threadIdx.x, b = 0; c < cnt; c += NT, ++b)
        if (rank_of(s_key, s_pos, cnt, s_key[c], s_pos[c]) < k) sel |= 1u << b;
    __syncthreads();
    for (int c = threadIdx.x, b = 0; c < cnt; c += NT, ++b)
        if (sel & (1u << b)) s_pos[c] |= static_cast<int32_t>(0x80000000u);
    __syncthreads();
    for (int c = threadIdx.x, b = 0; c < cnt; c += NT, ++b) {
        if (!(sel & (1u << b))) continue;
        const int32_t jc = s_pos[c] & 0x7FFFFFFF;
        emit_id<MARK>(a, out0 + selected_before(s_pos, cnt, jc), row[jc]);
    }
    __syncthreads();
}

// ---- all four classes in one launch ---------------------------------------------------------------
//
// Workgroups of kBlockThreads lanes.  The first nb_block workgroups take BLOCK nodes (a whole
// workgroup each), the next nb_wave take WAVE nodes (one wavefront each), the next nb_group GROUP
// nodes (16 lanes each), the rest FULL nodes (one lane each).  The long-running giant rows are
// dispatched first and the short classes fill the machine around them.  Each role walks its class
// list with a static stride, so no two wavefronts contend for a shared counter.
constexpr int kWavesPerBlock = kBlockThreads / 64;
static_assert(kWavesPerBlock * kWaveCap == kBlockCap, "WAVE slots fill the shared LDS arrays");
static_assert(kWavesPerBlock * (64 / kGroupLanes) * kGroupCap == kBlockCap,
              "GROUP slots fill the shared LDS arrays");

// Zeroes the sub-batch bitmaps (and byte maps) that the hop's distribution marks next; the
// sampler's grid does it, hidden under its own hashing.
__device__ __forceinline__ void zero_sub_maps(const HopArgs &a) {
    if (a.zero_words == nullptr) return;
    int64_t bound = *a.zero_da + *a.zero_db;
    bound = bound < 0 ? 0 : (bound > 32 * a.zero_stride ? 32 * a.zero_stride : bound);
    const int64_t words = (bound + 31) >> 5;
    // The grid's threads in zero_g equal shares, share g clearing sub-batch g's region (one
    // division per thread, none per store): its bitmap words, and its byte map (32 bytes a word,
    // two 16-byte stores; each byte map starts 32-byte aligned).
    const int64_t threads = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t share = threads / a.zero_g;
    share = share > 0 ? share : 1;
    const int64_t g = t / share;
    if (g >= a.zero_g) return;
    uint32_t *zw = a.zero_words + g * a.zero_stride;
    uint4 *zb = a.zero_bytes != nullptr
                    ? reinterpret_cast<uint4 *>(a.zero_bytes + g * 8 * a.zero_stride)
                    : nullptr;
    const int64_t n = zb != nullptr ? 2 * words : words;
    for (int64_t i = t - g * share; i < n; i += share) {
        if (i < words) zw[i] = 0u;
        if (zb != nullptr) zb[i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Compiled for each indptr width (IB bytes), for graphs with and without the HBM adjacency cache
// (ADJ) and for hops with and without a union bitmap to mark (MARK), so that no per-node code
// tests any of them.
template <int IB, bool ADJ, bool MARK>
__global__ __launch_bounds__(kBlockThreads, 8) void k_sample(HopArgs a, int32_t nb_block,
                                                         int32_t nb_wave, int32_t nb_group) {
    __shared__ uint64_t s_key[kBlockCap];
    __shared__ int32_t s_pos[kBlockCap];
    __shared__ uint32_t s_cnt;
    zero_sub_maps(a);
    const int lane = lane_id();
    // the wavefront's index as a scalar, so that a whole-wavefront row's bounds, seed and
    // threshold are computed once in scalar registers rather than by every lane
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    int bid = static_cast<int>(blockIdx.x);
    if (bid < nb_block) {
        const int64_t n = class_total(a.totals, kBlock);
        const int32_t *list = a.lists + static_cast<int64_t>(kCatBlock) * a.F_cap;
        for (int64_t item = bid; item < n; item += nb_block)
            sample_node_block<IB, ADJ, MARK>(a, list[item], s_key, s_pos, &s_cnt);
        return;
    }
    bid -= nb_block;
    if (bid < nb_wave) {
        // The list is ordered by degree bucket, largest first.  Rows of 1024 positions or more
        // take a wavefront each: wavefront w takes item w of even rounds and item W-1-w of odd ones
        // (W wavefronts), which pairs large rows with small.  With fanouts up to 10, rows of the
        // two smallest buckets (fewer than 1024 positions) go two to a wavefront, 32 lanes each,
        // consecutive items of one bucket together (degrees within 2x of each other), so the
        // per-row work -- row bounds, threshold, ranking, output -- is shared by two rows
        // (k_sample per super-batch: 111M-node 0.690 -> 0.673 ms, mid 0.237 -> 0.230; with the
        // dense workload's fanout 25 pairs measured 5% slower: each row then has ~46 candidates).
        const int64_t n = class_total(a.totals, kWave);
        const bool pairs_fit = 4 * a.k <= kWaveCap / 2 && a.k <= 10;
        const int64_t n_pair = pairs_fit ? static_cast<int64_t>(a.totals[3 + kWaveBuckets - 2]) +
                                               static_cast<int64_t>(a.totals[3 + kWaveBuckets - 1])
                                         : 0;
        const int64_t n_one = n - n_pair;
        const int64_t W = static_cast<int64_t>(nb_wave) * kWavesPerBlock;
        const int64_t w = static_cast<int64_t>(bid) * kWavesPerBlock + wv;
        for (int64_t r0 = 0, round = 0; r0 < n_one; r0 += W, ++round) {
            const int64_t item = r0 + ((round & 1) ? W - 1 - w : w);
            if (item < n_one)
                sample_node_lanes<64, kWaveCap, IB, ADJ, MARK>(a, wave_item(a, item), s_key + wv * kWaveCap,
                                                s_pos + wv * kWaveCap, lane, ~0ull);
        }
        const int half = lane >> 5;
        const uint64_t hmask = half ? 0xFFFFFFFF00000000ull : 0x00000000FFFFFFFFull;
        for (int64_t p = w; 2 * p < n_pair; p += W) {
            const int64_t item = n_one + 2 * p + half;
            if (item < n)
                sample_node_lanes<32, kWaveCap / 2, IB, ADJ, MARK>(a, wave_item(a, item),
                                                    s_key + wv * kWaveCap + half * (kWaveCap / 2),
                                                    s_pos + wv * kWaveCap + half * (kWaveCap / 2),
                                                    lane & 31, hmask);
        }
        return;
    }
    bid -= nb_wave;
    if (bid < nb_group) {
        constexpr int G = kGroupLanes;
        constexpr int SLOTS = kWavesPerBlock * (64 / G);
        const int grp = lane / G;
        const int slot = wv * (64 / G) + grp;
        const uint64_t gmask = ((1ull << G) - 1ull) << (grp * G);
        const int64_t n = class_total(a.totals, kGroup);
        const int32_t *list = a.lists + static_cast<int64_t>(kGroup) * a.F_cap;
        for (int64_t item = static_cast<int64_t>(bid) * SLOTS + slot; item < n;
             item += static_cast<int64_t>(nb_group) * SLOTS)
            sample_node_lanes<G, kGroupCap, IB, ADJ, MARK>(a, list[item], s_key + slot * kGroupCap,
                                            s_pos + slot * kGroupCap, lane % G, gmask);
        return;
    }
    bid -= nb_group;
    const int64_t n = class_total(a.totals, kFull);
    const int64_t nb_full = static_cast<int64_t>(gridDim.x) - nb_block - nb_wave - nb_group;
    for (int64_t t = static_cast<int64_t>(bid) * kBlockThreads + threadIdx.x; t < n;
         t += nb_full * kBlockThreads) {
        const int32_t i = a.lists[t];
        const int32_t v = a.front[i];
        if (v < 0 || v >= a.num_nodes) continue;
        const int64_t st = row_at<IB>(a.indptr, v);
        const int64_t deg = row_at<IB>(a.indptr, v + 1) - st;
        const int64_t o = a.blk_indptr[i];
        const int32_t *row = adj_row<ADJ>(a, v, st);
        for (int64_t j = 0; j < deg; ++j) emit_id<MARK>(a, o + j, row[j]);
    }
}

// ---- adjacency cache set-up (not on the mini-batch path) -------------------------------------

__global__ __launch_bounds__(256) void k_adj_degrees(const void *indptr, int32_t ib,
                                                     const int32_t *hot, int64_t n, int64_t *deg) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int32_t v = hot[i];
        deg[i] = row_ptr(indptr, ib, v + 1) - row_ptr(indptr, ib, v);
    }
}

// One wavefront per selected node: its row copied to rows + off[i], then its offset published.
__global__ __launch_bounds__(256) void k_adj_fill(const void *indptr, int32_t ib,
                                                  const int32_t *indices, const int32_t *node,
                                                  const int64_t *off, int64_t n, int32_t *rows,
                                                  int64_t *adj_off) {
    const int lane = lane_id();
    const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
    for (int64_t i = w0; i < n; i += nw) {
        const int32_t v = node[i];
        const int64_t st = row_ptr(indptr, ib, v);
        const int64_t deg = row_ptr(indptr, ib, v + 1) - st;
        const int64_t o = off[i];
        for (int64_t j = lane; j < deg; j += 64) rows[o + j] = indices[st + j];
        if (lane == 0) adj_off[v] = o;
    }
}

// ---- launchers ---------------------------------------------------------------------------------

// Words the classification grid clears itself (a few per thread); a larger clear region gets a
// fill kernel of its own, sized for it.
constexpr int64_t kClassifyClearPerThread = 16;

hipError_t launch_classify(HopArgs a, hipStream_t s) {
    if (a.clear_n > static_cast<int64_t>(a.nb) * kClassifyThreads * kClassifyClearPerThread) {
        const hipError_t e = launch_fill_u32(a.clear_ptr, a.clear_n, 0u, s);
        if (e != hipSuccess) return e;
        a.clear_n = 0;
    }
    hipLaunchKernelGGL(k_classify, dim3(a.nb), dim3(kClassifyThreads), 0, s, a);
    return hipGetLastError();
}

// Workgroups per role, capped.  Four sampler workgroups fit a CU, so 1024 are resident at a time:
// the one-wavefront role's 2048 run as two generations, the second taking the CUs that the first
// frees, which balances their uneven rows at workgroup granularity; the 16-lane role's 1024 fill
// the machine once the one-wavefront rows are done.  Measured (k_sample per super-batch, caps
// block/wave/group/full): 2048/1024/512/128 -> 256/2048/1024/256: 111M-node 0.724 -> 0.700 ms,
// dense 0.187 -> 0.174, mid 0.251 -> 0.240; 4096 or 8192 one-wavefront workgroups, 2048 16-lane
// ones, or 128 giant-row ones measured equal or slower.  With two short rows to a wavefront, 512
// giant-row workgroups instead of 256: 111M-node 0.667 -> 0.649 ms, dense and mid unchanged
// (1024: 0.645, the others unchanged or slower).
hipError_t launch_sample(const HopArgs &a, hipStream_t s) {
    const int64_t F = a.F_cap;
    const int nb_block = static_cast<int>(grid_for(F, 1, 512));
    const int nb_wave = static_cast<int>(grid_for(F, kWavesPerBlock, 2048));
    const int nb_group = static_cast<int>(grid_for(F, kWavesPerBlock * (64 / kGroupLanes), 1024));
    const int nb_full = static_cast<int>(grid_for(F, kBlockThreads, 256));
    const dim3 grid(nb_block + nb_wave + nb_group + nb_full);
    const dim3 block(kBlockThreads);
    const int shape = (a.ib == 8 ? 4 : 0) | (a.adj_off != nullptr ? 2 : 0) | (a.mark != nullptr ? 1 : 0);
    switch (shape) {
    case 0: hipLaunchKernelGGL((k_sample<4, false, false>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    case 1: hipLaunchKernelGGL((k_sample<4, false, true>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    case 2: hipLaunchKernelGGL((k_sample<4, true, false>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    case 3: hipLaunchKernelGGL((k_sample<4, true, true>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    case 4: hipLaunchKernelGGL((k_sample<8, false, false>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    case 5: hipLaunchKernelGGL((k_sample<8, false, true>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    case 6: hipLaunchKernelGGL((k_sample<8, true, false>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    default: hipLaunchKernelGGL((k_sample<8, true, true>), grid, block, 0, s, a, nb_block, nb_wave, nb_group); break;
    }
    return hipGetLastError();
}

hipError_t launch_adj_degrees(const void *indptr, int32_t ib, const int32_t *hot, int64_t n,
                              int64_t *deg, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_adj_degrees, dim3(grid_for(n, 256, 4096)), dim3(256), 0, s, indptr, ib,
                       hot, n, deg);
    return hipGetLastError();
}

hipError_t launch_adj_fill(const void *indptr, int32_t ib, const int32_t *indices,
                           const int32_t *node, const int64_t *off, int64_t n, int32_t *rows,
                           int64_t *adj_off, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_adj_fill, dim3(grid_for(n, 4, 8192)), dim3(256), 0, s, indptr, ib,
                       indices, node, off, n, rows, adj_off);
    return hipGetLastError();
}

}  // namespace gnnmb
