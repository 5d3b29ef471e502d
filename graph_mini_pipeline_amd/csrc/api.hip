// C ABI of the mini-batch library: argument validation, workspace carving, launch sequencing on
// one stream with no host synchronisation, the feature store and the stage timer.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "common.hpp"

using namespace gnnmb;

// Dynamic-Cache (GARDEN Sec. IV.B): host bookkeeping of the mini-batch count and weights, and
// the device arrays of the scores and of the refresh.
struct DynCache {
    gnn_dyn_cache_params p;
    std::mutex mu;
    double w_next = 1.0;          // weight of the next observed mini-batch: W * gamma^-t
    int64_t steps = 0, steps_at_refresh = 0;
    int32_t refreshes = 0;
    double *score = nullptr;      // [num_nodes] scaled scores
    uint32_t *touched = nullptr;  // [ceil(num_nodes / 32)]
    uint32_t *member = nullptr;   // [ceil(num_nodes / 32)]
    uint32_t *cand = nullptr;     // [num_nodes]
    uint32_t *key_hi = nullptr;   // [num_nodes]
    uint32_t *key_lo = nullptr;   // [num_nodes]
    int32_t *free_rows = nullptr; // [k_dyn]
    int32_t *admit = nullptr;     // [k_dyn]
    int32_t *row_node = nullptr;  // [k_dyn]
    uint8_t *filled = nullptr;    // [k_dyn rounded up to 4]
    DynState *state = nullptr;
};

struct gnn_feature_store {
    const float *table;  // device-addressable table (mapped pointer for pinned host memory)
    int32_t on_host;
    int64_t num_nodes, d, ld;
    int64_t cache_rows;  // static-cache rows (slots 0..cache_rows-1)
    float *cache;   // [cache_rows (+ k_dyn), ld] in HBM, or NULL
    int32_t *slot;  // [num_nodes] cache slot of each node, -1 if not cached; NULL if no cache
    DynCache *dyn;  // NULL: no Dynamic-Cache
};

struct gnn_adjacency_cache {
    int64_t num_nodes;
    int64_t *adj_off;  // [num_nodes] offset of each node's cached row in rows, -1 if not cached
    int32_t *rows;     // the cached rows, back to back
    int64_t n_rows, n_entries;
};

// Events per record: call start, end of sampling, then per sub-batch the ends of its gather and
// of its outermost-block mean (batched gather: slot 2 ends the one gather launch and slot 1 + 2G
// the one outermost-mean launch), then the end of the call; then two per hop around the sampling
// kernel (k_sample) of that hop.
constexpr int kSampleEvents = 3 + 2 * GNN_MAX_GROUP;
constexpr int kTimerSlots = kSampleEvents + 2 * GNN_MAX_HOPS;

struct gnn_timer {
    int32_t n_records;
    int32_t cursor;
    std::vector<hipEvent_t> ev;   // n_records * kTimerSlots
    std::vector<int32_t> group;   // sub-batches of each recorded call
    std::vector<int32_t> hops;    // hops of each recorded call
    std::vector<int32_t> batched; // 1: one gather launch and one outermost-mean launch
};

namespace {

#define GNN_TRY_HIP(expr)                                \
    do {                                                 \
        if ((expr) != hipSuccess) return GNN_ERR_HIP;    \
    } while (0)

#define GNN_TRY(expr)                                    \
    do {                                                 \
        const gnn_status st_ = (expr);                   \
        if (st_ != GNN_OK) return st_;                   \
    } while (0)

constexpr int64_t kInt32Max = 2147483647LL;
// Flattened (row, element) index spaces of the gather and mean kernels stay below 2^31 so that a
// grid-stride step never wraps a 32-bit index.
constexpr int64_t kFlatMax = 2147483647LL;

// Bump allocator over the caller's workspace; with base == NULL it only measures.
struct Carver {
    char *base;
    size_t off = 0;
    template <typename T>
    T *take(int64_t n) {
        off = (off + 255) & ~static_cast<size_t>(255);
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += static_cast<size_t>(n < 1 ? 1 : n) * sizeof(T);
        return p;
    }
};

struct Workspace {
    int32_t *status;       // [1] at offset 0
    uint32_t *totals;      // [kTotalsStride * GNN_MAX_HOPS] classification totals of each hop
    int64_t *d_U;          // [K + 1] |U_l| of a super-batch
    int64_t *d_uE;         // [K] edges of each union block
    int32_t *lists;        // [kCats FU_max]
    uint32_t *bitmaps;     // [W] over all node ids, then G more of W words (full super-batch
                           // relabel) or G of Wc words (compact super-batch relabel)
    uint2 *rdir;           // rank directory of every bitmap (word prefix, word), same layout
    uint32_t *bsum_w;      // [nbw], then G * nbw or G * nbwc tile popcounts
    uint8_t *bytemaps;     // super-batch: byte maps of the G sub-batch bitmaps (or NULL)
    // super-batch only (the union; the rest: compact relabel only)
    int32_t *U[2];         // U_l, ping-pong by hop parity (full relabel: one buffer)
    int32_t *u_indptr;     // union block
    int32_t *u_gid;
    int32_t *upos;         // [G * P] position of each sub-batch frontier node in U_l
    int32_t *f_pos;        // [G * Fs] position of each sub-batch destination in U_{l+1}
    int32_t *e_pos;        // [G * Es] position of each sub-batch sampled id in U_{l+1}
    // shared outermost means of a super-batch: for each node r of the last hop's union frontier
    // and each sub-batch g, 1 + r's position among g's destinations (0: not there)
    int32_t *inv;          // [U_cap(K-1) * G], valid where the bit of inv_mask is set
    uint32_t *inv_mask;    // [U_cap(K-1)]: bit g set when sub-batch g holds the node
    // union gather of a super-batch (full relabel only; the compact relabel builds U_K as its
    // last union level): U_K, the union of the sub-batches' V_K
    int32_t *uK;           // [U_cap(K)]
    int64_t P, Fs, Es;     // strides of the per-sub-batch arrays
    int64_t W, nbw, Wc, nbwc;
    int32_t mode;          // SuperMode
    size_t bytes;
    // Look-back words of the call's single-pass scans, right after the status word (the call's
    // first kernel zeroes both); each launch takes its slice in launch order.
    uint64_t *arena;
    int64_t arena_words;
    mutable int64_t arena_used = 0;
    int32_t relabel_force = 0;   // RelabelArgs::force of every relabel of the call
    // A slice of `tiles` look-back words followed by `counters` 32-bit ticket counters; NULL words
    // when the arena is exhausted (the bound of carve() covers every launch sequence, so this
    // does not happen).
    LbSlice take_lb(int64_t tiles, int64_t counters = 1) const {
        const int64_t need = tiles + (counters + 1) / 2;
        if (!arena || arena_used + need > arena_words) return LbSlice{nullptr, nullptr};
        LbSlice sl{arena + arena_used, reinterpret_cast<uint32_t *>(arena + arena_used + tiles)};
        arena_used += need;
        return sl;
    }
    // Bytes from the start of the workspace that the call's first kernel clears: the status
    // word, the classification totals and the look-back arena, which the carve lays out back to
    // back.
    int64_t cleared_bytes() const {
        return reinterpret_cast<const char *>(arena + arena_words) - reinterpret_cast<const char *>(status);
    }
};

// The classification of one hop with its look-back words taken from the call's arena.
gnn_status classify_launch(HopArgs h, const Workspace &w, hipStream_t s) {
    h.lb = w.take_lb(h.nb);
    if (h.lb.words == nullptr) return GNN_ERR_INTERNAL;
    return launch_classify(h, s) == hipSuccess ? GNN_OK : GNN_ERR_HIP;
}

// A relabel launch sequence with its look-back words taken from the call's arena.
gnn_status relabel_launch(RelabelArgs r, const Workspace &w, hipStream_t s) {
    r.force = w.relabel_force;
    r.lb = w.take_lb(relabel_lb_words(r), r.nbm);
    if (r.lb.words == nullptr) return GNN_ERR_INTERNAL;
    return launch_relabel(r, s) == hipSuccess ? GNN_OK : GNN_ERR_HIP;
}

// A super-batch distribution with its look-back words taken from the call's arena.
gnn_status dist_launch(DistArgs a, const Workspace &w, hipStream_t s) {
    a.lb = w.take_lb(a.ntiles, a.G);
    if (a.lb.words == nullptr) return GNN_ERR_INTERNAL;
    return launch_dist(a, s) == hipSuccess ? GNN_OK : GNN_ERR_HIP;
}

// Union bound of level l of a super-batch (l < K: hop l's frontier; l = K: the last node set):
// min(N, G * per-sub-batch bound).
int64_t union_cap(const gnn_caps &mc, int l, int G, int64_t N) {
    const int64_t f = l < mc.num_hops ? mc.frontier[l] : mc.nodes[mc.num_hops - 1];
    const int64_t u = static_cast<int64_t>(G) * f;
    return u < N ? u : N;
}

int64_t tiles_for(int64_t n) {
    const int64_t t = (n + kClassifyTile - 1) / kClassifyTile;
    return t < 1 ? 1 : t;
}

int64_t dist_tiles(int64_t n) {
    const int64_t t = (n + kDistTile - 1) / kDistTile;
    return t < 1 ? 1 : t;
}

int64_t bitmap_tiles(int64_t words) {
    const int64_t t = (words + kBitmapTile - 1) / kBitmapTile;
    return t < 1 ? 1 : t;
}

// How a super-batch relabels its sub-batches.
//  kSuperFull:    every sub-batch has a bitmap over all N node ids (three passes over G + 1
//                 bitmaps of N/32 words per hop: clear, popcount, emit).
//  kSuperCompact: the union of the sub-batches' node sets is relabelled first (one N-bit bitmap,
//                 accumulated over the hops), and each sub-batch relabels positions in it (bitmaps
//                 of |U_{l+1}|/32 words); extra work: marking and ranking the union block's ids.
enum SuperMode { kSuperNone = 0, kSuperFull = 1, kSuperCompact = 2 };

int64_t max_union_edges(const gnn_caps &mc, int64_t N, int G) {
    int64_t e = 0;
    for (int l = 0; l < mc.num_hops; ++l) {
        const int64_t x = union_cap(mc, l, G, N) * mc.fanouts[l];
        e = x > e ? x : e;
    }
    return e;
}

// Default mode: compact once the full-range bitmap passes (3 (G + 1) N/32 words a hop) outweigh
// the union block (its ids are marked and ranked once more); the options can force either.
SuperMode super_mode(const gnn_caps &mc, int64_t N, int G, uint32_t flags) {
    if (G <= 1) return kSuperNone;
    if (flags & GNN_SUPERBATCH_FULL) return kSuperFull;
    if (flags & GNN_SUPERBATCH_COMPACT) return kSuperCompact;
    const int64_t W = (N + 31) / 32;
    return 3 * static_cast<int64_t>(G + 1) * W >= max_union_edges(mc, N, G) ? kSuperCompact : kSuperFull;
}

// Narrowest rows (floats) that a super-batch gathers through the union of its node sets.
constexpr int64_t kUnionGatherMinD = 128;

// Largest byte-map region of a super-batch's sub-batch relabels (beyond it, marks stay atomic).
constexpr int64_t kByteMapsMax = 1LL << 30;

// mc: element-wise bound of every sub-batch's caps; G sub-batches relabelled the given way.
Workspace carve(const gnn_caps &mc, int64_t N, int G, SuperMode mode, void *ws) {
    Workspace w{};
    Carver c{static_cast<char *>(ws)};
    const int K = mc.num_hops;
    int64_t FU = 1, U_max = 1, F_max = 1, E_max = 1;
    for (int l = 0; l < K; ++l) {
        F_max = mc.frontier[l] > F_max ? mc.frontier[l] : F_max;
        E_max = mc.edges[l] > E_max ? mc.edges[l] : E_max;
        const int64_t u = G == 1 ? mc.frontier[l] : union_cap(mc, l, G, N);
        FU = u > FU ? u : FU;
    }
    const int64_t uE_max = G > 1 ? max_union_edges(mc, N, G) : 1;
    const int64_t nb_max = tiles_for(FU);
    w.mode = mode;
    w.W = (N + 31) / 32;
    w.nbw = bitmap_tiles(w.W);
    int64_t words = w.W, tiles = w.nbw;
    if (mode == kSuperFull) {
        words = (1 + static_cast<int64_t>(G)) * w.W;
        tiles = (1 + static_cast<int64_t>(G)) * w.nbw;
        U_max = FU;
    } else if (mode == kSuperCompact && K > 0) {
        U_max = union_cap(mc, K, G, N);  // the largest level
        w.Wc = (U_max + 31) / 32;
        w.nbwc = bitmap_tiles(w.Wc);
        w.P = mc.nodes[K - 1] > mc.frontier[0] ? mc.nodes[K - 1] : mc.frontier[0];
        w.Fs = F_max;
        w.Es = E_max;
        words += static_cast<int64_t>(G) * w.Wc;
        tiles += static_cast<int64_t>(G) * w.nbwc;
    }
    // Look-back chains of every single-pass scan one call launches: relabels (the seeds' union,
    // then per hop the union and the sub-batches; the standalone relabel and the union of the
    // gathered sets), one tile each per 1024 bitmap words of every bitmap, plus a ticket each.
    // And the classification of every hop: one tile per kClassifyTile frontier nodes; and a
    // super-batch's distribution of every hop: one tile per kDistTile destinations of each
    // sub-batch, plus a ticket each.
    const int64_t sub_tiles = mode == kSuperCompact ? w.nbwc : w.nbw;
    const int64_t dist_words = G > 1 ? K * (static_cast<int64_t>(G) * (dist_tiles(F_max) + 1) + 1) : 0;
    w.arena_words = (2 * K + 2) * (w.nbw + 1) + K * (static_cast<int64_t>(G) * (sub_tiles + 1) + 1) +
                    K * (nb_max + 1) + dist_words + 64;
    w.status = c.take<int32_t>(64);
    w.totals = c.take<uint32_t>(kTotalsStride * GNN_MAX_HOPS);
    w.arena = c.take<uint64_t>(w.arena_words);
    int64_t *cnt = c.take<int64_t>(32);
    w.d_U = cnt;
    w.d_uE = cnt ? cnt + 16 : nullptr;
    w.lists = c.take<int32_t>(kCats * FU);
    w.bitmaps = c.take<uint32_t>(words);
    w.rdir = c.take<uint2>(words);
    w.bsum_w = c.take<uint32_t>(tiles);
    if (mode != kSuperNone) {
        // byte maps of the sub-batch relabels: marks become plain byte stores
        const int64_t wx = mode == kSuperFull ? w.W : w.Wc;
        const int64_t nbytes = static_cast<int64_t>(G) * wx * 32;
        if (nbytes <= kByteMapsMax) w.bytemaps = reinterpret_cast<uint8_t *>(c.take<uint32_t>(nbytes / 4));
        w.U[0] = c.take<int32_t>(U_max);
        w.U[1] = mode == kSuperCompact ? c.take<int32_t>(U_max) : w.U[0];
        w.u_indptr = c.take<int32_t>(FU + 1);
        w.u_gid = c.take<int32_t>(uE_max);
    }
    if (mode == kSuperCompact) {
        w.upos = c.take<int32_t>(static_cast<int64_t>(G) * w.P);
        w.f_pos = c.take<int32_t>(static_cast<int64_t>(G) * w.Fs);
        w.e_pos = c.take<int32_t>(static_cast<int64_t>(G) * w.Es);
    }
    if (G > 1 && K > 0) {
        w.inv = c.take<int32_t>(union_cap(mc, K - 1, G, N) * G);
        w.inv_mask = c.take<uint32_t>(union_cap(mc, K - 1, G, N));
        if (mode == kSuperFull) w.uK = c.take<int32_t>(union_cap(mc, K, G, N));
    }
    w.bytes = c.off;
    return w;
}

struct Opts {
    int32_t group_max = 256;
    int32_t wave_max = 16384;   // measured best of 1024 .. 65536 on the four large workloads
    uint32_t flags = 0;
    int64_t *d_hits = nullptr;
};

gnn_status read_opts(const gnn_options *o, Opts *out) {
    Opts r;
    if (o) {
        if (o->group_max_deg) r.group_max = o->group_max_deg;
        if (o->wave_max_deg) r.wave_max = o->wave_max_deg;
        r.flags = o->flags;
        r.d_hits = o->d_hits;
    }
    if (r.group_max < 1 || r.wave_max < r.group_max) return GNN_ERR_INVALID_ARG;
    if ((r.flags & GNN_SUPERBATCH_FULL) && (r.flags & GNN_SUPERBATCH_COMPACT)) return GNN_ERR_INVALID_ARG;
    if ((r.flags & GNN_GATHER_INTERLEAVED) && (r.flags & GNN_GATHER_BATCHED)) return GNN_ERR_INVALID_ARG;
    if ((r.flags & GNN_RELABEL_SORT) && (r.flags & GNN_RELABEL_BITMAP)) return GNN_ERR_INVALID_ARG;
    *out = r;
    return GNN_OK;
}

int32_t relabel_force(const Opts &o) {
    return (o.flags & GNN_RELABEL_SORT) ? 1 : ((o.flags & GNN_RELABEL_BITMAP) ? 2 : 0);
}

gnn_status check_graph(const gnn_graph *g) {
    if (!g || g->num_nodes < 1 || g->num_nodes > kInt32Max || g->num_edges < 0) return GNN_ERR_INVALID_ARG;
    if (g->indptr_bytes != 4 && g->indptr_bytes != 8) return GNN_ERR_INVALID_ARG;
    if (g->indptr_bytes == 4 && g->num_edges > kInt32Max) return GNN_ERR_INVALID_ARG;
    if (!g->indptr || (g->num_edges > 0 && !g->indices)) return GNN_ERR_INVALID_ARG;
    if ((g->adj_off == nullptr) != (g->adj_rows == nullptr)) return GNN_ERR_INVALID_ARG;
    return GNN_OK;
}

gnn_status check_fanouts(const int32_t *fanouts, int32_t K) {
    if (!fanouts || K < 1 || K > GNN_MAX_HOPS) return GNN_ERR_INVALID_ARG;
    for (int l = 0; l < K; ++l)
        if (fanouts[l] < 1) return GNN_ERR_INVALID_ARG;
    for (int l = 0; l < K; ++l)
        if (fanouts[l] > kMaxFanout) return GNN_ERR_UNSUPPORTED;
    return GNN_OK;
}

// Caps must chain (frontier[0] = n_seeds, frontier[l] = nodes[l-1]), carry the call's fanouts,
// fit int32, and every array a non-empty cap refers to must exist.
gnn_status check_blocks(const gnn_blocks *b, int64_t n_seeds, const int32_t *fanouts, int32_t K) {
    if (!b || !b->counts) return GNN_ERR_INVALID_ARG;
    const gnn_caps &c = b->caps;
    if (c.num_hops != K || c.n_seeds != n_seeds || c.frontier[0] != n_seeds) return GNN_ERR_INVALID_ARG;
    for (int l = 0; l < K; ++l) {
        if (c.fanouts[l] != fanouts[l]) return GNN_ERR_INVALID_ARG;
        if (c.frontier[l] < 0 || c.edges[l] < 0 || c.nodes[l] < 0) return GNN_ERR_INVALID_ARG;
        if (c.frontier[l] > kInt32Max || c.edges[l] > kInt32Max || c.nodes[l] > kInt32Max)
            return GNN_ERR_UNSUPPORTED;
        if (l > 0 && c.frontier[l] != c.nodes[l - 1]) return GNN_ERR_INVALID_ARG;
        const gnn_block &h = b->hop[l];
        if (!h.indptr) return GNN_ERR_INVALID_ARG;
        if (c.edges[l] > 0 && (!h.gid || !h.lid)) return GNN_ERR_INVALID_ARG;
        if (c.frontier[l] > 0 && !h.dst_lid) return GNN_ERR_INVALID_ARG;
        if (c.nodes[l] > 0 && !h.nodes) return GNN_ERR_INVALID_ARG;
    }
    return GNN_OK;
}

HopArgs hop_args(const gnn_graph &g, int l, const int32_t *front, const int64_t *d_F,
                 int64_t F_cap, int32_t k, uint64_t hop_seed, int32_t *blk_indptr,
                 int32_t *blk_gid, int64_t E_cap, int64_t *d_E, const Workspace &w,
                 const Opts &o) {
    HopArgs h{};
    h.indptr = g.indptr;
    h.indices = g.indices;
    h.adj_off = g.adj_off;
    h.adj_rows = g.adj_rows;
    h.num_nodes = g.num_nodes;
    h.front = front;
    h.d_F = d_F;
    h.F_cap = F_cap;
    h.ib = g.indptr_bytes;
    h.k = k;
    h.hop_seed = hop_seed;
    h.group_max = o.group_max;
    h.wave_max = o.wave_max;
    h.exact_rank = (o.flags & GNN_SAMPLE_EXACT_RANK) ? 1 : 0;
    h.blk_indptr = blk_indptr;
    h.blk_gid = blk_gid;
    h.E_cap = E_cap;
    h.d_E = d_E;
    h.lists = w.lists;
    h.totals = w.totals + kTotalsStride * l;
    h.status = w.status;
    h.nb = static_cast<int32_t>(tiles_for(F_cap));
    return h;
}

// Relabel over all node ids into bitmaps first .. first + nbm - 1 of N bits.
RelabelArgs relabel_args(const gnn_graph &g, const Workspace &w, int first = 0, int nbm = 1) {
    RelabelArgs r{};
    r.nbm = nbm;
    r.id_bound = g.num_nodes;
    r.bitmap = w.bitmaps + first * w.W;
    r.rdir = w.rdir + first * w.W;
    r.bsum = w.bsum_w + first * w.nbw;
    r.W = w.W;
    r.nbw = static_cast<int32_t>(w.nbw);
    r.status = w.status;
    r.bitmap_cleared = 1;
    return r;
}

// Relabel of G sub-batches over positions in a sorted union list (the G compact bitmaps).
RelabelArgs compact_relabel_args(const Workspace &w, int G, const int32_t *ulist,
                                 const int64_t *d_n, int64_t cap) {
    RelabelArgs r{};
    r.nbm = G;
    r.id_bound = cap;
    r.d_bound = d_n;
    r.id_map = ulist;
    r.bitmap = w.bitmaps + w.W;
    r.rdir = w.rdir + w.W;
    r.bsum = w.bsum_w + w.nbw;
    r.W = w.Wc;
    r.nbw = static_cast<int32_t>(w.nbwc);
    r.status = w.status;
    r.bitmap_cleared = 1;
    return r;
}

// One hop of a super-batch with full-range sub-batch bitmaps: the union U of the G frontiers
// (bitmap 0) is relabelled, classified and sampled once; each sub-batch takes its rows from the
// union block (union rank by bitmap 0) and is relabelled into its own bitmap over all node ids.
template <typename FrontFn, typename CountFn, typename CapFn>
gnn_status run_super_full_hop(const gnn_graph &g, FrontFn front, CountFn d_F, CapFn F_cap, int G,
                              int32_t k, uint64_t hs, int l, const gnn_caps &mc,
                              gnn_blocks *const *outs, const Workspace &w, const Opts &o,
                              hipStream_t s, hipEvent_t *sev, bool last) {
    const int64_t Ucap = union_cap(mc, l, G, g.num_nodes);
    const int64_t uEcap = Ucap * k;
    RelabelArgs ru = relabel_args(g, w);
    ru.nlist = G;
    for (int gi = 0; gi < G; ++gi) ru.list[gi] = IdList{front(gi, l), d_F(gi, l), F_cap(gi, l), nullptr, 0, 0};
    ru.out[0] = BitmapOut{w.U[0], Ucap, w.d_U, nullptr};
    ru.bitmap_read_after = 1;   // the distribution ranks destinations in U by this bitmap
    GNN_TRY(relabel_launch(ru, w, s));
    HopArgs h = hop_args(g, l, w.U[0], w.d_U, Ucap, k, hs, w.u_indptr, w.u_gid, uEcap, w.d_uE, w, o);
    if (last) h.inv_mask = w.inv_mask;   // the union positions table's mask, for the distribution
    if (w.bytemaps) {
        // the sub-batch byte maps are zeroed before their relabel; the bitmaps are rewritten
        // whole from them, except that the seeds' duplicate check needs clean bitmaps at hop 0
        h.clear_ptr = reinterpret_cast<uint32_t *>(w.bytemaps);
        h.clear_n = static_cast<int64_t>(G) * w.W * 8;
        if (l == 0) GNN_TRY_HIP(launch_fill_u32(w.bitmaps + w.W, static_cast<int64_t>(G) * w.W, 0u, s));
    } else {
        h.clear_ptr = w.bitmaps + w.W;  // the sub-batch bitmaps, zeroed before their relabel
        h.clear_n = static_cast<int64_t>(G) * w.W;
    }
    GNN_TRY(classify_launch(h, w, s));
    if (sev) GNN_TRY_HIP(hipEventRecord(sev[2 * l], s));
    GNN_TRY_HIP(launch_sample(h, s));
    if (sev) GNN_TRY_HIP(hipEventRecord(sev[2 * l + 1], s));
    DistArgs da{};
    da.G = G;
    int32_t tiles = 0;
    for (int gi = 0; gi < G; ++gi) {
        gnn_blocks &out = *outs[gi];
        const int32_t nt = static_cast<int32_t>(dist_tiles(F_cap(gi, l)));
        da.sub[gi] = DistSub{front(gi, l), d_F(gi, l), F_cap(gi, l), nullptr, nullptr,
                             out.hop[l].indptr, out.hop[l].gid, nullptr, out.caps.edges[l],
                             out.counts + 2 * l, tiles, nt};
        tiles += nt;
    }
    da.ntiles = tiles;
    da.rdir0 = w.rdir;
    da.id_bound = g.num_nodes;
    da.u_indptr = w.u_indptr;
    da.u_gid = w.u_gid;
    da.uE_cap = uEcap;
    da.d_U = w.d_U;
    da.U_cap = Ucap;
    da.status = w.status;
    if (last) {
        da.inv = w.inv;
        da.inv_mask = w.inv_mask;
    }
    GNN_TRY(dist_launch(da, w, s));
    // Per-sub-batch relabel into bitmaps 1..G; the union bitmap is zeroed for the next hop.
    RelabelArgs rs = relabel_args(g, w, 1, G);
    rs.bytes = w.bytemaps;
    rs.nlist = 2 * G;
    for (int gi = 0; gi < G; ++gi) {
        gnn_blocks &out = *outs[gi];
        rs.list[2 * gi] = IdList{front(gi, l), d_F(gi, l), F_cap(gi, l), out.hop[l].dst_lid, gi,
                                 l == 0 ? 1 : 0};
        rs.list[2 * gi + 1] = IdList{out.hop[l].gid, out.counts + 2 * l, out.caps.edges[l],
                                     out.hop[l].lid, gi, 0};
        rs.out[gi] = BitmapOut{out.hop[l].nodes, out.caps.nodes[l], out.counts + 2 * l + 1, nullptr};
    }
    rs.clear_ptr = w.bitmaps;
    rs.clear_n = w.W;
    GNN_TRY(relabel_launch(rs, w, s));
    return GNN_OK;
}

// Sampling and relabel of every hop of G sub-batches (G = 1: one batch); no host synchronisation.
// seeds_g[g] / n_seeds_g[g] are the sub-batches' seeds, outs[g] their blocks.
//
// G > 1, compact relabel: the node-id bitmap accumulates the union U_l of the sub-batch frontiers
// over the hops (U_0 = the seeds, U_{l+1} = U_l + the ids sampled from U_l); U_l is sampled once
// per hop and every sub-batch relabels in positions of U_{l+1}.  Full relabel: run_super_full_hop.
gnn_status run_sample(const gnn_graph &g, const int32_t *const *seeds_g, const int64_t *n_seeds_g,
                      int G, const int32_t *fanouts, int32_t K, uint64_t seed64,
                      gnn_blocks *const *outs, const Workspace &w, const Opts &o, hipStream_t s,
                      hipEvent_t *sev = nullptr) {
    gnn_caps mc = outs[0]->caps;
    for (int gi = 1; gi < G; ++gi) {
        for (int l = 0; l < K; ++l) {
            const gnn_caps &c = outs[gi]->caps;
            mc.frontier[l] = c.frontier[l] > mc.frontier[l] ? c.frontier[l] : mc.frontier[l];
            mc.edges[l] = c.edges[l] > mc.edges[l] ? c.edges[l] : mc.edges[l];
            mc.nodes[l] = c.nodes[l] > mc.nodes[l] ? c.nodes[l] : mc.nodes[l];
        }
    }
    auto front = [&](int gi, int l) { return l == 0 ? seeds_g[gi] : outs[gi]->hop[l - 1].nodes; };
    auto d_F = [&](int gi, int l) -> const int64_t * {
        return l == 0 ? nullptr : outs[gi]->counts + 2 * (l - 1) + 1;
    };
    auto F_cap = [&](int gi, int l) { return l == 0 ? n_seeds_g[gi] : outs[gi]->caps.frontier[l]; };
    const bool compact = w.mode == kSuperCompact;
    if (G > 1) GNN_TRY_HIP(launch_fill_u32(w.bitmaps, w.W, 0u, s));
    // U_0 as the concatenation of the seeds where it fits the level's bound (G times the
    // per-sub-batch seed bound at most N), else their sorted union.
    const bool concat0 = compact && static_cast<int64_t>(G) * mc.frontier[0] <= g.num_nodes;
    if (concat0) {
        SeedConcatArgs sc{};
        sc.G = G;
        sc.off[0] = 0;
        for (int gi = 0; gi < G; ++gi) {
            sc.seeds[gi] = seeds_g[gi];
            sc.off[gi + 1] = sc.off[gi] + n_seeds_g[gi];
        }
        sc.U0 = w.U[0];
        sc.d_U0 = w.d_U;
        sc.upos = w.upos;
        sc.P = w.P;
        sc.bitmap = w.bitmaps;
        sc.num_nodes = g.num_nodes;
        GNN_TRY_HIP(launch_seed_concat(sc, s));
    } else if (compact) {
        // U_0: the union of the seeds, and each seed's position in it.
        RelabelArgs r0 = relabel_args(g, w);
        r0.nlist = G;
        for (int gi = 0; gi < G; ++gi)
            r0.list[gi] = IdList{seeds_g[gi], nullptr, n_seeds_g[gi], w.upos + gi * w.P, 0, 0};
        r0.out[0] = BitmapOut{w.U[0], union_cap(mc, 0, G, g.num_nodes), w.d_U, nullptr};
        r0.sort_sets_bits = 1;   // U_0 starts the union that the node-id bitmap accumulates
        GNN_TRY(relabel_launch(r0, w, s));
    }
    for (int l = 0; l < K; ++l) {
        const uint64_t hs = mix64(seed64 + kGamma * static_cast<uint64_t>(l + 1));
        if (G == 1) {
            gnn_blocks &out = *outs[0];
            const gnn_caps &c = out.caps;
            HopArgs h = hop_args(g, l, front(0, l), d_F(0, l), F_cap(0, l), fanouts[l], hs,
                                 out.hop[l].indptr, out.hop[l].gid, c.edges[l], out.counts + 2 * l,
                                 w, o);
            RelabelArgs r = relabel_args(g, w);
            r.nlist = 2;
            r.list[0] = IdList{front(0, l), d_F(0, l), F_cap(0, l), out.hop[l].dst_lid, 0, l == 0 ? 1 : 0};
            r.list[1] = IdList{out.hop[l].gid, out.counts + 2 * l, c.edges[l], out.hop[l].lid, 0, 0};
            r.out[0] = BitmapOut{out.hop[l].nodes, c.nodes[l], out.counts + 2 * l + 1, nullptr};
            if (!relabel_sorts(r)) {   // the bitmap path marks a cleared bitmap
                h.clear_ptr = w.bitmaps;
                h.clear_n = w.W;
            }
            GNN_TRY(classify_launch(h, w, s));
            if (sev) GNN_TRY_HIP(hipEventRecord(sev[2 * l], s));
            GNN_TRY_HIP(launch_sample(h, s));
            if (sev) GNN_TRY_HIP(hipEventRecord(sev[2 * l + 1], s));
            GNN_TRY(relabel_launch(r, w, s));
            continue;
        }
        if (!compact) {
            const gnn_status st = run_super_full_hop(g, front, d_F, F_cap, G, fanouts[l], hs, l, mc,
                                                     outs, w, o, s, sev, l == K - 1);
            if (st != GNN_OK) return st;
            continue;
        }
        // Super-batch hop l: sample U_l once.
        const int64_t Ucap = union_cap(mc, l, G, g.num_nodes);
        const int64_t U1cap = union_cap(mc, l + 1, G, g.num_nodes);
        const int64_t uEcap = Ucap * fanouts[l];
        int32_t *Ul = w.U[l & 1];
        int32_t *Ul1 = w.U[(l + 1) & 1];
        HopArgs h = hop_args(g, l, Ul, w.d_U + l, Ucap, fanouts[l], hs, w.u_indptr, w.u_gid, uEcap,
                             w.d_uE + l, w, o);
        if (l == K - 1) h.inv_mask = w.inv_mask;   // the union positions table's mask
        h.mark = w.bitmaps;   // the sampled ids join U_l in the node-id bitmap
        // the sub-batch bitmaps (and byte maps) that this hop's distribution marks, zeroed by the
        // sampler up to |U_l| + |uE_l| >= |U_{l+1}| ids
        h.zero_words = w.bitmaps + w.W;
        h.zero_bytes = reinterpret_cast<uint32_t *>(w.bytemaps);
        h.zero_stride = w.Wc;
        h.zero_g = G;
        h.zero_da = w.d_U + l;
        h.zero_db = w.d_uE + l;
        GNN_TRY(classify_launch(h, w, s));
        if (sev) GNN_TRY_HIP(hipEventRecord(sev[2 * l], s));
        GNN_TRY_HIP(launch_sample(h, s));
        if (sev) GNN_TRY_HIP(hipEventRecord(sev[2 * l + 1], s));
        // U_{l+1} = U_l + the sampled ids, whose bits the sampler has set in the accumulated
        // node-id bitmap: emit its ids (and word prefixes, for ranks in U_{l+1}).
        RelabelArgs ru = relabel_args(g, w);
        ru.nlist = 0;
        ru.out[0] = BitmapOut{Ul1, U1cap, w.d_U + l + 1, nullptr};
        ru.bitmap_read_after = 1;   // positions in U_{l+1} are ranks in this bitmap
        GNN_TRY(relabel_launch(ru, w, s));
        // Each sub-batch's block from the union block, with U_{l+1} positions of its ids.
        DistArgs da{};
        da.G = G;
        int32_t tiles = 0;
        for (int gi = 0; gi < G; ++gi) {
            gnn_blocks &out = *outs[gi];
            const int32_t nt = static_cast<int32_t>(dist_tiles(F_cap(gi, l)));
            da.sub[gi] = DistSub{front(gi, l), d_F(gi, l), F_cap(gi, l), w.upos + gi * w.P,
                                 w.f_pos + gi * w.Fs, out.hop[l].indptr, out.hop[l].gid,
                                 w.e_pos + gi * w.Es, out.caps.edges[l], out.counts + 2 * l,
                                 tiles, nt};
            tiles += nt;
        }
        da.ntiles = tiles;
        da.u_indptr = w.u_indptr;
        da.u_gid = w.u_gid;
        da.Ul = Ul;
        da.rdir1 = w.rdir;
        da.id_bound = g.num_nodes;
        da.uE_cap = uEcap;
        da.d_U = w.d_U + l;
        da.U_cap = Ucap;
        // the sub-batch relabel's marks (positions in U_{l+1}), made by the distribution
        da.mark_words = w.bitmaps + w.W;
        da.mark_bytes = w.bytemaps;
        da.mark_stride = w.Wc;
        da.mark_dup = l == 0 ? 1 : 0;
        da.d_U1 = w.d_U + l + 1;
        da.U1_cap = U1cap;
        da.status = w.status;
        if (l == K - 1) {
            da.inv = w.inv;
            da.inv_mask = w.inv_mask;
        }
        GNN_TRY(dist_launch(da, w, s));
        // Per-sub-batch relabel in U_{l+1} positions; the positions of V_l become the next hop's.
        RelabelArgs rs = compact_relabel_args(w, G, Ul1, w.d_U + l + 1, U1cap);
        rs.bytes = w.bytemaps;
        rs.nlist = 2 * G;
        for (int gi = 0; gi < G; ++gi) {
            gnn_blocks &out = *outs[gi];
            // marked by the distribution: ranked only
            rs.list[2 * gi] = IdList{w.f_pos + gi * w.Fs, d_F(gi, l), F_cap(gi, l),
                                     out.hop[l].dst_lid, gi, 2};
            rs.list[2 * gi + 1] = IdList{w.e_pos + gi * w.Es, out.counts + 2 * l, out.caps.edges[l],
                                         out.hop[l].lid, gi, 2};
            rs.out[gi] = BitmapOut{out.hop[l].nodes, out.caps.nodes[l], out.counts + 2 * l + 1,
                                   w.upos + gi * w.P};
        }
        GNN_TRY(relabel_launch(rs, w, s));
    }
    return GNN_OK;
}

// The union gather (table in HBM, G > 1): whether the rows allow it (16-byte aligned), ...
bool union_gather_fits(const gnn_feature_store *fs, const gnn_minibatch_out *outs, int G,
                       const Workspace &w) {
    bool ok = (w.mode == kSuperCompact || w.uK != nullptr) && fs->ld % 4 == 0 &&
              outs[0].ld_h % 4 == 0 && reinterpret_cast<uintptr_t>(fs->table) % 16 == 0;
    for (int gi = 0; gi < G; ++gi) ok = ok && reinterpret_cast<uintptr_t>(outs[gi].x) % 16 == 0;
    return ok;
}

// ... and U_K, the union of the sub-batches' V_K (relabel work, timed with stage 1): the compact
// relabel has built it as its last union level; with full-range bitmaps the node-id bitmap, cleared
// by the last hop's sub-batch relabel, takes the sub-batches' V_K.  A union row's position in
// sub-batch g is its rank in g's relabel bitmap (by union position, or by node id in full mode).
const int32_t *union_prepare(const gnn_graph &g, const gnn_minibatch_out *outs, int G, int K,
                             const gnn_caps &mc, const Workspace &w, hipStream_t s,
                             gnn_status *st) {
    *st = GNN_OK;
    if (w.mode == kSuperCompact) return w.U[K & 1];
    RelabelArgs ru = relabel_args(g, w);
    ru.nlist = G;
    for (int gi = 0; gi < G; ++gi) {
        const gnn_blocks &b = outs[gi].blocks;
        ru.list[gi] = IdList{b.hop[K - 1].nodes, b.counts + 2 * (K - 1) + 1, b.caps.nodes[K - 1],
                             nullptr, 0, 0};
    }
    ru.out[0] = BitmapOut{w.uK, union_cap(mc, K, G, g.num_nodes), w.d_U + K, nullptr};
    *st = relabel_launch(ru, w, s);
    return w.uK;
}

// Fault injection for tests of the error paths: GNN_FAULT (read once per process) lists kinds,
// comma-separated: "alloc" fails every set-up allocation before it is made, "launch" fails every
// hot-path call after its argument checks, before anything is enqueued; both return GNN_ERR_HIP.
enum : int { kFaultAlloc = 1, kFaultLaunch = 2 };
int fault_mask() {
    static const int mask = [] {
        const char *e = getenv("GNN_FAULT");
        int m = 0;
        if (e != nullptr) {
            if (strstr(e, "alloc")) m |= kFaultAlloc;
            if (strstr(e, "launch")) m |= kFaultLaunch;
        }
        return m;
    }();
    return mask;
}
bool fault(int kind) { return (fault_mask() & kind) != 0; }

gnn_status check_unique_relabel(const int32_t *keep, int64_t n_keep, const int32_t *add,
                                int64_t n_add, int64_t id_bound, const int32_t *uniq,
                                int64_t cap_uniq, const int64_t *d_n_uniq, const int32_t *add_lid,
                                const int32_t *keep_lid) {
    if (n_keep < 0 || n_add < 0 || cap_uniq < 0 || id_bound < 1 || id_bound > kInt32Max + 1)
        return GNN_ERR_INVALID_ARG;
    if ((n_keep > 0 && (!keep || !keep_lid)) || (n_add > 0 && (!add || !add_lid)))
        return GNN_ERR_INVALID_ARG;
    if (!d_n_uniq || (cap_uniq > 0 && !uniq)) return GNN_ERR_INVALID_ARG;
    if (n_keep > kInt32Max || n_add > kInt32Max) return GNN_ERR_UNSUPPORTED;
    return GNN_OK;
}

// The relabel of two lists in a carved workspace; device errors go to `status` (cleared first).
gnn_status unique_relabel_in(const Workspace &w, int32_t *status, const int32_t *keep,
                             int64_t n_keep, const int32_t *add, const int64_t *d_n_add,
                             int64_t n_add, int64_t id_bound, int32_t *uniq, int64_t cap_uniq,
                             int64_t *d_n_uniq, int32_t *add_lid, int32_t *keep_lid,
                             hipStream_t s) {
    GNN_TRY_HIP(launch_fill_u32(reinterpret_cast<uint32_t *>(w.arena), 2 * w.arena_words, 0u, s));
    if (status) GNN_TRY_HIP(launch_fill_i32(status, 1, 0, s));
    RelabelArgs r{};
    r.nlist = 2;
    r.list[0] = IdList{keep, nullptr, n_keep, keep_lid, 0, 0};
    r.list[1] = IdList{add, d_n_add, n_add, add_lid, 0, 0};
    r.nbm = 1;
    r.out[0] = BitmapOut{uniq, cap_uniq, d_n_uniq, nullptr};
    r.id_bound = id_bound;
    r.bitmap = w.bitmaps;
    r.rdir = w.rdir;
    r.bsum = w.bsum_w;
    r.W = w.W;
    r.nbw = static_cast<int32_t>(w.nbw);
    r.status = status;
    r.bitmap_cleared = 0;
    GNN_TRY(relabel_launch(r, w, s));
    return GNN_OK;
}

// Scratch of gnn_unique_relabel_noalloc: one array per GPU for the life of the process, shared
// by every call on that GPU (calls that overlap on one GPU race).  Host code never passes the
// array's name to a kernel: its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and kept here.
static __device__ __align__(256) unsigned char scratch[GNN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of stream s (the current device for the null stream).
gnn_status scratch_address(hipStream_t s, void **out) {
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return GNN_ERR_HIP;
    dev = cur;
    if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return GNN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GNN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GNN_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return GNN_ERR_HIP;
        if (e != hipSuccess || p == nullptr) return GNN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GNN_OK;
}

gnn_status finish(const Opts &o, const Workspace &w, hipStream_t s) {
    if (!(o.flags & GNN_SYNC)) return GNN_OK;
    int32_t st = 0;
    GNN_TRY_HIP(hipMemcpyAsync(&st, w.status, sizeof(st), hipMemcpyDeviceToHost, s));
    GNN_TRY_HIP(hipStreamSynchronize(s));
    return st;
}

}  // namespace

extern "C" {

const char *gnn_status_string(gnn_status s) {
    switch (s) {
        case GNN_OK: return "ok";
        case GNN_ERR_INVALID_ARG: return "invalid argument";
        case GNN_ERR_CAPACITY: return "buffer too small";
        case GNN_ERR_OUT_OF_RANGE: return "node id out of range";
        case GNN_ERR_HIP: return "HIP runtime error";
        case GNN_ERR_UNSUPPORTED: return "unsupported size or option";
        case GNN_ERR_INTERNAL: return "internal invariant failed";
        default: return "unknown status";
    }
}

uint64_t gnn_batch_seed(uint64_t rng_seed, uint64_t b) { return mix64(rng_seed + kGamma * (b + 1)); }

gnn_status gnn_capacity(int64_t n_seeds, const int32_t *fanouts, int32_t num_hops,
                        int64_t num_nodes, gnn_caps *out) {
    if (!out || n_seeds < 0 || num_nodes < 1) return GNN_ERR_INVALID_ARG;
    gnn_status st = check_fanouts(fanouts, num_hops);
    if (st != GNN_OK) return st;
    gnn_caps c;
    memset(&c, 0, sizeof(c));
    c.num_hops = num_hops;
    c.n_seeds = n_seeds;
    int64_t f = n_seeds;
    for (int l = 0; l < num_hops; ++l) {
        c.fanouts[l] = fanouts[l];
        c.frontier[l] = f;
        const int64_t e = f * fanouts[l];
        if (f > kInt32Max || e > kInt32Max) return GNN_ERR_UNSUPPORTED;
        c.edges[l] = e;
        c.nodes[l] = f + e < num_nodes ? f + e : num_nodes;
        f = c.nodes[l];
    }
    *out = c;
    return GNN_OK;
}

gnn_status gnn_workspace_size(const gnn_caps *caps, int64_t num_nodes, int32_t group,
                              size_t *out_bytes) {
    if (!caps || !out_bytes || num_nodes < 1 || group < 1) return GNN_ERR_INVALID_ARG;
    if (group > GNN_MAX_GROUP) return GNN_ERR_UNSUPPORTED;
    if (caps->num_hops < 1 || caps->num_hops > GNN_MAX_HOPS) return GNN_ERR_INVALID_ARG;
    // any relabel mode the options may pick
    size_t b = carve(*caps, num_nodes, group, group > 1 ? kSuperFull : kSuperNone, nullptr).bytes;
    if (group > 1) {
        const size_t bc = carve(*caps, num_nodes, group, kSuperCompact, nullptr).bytes;
        b = bc > b ? bc : b;
    }
    *out_bytes = b;
    return GNN_OK;
}

gnn_status gnn_sample_khop(const gnn_graph *g, const int32_t *seeds, int64_t n_seeds,
                           const int32_t *fanouts, int32_t num_hops, uint64_t seed64,
                           gnn_blocks *out, void *ws, size_t ws_bytes,
                           const gnn_options *opt, gnn_stream stream) {
    gnn_status st = check_graph(g);
    if (st == GNN_OK) st = check_fanouts(fanouts, num_hops);
    if (st != GNN_OK) return st;
    if (n_seeds < 0 || (n_seeds > 0 && !seeds)) return GNN_ERR_INVALID_ARG;
    if ((st = check_blocks(out, n_seeds, fanouts, num_hops)) != GNN_OK) return st;
    Opts o;
    if ((st = read_opts(opt, &o)) != GNN_OK) return st;
    if (!ws) return GNN_ERR_INVALID_ARG;
    const Workspace need = carve(out->caps, g->num_nodes, 1, kSuperNone, nullptr);
    if (ws_bytes < need.bytes) return GNN_ERR_CAPACITY;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    Workspace w = carve(out->caps, g->num_nodes, 1, kSuperNone, ws);
    w.relabel_force = relabel_force(o);
    hipStream_t s = static_cast<hipStream_t>(stream);
    GNN_TRY_HIP(launch_fill_u32(reinterpret_cast<uint32_t *>(w.status), w.cleared_bytes() / 4, 0u, s));
    const int32_t *sp[1] = {seeds};
    const int64_t ns[1] = {n_seeds};
    gnn_blocks *ob[1] = {out};
    st = run_sample(*g, sp, ns, 1, fanouts, num_hops, seed64, ob, w, o, s);
    if (st != GNN_OK) return st;
    return finish(o, w, s);
}

gnn_status gnn_relabel_workspace_size(int64_t id_bound, size_t *out_bytes) {
    if (!out_bytes || id_bound < 1 || id_bound > kInt32Max + 1) return GNN_ERR_INVALID_ARG;
    gnn_caps none{};
    *out_bytes = carve(none, id_bound, 1, kSuperNone, nullptr).bytes;
    return GNN_OK;
}

gnn_status gnn_unique_relabel(const int32_t *keep, int64_t n_keep, const int32_t *add,
                              const int64_t *d_n_add, int64_t n_add, int64_t id_bound,
                              int32_t *uniq, int64_t cap_uniq, int64_t *d_n_uniq,
                              int32_t *add_lid, int32_t *keep_lid, void *ws, size_t ws_bytes,
                              gnn_stream stream) {
    gnn_status st = check_unique_relabel(keep, n_keep, add, n_add, id_bound, uniq, cap_uniq,
                                         d_n_uniq, add_lid, keep_lid);
    if (st != GNN_OK) return st;
    if (!ws) return GNN_ERR_INVALID_ARG;
    gnn_caps none{};
    const Workspace need = carve(none, id_bound, 1, kSuperNone, nullptr);
    if (ws_bytes < need.bytes) return GNN_ERR_CAPACITY;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    const Workspace w = carve(none, id_bound, 1, kSuperNone, ws);
    return unique_relabel_in(w, w.status, keep, n_keep, add, d_n_add, n_add, id_bound, uniq,
                             cap_uniq, d_n_uniq, add_lid, keep_lid, static_cast<hipStream_t>(stream));
}

gnn_status gnn_unique_relabel_noalloc(const int32_t *keep, int64_t n_keep, const int32_t *add,
                                      const int64_t *d_n_add, int64_t n_add, int64_t id_bound,
                                      int32_t *uniq, int64_t cap_uniq, int64_t *d_n_uniq,
                                      int32_t *add_lid, int32_t *keep_lid, int32_t *d_status,
                                      gnn_stream stream) {
    gnn_status st = check_unique_relabel(keep, n_keep, add, n_add, id_bound, uniq, cap_uniq,
                                         d_n_uniq, add_lid, keep_lid);
    if (st != GNN_OK) return st;
    if (id_bound > GNN_NOALLOC_MAX_IDS) return GNN_ERR_UNSUPPORTED;
    gnn_caps none{};
    const Workspace need = carve(none, id_bound, 1, kSuperNone, nullptr);
    if (need.bytes > sizeof(scratch)) return GNN_ERR_INTERNAL;   // the bound above keeps it in
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *base = nullptr;
    if ((st = scratch_address(s, &base)) != GNN_OK) return st;
    const Workspace w = carve(none, id_bound, 1, kSuperNone, base);
    return unique_relabel_in(w, d_status, keep, n_keep, add, d_n_add, n_add, id_bound, uniq,
                             cap_uniq, d_n_uniq, add_lid, keep_lid, s);
}

namespace {

// Scaled scores are brought back by 2^-512 (exact for normal doubles) once the weights reach
// 2^512: at a refresh, or -- when no refresh comes -- on the stream of the observing call (with
// observations from other streams in flight this may mix scales for a node, which moves the
// ranking but never a gathered row).
constexpr double kDynRescaleAt = 0x1p512;
constexpr double kDynRescaleBy = 0x1p-512;

bool dyn_frozen(const DynCache *dc) {
    return dc->p.max_refreshes > 0 && dc->refreshes >= dc->p.max_refreshes;
}

// Observation weights of the next n mini-batches of the store, w[0..n) (GARDEN Sec. IV.B, eq.
// (5) in the scaled form S(v) = w_t * Score(v, t), w_t = W * gamma^-t).  *obs.score stays NULL
// when nothing is observed (no Dynamic-Cache, or a frozen one); obs.filled is set whenever there
// is a Dynamic-Cache, whose reserved rows the gathers fill.
gnn_status dyn_observe_steps(const gnn_feature_store *fs, int n, double *w, DynObserve *obs,
                             hipStream_t s) {
    *obs = DynObserve{};
    DynCache *dc = fs->dyn;
    if (!dc) return GNN_OK;
    std::lock_guard<std::mutex> lk(dc->mu);
    obs->static_rows = static_cast<int32_t>(fs->cache_rows);
    obs->filled = dc->filled;
    dc->steps += n;
    if (dyn_frozen(dc)) return GNN_OK;
    if (dc->w_next >= kDynRescaleAt) {
        GNN_TRY_HIP(launch_dyn_rescale(dc->score, fs->num_nodes, kDynRescaleBy, s));
        dc->w_next *= kDynRescaleBy;
    }
    for (int i = 0; i < n; ++i) {
        w[i] = dc->w_next;
        dc->w_next /= dc->p.gamma;
    }
    obs->score = dc->score;
    obs->touched = dc->touched;
    return GNN_OK;
}

// A refresh (eq. (6)) on s if one is due: at least t_update mini-batches since the last one.  A
// frozen cache only makes its filled rows resident.
gnn_status dyn_refresh(const gnn_feature_store *fs, int32_t *d_status, hipStream_t s,
                       int32_t *refreshed) {
    if (refreshed) *refreshed = 0;
    DynCache *dc = fs->dyn;
    std::lock_guard<std::mutex> lk(dc->mu);
    if (dc->steps - dc->steps_at_refresh < dc->p.t_update) return GNN_OK;
    const bool frozen = dyn_frozen(dc);
    if (!frozen && dc->w_next >= kDynRescaleAt) {
        GNN_TRY_HIP(launch_dyn_rescale(dc->score, fs->num_nodes, kDynRescaleBy, s));
        dc->w_next *= kDynRescaleBy;
    }
    DynRefreshArgs a{};
    a.st = dc->state;
    a.score = dc->score;
    a.touched = dc->touched;
    a.member = dc->member;
    a.num_rows = fs->num_nodes;
    a.cand = dc->cand;
    a.key_hi = dc->key_hi;
    a.key_lo = dc->key_lo;
    a.free_rows = dc->free_rows;
    a.admit = dc->admit;
    a.row_node = dc->row_node;
    a.filled = dc->filled;
    a.k_dyn = dc->p.k_dyn;
    a.static_rows = static_cast<int32_t>(fs->cache_rows);
    a.slot = fs->slot;
    a.status = d_status;
    GNN_TRY_HIP(launch_dyn_refresh(a, frozen, s));
    dc->steps_at_refresh = dc->steps;
    if (!frozen) {
        dc->refreshes += 1;
        if (refreshed) *refreshed = 1;
    }
    return GNN_OK;
}

gnn_status dyn_auto_refresh(const gnn_feature_store *fs, int32_t *d_status, hipStream_t s) {
    if (!fs->dyn || !(fs->dyn->p.flags & GNN_DYN_AUTO)) return GNN_OK;
    return dyn_refresh(fs, d_status, s, nullptr);
}

void dyn_free(DynCache *dc) {
    if (!dc) return;
    if (dc->score) (void)hipFree(dc->score);
    if (dc->touched) (void)hipFree(dc->touched);
    if (dc->member) (void)hipFree(dc->member);
    if (dc->cand) (void)hipFree(dc->cand);
    if (dc->key_hi) (void)hipFree(dc->key_hi);
    if (dc->key_lo) (void)hipFree(dc->key_lo);
    if (dc->free_rows) (void)hipFree(dc->free_rows);
    if (dc->admit) (void)hipFree(dc->admit);
    if (dc->row_node) (void)hipFree(dc->row_node);
    if (dc->filled) (void)hipFree(dc->filled);
    if (dc->state) (void)hipFree(dc->state);
    delete dc;
}

}  // namespace

gnn_status gnn_feature_store_create(const float *table, int32_t table_on_host, int64_t num_nodes,
                                    int64_t d, int64_t ld, int64_t cache_rows,
                                    const int32_t *hot_order, gnn_feature_store **out) {
    if (!out || !table || num_nodes < 1 || num_nodes > kInt32Max || d < 1 || ld < d)
        return GNN_ERR_INVALID_ARG;
    if (cache_rows < 0 || cache_rows > num_nodes || (cache_rows > 0 && !hot_order))
        return GNN_ERR_INVALID_ARG;
    *out = nullptr;
    const float *dev_table = table;
    if (table_on_host) {
        void *p = nullptr;
        if (hipHostGetDevicePointer(&p, const_cast<float *>(table), 0) != hipSuccess || !p)
            return GNN_ERR_HIP;
        dev_table = static_cast<const float *>(p);
    }
    gnn_feature_store *fs = new (std::nothrow) gnn_feature_store{};
    if (!fs) return GNN_ERR_INVALID_ARG;
    fs->table = dev_table;
    fs->on_host = table_on_host ? 1 : 0;
    fs->num_nodes = num_nodes;
    fs->d = d;
    fs->ld = ld;
    fs->cache_rows = cache_rows;
    if (cache_rows > 0 && fault(kFaultAlloc)) {
        delete fs;
        return GNN_ERR_HIP;
    }
    if (cache_rows > 0) {
        int32_t *st_dev = nullptr;
        bool ok = hipMalloc(reinterpret_cast<void **>(&fs->cache),
                            static_cast<size_t>(cache_rows) * ld * sizeof(float)) == hipSuccess;
        ok = ok && hipMalloc(reinterpret_cast<void **>(&fs->slot),
                             static_cast<size_t>(num_nodes) * sizeof(int32_t)) == hipSuccess;
        ok = ok && hipMalloc(reinterpret_cast<void **>(&st_dev), sizeof(int32_t)) == hipSuccess;
        ok = ok && launch_fill_i32(st_dev, 1, 0, nullptr) == hipSuccess;
        ok = ok && launch_fill_i32(fs->slot, num_nodes, -1, nullptr) == hipSuccess;
        ok = ok && launch_cache_fill(dev_table, ld, d, num_nodes, hot_order, cache_rows,
                                     fs->cache, fs->slot, st_dev, nullptr) == hipSuccess;
        int32_t st = 0;
        ok = ok && hipMemcpy(&st, st_dev, sizeof(st), hipMemcpyDeviceToHost) == hipSuccess;
        ok = ok && hipDeviceSynchronize() == hipSuccess;
        if (st_dev) (void)hipFree(st_dev);
        if (!ok || st != 0) {
            gnn_feature_store_destroy(fs);
            return ok ? st : GNN_ERR_HIP;
        }
    }
    *out = fs;
    return GNN_OK;
}

gnn_status gnn_host_mapped_pointer(const void *host, const void **out_device) {
    if (!host || !out_device) return GNN_ERR_INVALID_ARG;
    *out_device = nullptr;
    void *p = nullptr;
    if (hipHostGetDevicePointer(&p, const_cast<void *>(host), 0) != hipSuccess || !p) {
        (void)hipGetLastError();
        return GNN_ERR_HIP;
    }
    *out_device = p;
    return GNN_OK;
}

gnn_status gnn_adjacency_cache_create(const gnn_graph *g, const int32_t *hot_order, int64_t n_hot,
                                      int64_t max_entries, gnn_adjacency_cache **out,
                                      int64_t *out_rows, int64_t *out_entries) {
    if (!out) return GNN_ERR_INVALID_ARG;
    *out = nullptr;
    const gnn_status gs = check_graph(g);
    if (gs != GNN_OK) return gs;
    if (n_hot < 0 || n_hot > g->num_nodes || max_entries < 0 || (n_hot > 0 && !hot_order))
        return GNN_ERR_INVALID_ARG;
    if (fault(kFaultAlloc)) return GNN_ERR_HIP;
    // the hot ids and their degrees, on the host: the longest prefix of the order that fits
    std::vector<int32_t> hot(static_cast<size_t>(n_hot));
    std::vector<int64_t> deg(static_cast<size_t>(n_hot));
    if (n_hot > 0) {
        if (hipMemcpy(hot.data(), hot_order, n_hot * sizeof(int32_t), hipMemcpyDeviceToHost) !=
            hipSuccess)
            return GNN_ERR_HIP;
        for (int32_t v : hot)
            if (v < 0 || v >= g->num_nodes) return GNN_ERR_INVALID_ARG;
        int64_t *d_deg = nullptr;
        bool ok = hipMalloc(reinterpret_cast<void **>(&d_deg), n_hot * sizeof(int64_t)) == hipSuccess;
        ok = ok && launch_adj_degrees(g->indptr, g->indptr_bytes, hot_order, n_hot, d_deg,
                                      nullptr) == hipSuccess;
        ok = ok && hipMemcpy(deg.data(), d_deg, n_hot * sizeof(int64_t), hipMemcpyDeviceToHost) ==
                       hipSuccess;
        if (d_deg) (void)hipFree(d_deg);
        if (!ok) return GNN_ERR_HIP;
    }
    std::vector<int32_t> node;
    std::vector<int64_t> off;
    int64_t used = 0;
    for (int64_t i = 0; i < n_hot; ++i) {
        const int64_t dv = deg[static_cast<size_t>(i)];
        if (used + dv > max_entries) break;   // the hottest rows that fit, in order
        if (dv <= 0) continue;                // an empty row needs no copy
        node.push_back(hot[static_cast<size_t>(i)]);
        off.push_back(used);
        used += dv;
    }
    gnn_adjacency_cache *c = new (std::nothrow) gnn_adjacency_cache{};
    if (!c) return GNN_ERR_INVALID_ARG;
    c->num_nodes = g->num_nodes;
    const int64_t n = static_cast<int64_t>(node.size());
    int32_t *d_node = nullptr;
    int64_t *d_off = nullptr;
    bool ok = hipMalloc(reinterpret_cast<void **>(&c->adj_off), g->num_nodes * sizeof(int64_t)) ==
              hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&c->rows),
                         (used > 0 ? used : 1) * sizeof(int32_t)) == hipSuccess;
    ok = ok && hipMemset(c->adj_off, 0xFF, g->num_nodes * sizeof(int64_t)) == hipSuccess;  // -1
    if (ok && n > 0) {
        ok = hipMalloc(reinterpret_cast<void **>(&d_node), n * sizeof(int32_t)) == hipSuccess;
        ok = ok && hipMalloc(reinterpret_cast<void **>(&d_off), n * sizeof(int64_t)) == hipSuccess;
        ok = ok && hipMemcpy(d_node, node.data(), n * sizeof(int32_t), hipMemcpyHostToDevice) ==
                       hipSuccess;
        ok = ok && hipMemcpy(d_off, off.data(), n * sizeof(int64_t), hipMemcpyHostToDevice) ==
                       hipSuccess;
        ok = ok && launch_adj_fill(g->indptr, g->indptr_bytes, g->indices, d_node, d_off, n,
                                   c->rows, c->adj_off, nullptr) == hipSuccess;
    }
    ok = ok && hipDeviceSynchronize() == hipSuccess;
    if (d_node) (void)hipFree(d_node);
    if (d_off) (void)hipFree(d_off);
    if (!ok) {
        gnn_adjacency_cache_destroy(c);
        return GNN_ERR_HIP;
    }
    c->n_rows = n;
    c->n_entries = used;
    if (out_rows) *out_rows = n;
    if (out_entries) *out_entries = used;
    *out = c;
    return GNN_OK;
}

gnn_status gnn_adjacency_cache_attach(const gnn_adjacency_cache *c, gnn_graph *g) {
    if (!g) return GNN_ERR_INVALID_ARG;
    if (!c) {
        g->adj_off = nullptr;
        g->adj_rows = nullptr;
        return GNN_OK;
    }
    if (c->num_nodes != g->num_nodes) return GNN_ERR_INVALID_ARG;
    g->adj_off = c->adj_off;
    g->adj_rows = c->rows;
    return GNN_OK;
}

gnn_status gnn_adjacency_cache_destroy(gnn_adjacency_cache *c) {
    if (!c) return GNN_OK;
    if (c->adj_off) (void)hipFree(c->adj_off);
    if (c->rows) (void)hipFree(c->rows);
    delete c;
    return GNN_OK;
}

gnn_status gnn_feature_store_destroy(gnn_feature_store *fs) {
    if (!fs) return GNN_OK;
    if (fs->cache) (void)hipFree(fs->cache);
    if (fs->slot) (void)hipFree(fs->slot);
    dyn_free(fs->dyn);
    delete fs;
    return GNN_OK;
}

gnn_status gnn_feature_store_enable_dynamic(gnn_feature_store *fs, const gnn_dyn_cache_params *p) {
    if (!fs || !p || fs->dyn) return GNN_ERR_INVALID_ARG;
    if (!(p->gamma > 0.0 && p->gamma < 1.0) || p->k_dyn < 1 || p->t_update < 1 ||
        p->max_refreshes < 0 || (p->flags & ~GNN_DYN_AUTO) != 0)
        return GNN_ERR_INVALID_ARG;
    if (p->k_dyn > fs->num_nodes - fs->cache_rows) return GNN_ERR_INVALID_ARG;
    if (fault(kFaultAlloc)) return GNN_ERR_HIP;
    DynCache *dc = new (std::nothrow) DynCache();
    if (!dc) return GNN_ERR_HIP;
    dc->p = *p;
    const int64_t N = fs->num_nodes;
    const int64_t words = (N + 31) / 32;
    const int64_t rows = fs->cache_rows + p->k_dyn;
    float *cache = nullptr;
    int32_t *slot = nullptr;
    bool ok = hipDeviceSynchronize() == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&cache),
                         static_cast<size_t>(rows) * fs->ld * sizeof(float)) == hipSuccess;
    if (ok && fs->cache_rows > 0)
        ok = hipMemcpy(cache, fs->cache, static_cast<size_t>(fs->cache_rows) * fs->ld * sizeof(float),
                       hipMemcpyDeviceToDevice) == hipSuccess;
    if (ok && !fs->slot) {
        ok = hipMalloc(reinterpret_cast<void **>(&slot), static_cast<size_t>(N) * sizeof(int32_t)) ==
             hipSuccess;
        ok = ok && launch_fill_i32(slot, N, -1, nullptr) == hipSuccess;
    }
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->score), static_cast<size_t>(N) * 8) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->touched), static_cast<size_t>(words) * 4) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->member), static_cast<size_t>(words) * 4) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->cand), static_cast<size_t>(N) * 4) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->key_hi), static_cast<size_t>(N) * 4) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->key_lo), static_cast<size_t>(N) * 4) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->free_rows),
                         static_cast<size_t>(p->k_dyn) * 4) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->admit), static_cast<size_t>(p->k_dyn) * 4) ==
               hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->row_node), static_cast<size_t>(p->k_dyn) * 4) ==
               hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->filled),
                         static_cast<size_t>((p->k_dyn + 3) / 4 * 4)) == hipSuccess;
    ok = ok && hipMalloc(reinterpret_cast<void **>(&dc->state), sizeof(DynState)) == hipSuccess;
    ok = ok && launch_fill_u32(reinterpret_cast<uint32_t *>(dc->score), 2 * N, 0u, nullptr) == hipSuccess;
    ok = ok && launch_fill_u32(dc->touched, words, 0u, nullptr) == hipSuccess;
    ok = ok && launch_fill_u32(dc->member, words, 0u, nullptr) == hipSuccess;
    ok = ok && launch_dyn_init(dc->state, dc->free_rows, dc->row_node, dc->filled, p->k_dyn,
                               nullptr) == hipSuccess;
    ok = ok && hipDeviceSynchronize() == hipSuccess;
    if (!ok) {
        if (cache) (void)hipFree(cache);
        if (slot) (void)hipFree(slot);
        dyn_free(dc);
        return GNN_ERR_HIP;
    }
    if (fs->cache) (void)hipFree(fs->cache);
    fs->cache = cache;
    if (slot) fs->slot = slot;
    fs->dyn = dc;
    return GNN_OK;
}

gnn_status gnn_dyn_cache_update(const gnn_feature_store *fs, int32_t *refreshed, int32_t *d_status,
                                gnn_stream stream) {
    if (refreshed) *refreshed = 0;
    if (!fs || !fs->dyn) return GNN_ERR_INVALID_ARG;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    return dyn_refresh(fs, d_status, static_cast<hipStream_t>(stream), refreshed);
}

gnn_status gnn_dyn_cache_query(const gnn_feature_store *fs, gnn_dyn_cache_info *out) {
    if (!fs || !fs->dyn || !out) return GNN_ERR_INVALID_ARG;
    DynCache *dc = fs->dyn;
    DynState st;
    GNN_TRY_HIP(hipDeviceSynchronize());
    GNN_TRY_HIP(hipMemcpy(&st, dc->state, sizeof(st), hipMemcpyDeviceToHost));
    std::lock_guard<std::mutex> lk(dc->mu);
    *out = gnn_dyn_cache_info{};
    out->steps = dc->steps;
    out->since_refresh = dc->steps - dc->steps_at_refresh;
    out->refreshes = dc->refreshes;
    out->frozen = dyn_frozen(dc) ? 1 : 0;
    out->due = !out->frozen && out->since_refresh >= dc->p.t_update ? 1 : 0;
    out->members = st.members;
    out->last_candidates = st.n_cand;
    out->last_admitted = st.n_admit;
    out->last_evicted = st.n_evict;
    out->resident = st.n_resident;
    out->last_published = st.n_published;
    return GNN_OK;
}

gnn_status gnn_dyn_cache_state(const gnn_feature_store *fs, double *score, uint8_t *member,
                               gnn_stream stream) {
    if (!fs || !fs->dyn) return GNN_ERR_INVALID_ARG;
    DynCache *dc = fs->dyn;
    double scale;
    {
        std::lock_guard<std::mutex> lk(dc->mu);
        // Score(v, t) = S(v) / w_t, and the last observed mini-batch's weight is w_next * gamma
        scale = dc->steps > 0 ? 1.0 / (dc->w_next * dc->p.gamma) : 0.0;
    }
    GNN_TRY_HIP(launch_dyn_state(dc->score, fs->num_nodes, scale, fs->slot,
                                 static_cast<int32_t>(fs->cache_rows), score, member,
                                 static_cast<hipStream_t>(stream)));
    return GNN_OK;
}

gnn_status gnn_gather_features(const gnn_feature_store *fs, const int32_t *ids,
                               const int64_t *d_n, int64_t n, float *out, int64_t ld_out,
                               int64_t *d_hits, int32_t *d_status, gnn_stream stream) {
    if (!fs || n < 0 || ld_out < fs->d) return GNN_ERR_INVALID_ARG;
    if (n > 0 && (!ids || !out)) return GNN_ERR_INVALID_ARG;
    if (n * fs->d > kFlatMax) return GNN_ERR_UNSUPPORTED;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    double w = 0.0;
    DynObserve obs;
    GNN_TRY(dyn_observe_steps(fs, 1, &w, &obs, s));
    GNN_TRY_HIP(launch_gather(fs->table, fs->cache, fs->slot, fs->ld, fs->d, fs->num_nodes, ids,
                              d_n, n, out, ld_out, d_hits, d_status, s,
                              obs.filled ? &obs : nullptr, w));
    return dyn_auto_refresh(fs, d_status, s);
}

gnn_status gnn_gather_features_match(const gnn_feature_store *fs, const int32_t *ids,
                                     const int64_t *d_n, int64_t n, float *out, int64_t ld_out,
                                     const int32_t *prev_ids, const int64_t *d_prev_n,
                                     int64_t prev_n, const float *prev_x, int64_t ld_prev,
                                     int32_t *match, int64_t *d_matched, int64_t *d_hits,
                                     int32_t *d_status, gnn_stream stream) {
    if (!fs || n < 0 || ld_out < fs->d || prev_n < 0 || ld_prev < fs->d) return GNN_ERR_INVALID_ARG;
    if (n > 0 && (!ids || !out || !match)) return GNN_ERR_INVALID_ARG;
    if (prev_n > 0 && (!prev_ids || !prev_x)) return GNN_ERR_INVALID_ARG;
    if (n * fs->d > kFlatMax) return GNN_ERR_UNSUPPORTED;
    if (fs->dyn != nullptr) return GNN_ERR_UNSUPPORTED;
    if (fs->cache_rows >= kPrevCodeBound || prev_n >= kPrevCodeBound) return GNN_ERR_UNSUPPORTED;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const MatchArgs ma{ids, d_n, n, prev_ids, d_prev_n, prev_n, match, d_matched};
    GNN_TRY_HIP(launch_match(ma, s));
    GNN_TRY_HIP(launch_gather(fs->table, fs->cache, fs->slot, fs->ld, fs->d, fs->num_nodes, ids,
                              d_n, n, out, ld_out, d_hits, d_status, s, nullptr, 0.0,
                              prev_n > 0 ? match : nullptr, prev_x, ld_prev));
    return GNN_OK;
}

gnn_status gnn_batch_overlap(const int32_t *const *ids, const int64_t *const *d_n, const int64_t *n,
                             int32_t B, int64_t *overlap, gnn_stream stream) {
    if (B < 1 || B > GNN_MAX_GROUP || !ids || !n || !overlap) return GNN_ERR_INVALID_ARG;
    OverlapArgs a{};
    a.B = B;
    for (int l = 0; l < B; ++l) {
        if (n[l] < 0 || (n[l] > 0 && !ids[l])) return GNN_ERR_INVALID_ARG;
        a.ids[l] = ids[l];
        a.d_n[l] = d_n ? d_n[l] : nullptr;
        a.cap[l] = n[l];
    }
    for (int x = 0; x < B; ++x)
        for (int y = x + 1; y < B; ++y) {
            a.pa[a.npairs] = static_cast<uint8_t>(x);
            a.pb[a.npairs] = static_cast<uint8_t>(y);
            ++a.npairs;
        }
    a.out = reinterpret_cast<unsigned long long *>(overlap);
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    GNN_TRY_HIP(launch_overlap(a, static_cast<hipStream_t>(stream)));
    return GNN_OK;
}

gnn_status gnn_greedy_order(const int64_t *overlap, int32_t B, int32_t first, int32_t *order) {
    if (!overlap || !order || B < 1 || first < 0 || first >= B) return GNN_ERR_INVALID_ARG;
    std::vector<char> placed(static_cast<size_t>(B), 0);
    order[0] = first;
    placed[static_cast<size_t>(first)] = 1;
    for (int i = 1; i < B; ++i) {
        const int last = order[i - 1];
        int best = -1;
        for (int b = 0; b < B; ++b) {
            if (placed[static_cast<size_t>(b)]) continue;
            if (best < 0 || overlap[static_cast<int64_t>(last) * B + b] >
                                overlap[static_cast<int64_t>(last) * B + best])
                best = b;
        }
        order[i] = best;
        placed[static_cast<size_t>(best)] = 1;
    }
    return GNN_OK;
}

gnn_status gnn_mean_aggregate(const int32_t *indptr, const int32_t *lid, int64_t n_lid,
                              const int64_t *d_n_dst, int64_t n_dst, const float *src,
                              int64_t ld_src, int64_t n_src, int64_t d, float *out,
                              int64_t ld_out, int32_t *d_status, gnn_stream stream) {
    if (n_dst < 0 || n_lid < 0 || n_src < 0 || d < 1 || ld_src < d || ld_out < d)
        return GNN_ERR_INVALID_ARG;
    if (n_dst > 0 && (!indptr || !out)) return GNN_ERR_INVALID_ARG;
    if (n_lid > 0 && (!lid || !src)) return GNN_ERR_INVALID_ARG;
    if (n_dst * d > kFlatMax) return GNN_ERR_UNSUPPORTED;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    const MeanJob job{indptr, lid, n_lid, d_n_dst, n_dst, src, n_src, out};
    GNN_TRY_HIP(launch_mean(&job, 1, ld_src, ld_out, d, 16, d_status,
                            static_cast<hipStream_t>(stream)));
    return GNN_OK;
}

namespace {
gnn_status check_sage(const int32_t *dst_lid, int64_t n_dst, const float *src, int64_t ld_src,
                      int64_t n_src, int64_t d, const float *agg, int64_t ld_agg, const float *W,
                      int64_t d_out, const float *out, int64_t ld_out) {
    if (n_dst < 0 || n_src < 0 || d < 1 || ld_src < d || ld_agg < d) return GNN_ERR_INVALID_ARG;
    if (d_out < 1 || d_out > 65536 || ld_out < d_out) return GNN_ERR_INVALID_ARG;
    if (n_dst > 0 && (!dst_lid || !src || !W || !agg || !out || n_src < 1))
        return GNN_ERR_INVALID_ARG;
    if (n_dst * d > kFlatMax || n_dst * d_out > kFlatMax || n_dst > kFlatMax / 64)
        return GNN_ERR_UNSUPPORTED;
    return GNN_OK;
}
}  // namespace

gnn_status gnn_sage_update(const int32_t *dst_lid, const int64_t *d_n_dst, int64_t n_dst,
                           const float *src, int64_t ld_src, int64_t n_src, int64_t d,
                           const float *agg, int64_t ld_agg, const float *W, const float *bias,
                           int64_t d_out, int32_t relu, float *out, int64_t ld_out,
                           int32_t *d_status, gnn_stream stream) {
    const gnn_status st =
        check_sage(dst_lid, n_dst, src, ld_src, n_src, d, agg, ld_agg, W, d_out, out, ld_out);
    if (st != GNN_OK) return st;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    GNN_TRY_HIP(launch_sage_update(dst_lid, d_n_dst, n_dst, src, ld_src, n_src, agg, ld_agg, d, W,
                                   bias, d_out, relu, out, ld_out, d_status,
                                   static_cast<hipStream_t>(stream)));
    return GNN_OK;
}

gnn_status gnn_sage_layer(const int32_t *indptr, const int32_t *lid, int64_t n_lid,
                          const int32_t *dst_lid, const int64_t *d_n_dst, int64_t n_dst,
                          const float *src, int64_t ld_src, int64_t n_src, int64_t d,
                          const float *W, const float *bias, int64_t d_out, int32_t relu,
                          float *agg, int64_t ld_agg, float *out, int64_t ld_out,
                          int32_t *d_status, gnn_stream stream) {
    gnn_status st =
        check_sage(dst_lid, n_dst, src, ld_src, n_src, d, agg, ld_agg, W, d_out, out, ld_out);
    if (st != GNN_OK) return st;
    if (n_lid < 0 || (n_dst > 0 && !indptr) || (n_lid > 0 && !lid)) return GNN_ERR_INVALID_ARG;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const MeanJob job{indptr, lid, n_lid, d_n_dst, n_dst, src, n_src, agg};
    GNN_TRY_HIP(launch_mean(&job, 1, ld_src, ld_agg, d, 16, d_status, s));
    GNN_TRY_HIP(launch_sage_update(dst_lid, d_n_dst, n_dst, src, ld_src, n_src, agg, ld_agg, d, W,
                                   bias, d_out, relu, out, ld_out, d_status, s));
    return GNN_OK;
}

gnn_status gnn_minibatch(const gnn_graph *g, const gnn_feature_store *fs, const int32_t *seeds,
                         const int64_t *batch_ptr, int32_t group, const int32_t *fanouts,
                         int32_t num_hops, uint64_t seed64, gnn_minibatch_out *outs, void *ws,
                         size_t ws_bytes, const gnn_options *opt, gnn_stream stream,
                         gnn_timer *timer) {
    gnn_status st = check_graph(g);
    if (st == GNN_OK) st = check_fanouts(fanouts, num_hops);
    if (st != GNN_OK) return st;
    if (!fs || fs->num_nodes != g->num_nodes || !batch_ptr || !outs || group < 1 || !ws)
        return GNN_ERR_INVALID_ARG;
    if (group > GNN_MAX_GROUP) return GNN_ERR_UNSUPPORTED;
    if (batch_ptr[0] != 0) return GNN_ERR_INVALID_ARG;
    Opts o;
    if ((st = read_opts(opt, &o)) != GNN_OK) return st;
    const int K = num_hops;
    const int64_t d = fs->d;
    gnn_caps mc = outs[0].blocks.caps;
    const int32_t *sp[GNN_MAX_GROUP];
    int64_t nsg[GNN_MAX_GROUP];
    gnn_blocks *ob[GNN_MAX_GROUP];
    for (int gi = 0; gi < group; ++gi) {
        const int64_t ns = batch_ptr[gi + 1] - batch_ptr[gi];
        if (ns < 0 || (ns > 0 && !seeds)) return GNN_ERR_INVALID_ARG;
        gnn_minibatch_out &mo = outs[gi];
        if ((st = check_blocks(&mo.blocks, ns, fanouts, K)) != GNN_OK) return st;
        if (mo.ld_h < d || mo.ld_h != outs[0].ld_h) return GNN_ERR_INVALID_ARG;
        const gnn_caps &c = mo.blocks.caps;
        if (c.nodes[K - 1] > 0 && !mo.x) return GNN_ERR_INVALID_ARG;
        for (int l = 0; l < K; ++l) {
            const int64_t rows = l == 0 ? ns : c.nodes[l - 1];
            if (rows > 0 && !mo.h[l]) return GNN_ERR_INVALID_ARG;
            if (c.nodes[l] * d > kFlatMax || rows * d > kFlatMax) return GNN_ERR_UNSUPPORTED;
            mc.frontier[l] = c.frontier[l] > mc.frontier[l] ? c.frontier[l] : mc.frontier[l];
            mc.edges[l] = c.edges[l] > mc.edges[l] ? c.edges[l] : mc.edges[l];
            mc.nodes[l] = c.nodes[l] > mc.nodes[l] ? c.nodes[l] : mc.nodes[l];
        }
        sp[gi] = seeds ? seeds + batch_ptr[gi] : nullptr;
        nsg[gi] = ns;
        ob[gi] = &mo.blocks;
    }
    // A super-batch samples the union of its sub-batches' frontiers into one block whose offsets
    // are int32 (like every block): its worst case, G times a sub-batch's frontier bound (at most
    // N) times the fanout, must fit, although each sub-batch's own caps already do.
    if (group > 1 && max_union_edges(mc, g->num_nodes, group) > kInt32Max) return GNN_ERR_UNSUPPORTED;
    const SuperMode mode = super_mode(mc, g->num_nodes, group, o.flags);
    const Workspace need = carve(mc, g->num_nodes, group, mode, nullptr);
    if (ws_bytes < need.bytes) return GNN_ERR_CAPACITY;
    if (fault(kFaultLaunch)) return GNN_ERR_HIP;
    // How stages 2 and 3 run (below).  Batched unless interleaving is asked for: one launch's
    // start-up and drain instead of G, G times as many host-link reads in flight for a
    // host-resident table, and (with a table in HBM) the shared outermost means; measured faster
    // or equal on the 602-, 128-, 100- and 64-float workloads.
    const bool batched = !(o.flags & GNN_GATHER_INTERLEAVED);
    // Batched from a table in HBM without a cache, the outermost means read table rows by global
    // id; with room in the workspace they are then taken once per node of the union frontier
    // U_{K-1} and copied to the sub-batches that hold it (the G sub-batches share one seed, so a
    // node's sampled neighbours, hence its mean, are the same in each).
    const bool from_table = batched && !fs->on_host && fs->slot == nullptr;
    const bool shared_means = from_table && group > 1;
    Workspace w = carve(mc, g->num_nodes, group, mode, ws);
    w.relabel_force = relabel_force(o);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t *ev = nullptr;
    if (timer) {
        if (timer->cursor >= timer->n_records) return GNN_ERR_CAPACITY;
        ev = timer->ev.data() + static_cast<size_t>(timer->cursor) * kTimerSlots;
        timer->group[timer->cursor] = group;
        timer->hops[timer->cursor] = K;
        timer->batched[timer->cursor] = batched ? 1 : 0;
        timer->cursor += 1;
        GNN_TRY_HIP(hipEventRecord(ev[0], s));
    }
    GNN_TRY_HIP(launch_fill_u32(reinterpret_cast<uint32_t *>(w.status), w.cleared_bytes() / 4, 0u, s));
    // Stage 1: sampling and relabel of every sub-batch (one shared seed64).
    st = run_sample(*g, sp, nsg, group, fanouts, K, seed64, ob, w, o, s,
                    ev ? ev + kSampleEvents : nullptr);
    if (st != GNN_OK) return st;
    // From a table in HBM, a super-batch with rows wider than 128 floats gathers the union U_K of
    // its sub-batches' V_K: each distinct row is read once and stored to the X of every sub-batch
    // that holds it (dense 602-d workload, union 31% of the sub-batches' rows: 3-stream throughput
    // +12%).  With narrower rows the reads saved are smaller than the cost of building U_K and
    // finding each row's destinations (100-d, union 43%: +1%; 128-d, union 76%: -4%), so they keep
    // the per-sub-batch gather.  Building U_K is relabel work and is timed with stage 1.
    const bool union_path = from_table && group > 1 && d > kUnionGatherMinD &&
                            union_gather_fits(fs, outs, group, w);
    const int32_t *uK = nullptr;
    if (union_path) {
        uK = union_prepare(*g, outs, group, K, mc, w, s, &st);
        if (st != GNN_OK) return st;
    }
    if (ev) GNN_TRY_HIP(hipEventRecord(ev[1], s));
    // With a Dynamic-Cache, each sub-batch's gather is one observed mini-batch.
    double obs_w[GNN_MAX_GROUP] = {};
    DynObserve obs;
    GNN_TRY(dyn_observe_steps(fs, group, obs_w, &obs, s));
    // Stages 2 and 3: gather X = rows of V_K, then the outermost block's mean.  Batched: every
    // sub-batch's gather in one launch, then every outermost mean in one launch.  Interleaved: per
    // sub-batch, so the mean reads X while it is still in the caches.
    if (batched) {
        GatherBatchArgs ga{};
        ga.nseg = group;
        ga.table = fs->table;
        ga.cache = fs->cache;
        ga.slot = fs->slot;
        ga.ld = fs->ld;
        ga.d = static_cast<int32_t>(d);
        ga.num_rows = fs->num_nodes;
        ga.ld_out = outs[0].ld_h;
        ga.status = w.status;
        ga.obs = obs;
        ga.d_hits = o.d_hits;
        int64_t rows_cap = 0;
        MeanJob jobs[GNN_MAX_GROUP];
        for (int gi = 0; gi < group; ++gi) {
            gnn_minibatch_out &mo = outs[gi];
            const gnn_caps &c = mo.blocks.caps;
            ga.seg[gi] = GatherSeg{mo.blocks.hop[K - 1].nodes, mo.blocks.counts + 2 * (K - 1) + 1,
                                   c.nodes[K - 1], mo.x, obs_w[gi]};
            rows_cap += c.nodes[K - 1];
            const int64_t *d_n = K == 1 ? nullptr : mo.blocks.counts + 2 * (K - 2) + 1;
            if (from_table)   // X[lid[e]] is table row gid[e], bit for bit
                jobs[gi] = MeanJob{mo.blocks.hop[K - 1].indptr, mo.blocks.hop[K - 1].gid, c.edges[K - 1],
                                   d_n, c.frontier[K - 1], fs->table, fs->num_nodes, mo.h[K - 1]};
            else
                jobs[gi] = MeanJob{mo.blocks.hop[K - 1].indptr, mo.blocks.hop[K - 1].lid, c.edges[K - 1],
                                   d_n, c.frontier[K - 1], mo.x, c.nodes[K - 1], mo.h[K - 1]};
        }
        if (union_path) {
            float *xs[GNN_MAX_GROUP];
            for (int gi = 0; gi < group; ++gi) xs[gi] = outs[gi].x;
            // the sub-batch relabel bitmaps of the last hop: over U_K positions (compact) or node
            // ids (full), by their rank directories
            const bool compact = w.mode == kSuperCompact;
            GNN_TRY_HIP(launch_gather_union(fs->table, fs->ld, d, fs->num_nodes, uK, w.d_U + K,
                                            union_cap(mc, K, group, g->num_nodes), w.rdir + w.W,
                                            compact ? w.Wc : w.W, compact ? 0 : 1,
                                            group, xs, outs[0].ld_h, w.status, s));
        } else {
            GNN_TRY_HIP(launch_gather_batch(ga, rows_cap, s));
        }
        if (ev) GNN_TRY_HIP(hipEventRecord(ev[2], s));
        if (shared_means) {
            // the union block of the last hop (destinations U_{K-1} in U order, global ids): each
            // union node's mean is stored to its row in every sub-batch that holds it
            const int64_t Ucap = union_cap(mc, K - 1, group, g->num_nodes);
            const int64_t *d_U = w.d_U + (w.mode == kSuperCompact ? K - 1 : 0);
            const MeanJob uj{w.u_indptr, w.u_gid, Ucap * fanouts[K - 1], d_U, Ucap, fs->table,
                             fs->num_nodes, nullptr};
            float *hk[GNN_MAX_GROUP];
            for (int gi = 0; gi < group; ++gi) hk[gi] = outs[gi].h[K - 1];
            GNN_TRY_HIP(launch_mean_scatter(uj, w.inv, w.inv_mask, group, hk, fs->ld, outs[0].ld_h, d,
                                            w.status, s));
        } else {
            GNN_TRY_HIP(launch_mean(jobs, group, from_table ? fs->ld : outs[0].ld_h, outs[0].ld_h, d,
                                    fanouts[K - 1], w.status, s));
        }
        if (ev) GNN_TRY_HIP(hipEventRecord(ev[1 + 2 * group], s));
    } else {
        for (int gi = 0; gi < group; ++gi) {
            gnn_minibatch_out &mo = outs[gi];
            const gnn_caps &c = mo.blocks.caps;
            GNN_TRY_HIP(launch_gather(fs->table, fs->cache, fs->slot, fs->ld, d, fs->num_nodes,
                                      mo.blocks.hop[K - 1].nodes, mo.blocks.counts + 2 * (K - 1) + 1,
                                      c.nodes[K - 1], mo.x, mo.ld_h, o.d_hits, w.status, s,
                                      obs.filled ? &obs : nullptr, obs_w[gi]));
            if (ev) GNN_TRY_HIP(hipEventRecord(ev[2 + 2 * gi], s));
            const int64_t *d_n = K == 1 ? nullptr : mo.blocks.counts + 2 * (K - 2) + 1;
            const MeanJob job{mo.blocks.hop[K - 1].indptr, mo.blocks.hop[K - 1].lid, c.edges[K - 1],
                              d_n, c.frontier[K - 1], mo.x, c.nodes[K - 1], mo.h[K - 1]};
            GNN_TRY_HIP(launch_mean(&job, 1, mo.ld_h, mo.ld_h, d, fanouts[K - 1], w.status, s));
            if (ev) GNN_TRY_HIP(hipEventRecord(ev[3 + 2 * gi], s));
        }
    }
    // Stage 4: the inner blocks, h_{l-1} from h_l for l = K-1..1, every sub-batch in one launch.
    for (int l = K - 1; l >= 1; --l) {
        MeanJob jobs[GNN_MAX_GROUP];
        for (int gi = 0; gi < group; ++gi) {
            gnn_minibatch_out &mo = outs[gi];
            const gnn_caps &c = mo.blocks.caps;
            const int64_t *d_n = l == 1 ? nullptr : mo.blocks.counts + 2 * (l - 2) + 1;
            jobs[gi] = MeanJob{mo.blocks.hop[l - 1].indptr, mo.blocks.hop[l - 1].lid, c.edges[l - 1],
                               d_n, c.frontier[l - 1], mo.h[l], c.nodes[l - 1], mo.h[l - 1]};
        }
        GNN_TRY_HIP(launch_mean(jobs, group, outs[0].ld_h, outs[0].ld_h, d, fanouts[l - 1],
                                w.status, s));
    }
    if (ev) GNN_TRY_HIP(hipEventRecord(ev[2 + 2 * group], s));
    GNN_TRY(dyn_auto_refresh(fs, w.status, s));
    return finish(o, w, s);
}

gnn_status gnn_read_device_status(const void *ws, gnn_stream stream, gnn_status *out) {
    if (!ws || !out) return GNN_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t st = 0;
    GNN_TRY_HIP(hipMemcpyAsync(&st, ws, sizeof(st), hipMemcpyDeviceToHost, s));
    GNN_TRY_HIP(hipStreamSynchronize(s));
    *out = st;
    return GNN_OK;
}

gnn_status gnn_timer_create(int32_t n_records, gnn_timer **out) {
    if (!out || n_records < 1) return GNN_ERR_INVALID_ARG;
    gnn_timer *t = new (std::nothrow) gnn_timer{};
    if (!t) return GNN_ERR_INVALID_ARG;
    t->n_records = n_records;
    t->cursor = 0;
    t->ev.assign(static_cast<size_t>(n_records) * kTimerSlots, nullptr);
    t->group.assign(static_cast<size_t>(n_records), 0);
    t->hops.assign(static_cast<size_t>(n_records), 0);
    t->batched.assign(static_cast<size_t>(n_records), 0);
    for (auto &e : t->ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            gnn_timer_destroy(t);
            return GNN_ERR_HIP;
        }
    }
    *out = t;
    return GNN_OK;
}

gnn_status gnn_timer_destroy(gnn_timer *t) {
    if (!t) return GNN_OK;
    for (auto &e : t->ev)
        if (e) (void)hipEventDestroy(e);
    delete t;
    return GNN_OK;
}

gnn_status gnn_timer_reset(gnn_timer *t) {
    if (!t) return GNN_ERR_INVALID_ARG;
    t->cursor = 0;
    return GNN_OK;
}

gnn_status gnn_timer_elapsed(gnn_timer *t, int32_t *n_records, float *ms) {
    if (!t || !n_records) return GNN_ERR_INVALID_ARG;
    *n_records = t->cursor;
    if (t->cursor == 0) return GNN_OK;
    if (!ms) return GNN_ERR_INVALID_ARG;
    for (int r = 0; r < t->cursor; ++r) {
        const hipEvent_t *e = t->ev.data() + static_cast<size_t>(r) * kTimerSlots;
        const int G = t->group[r];
        GNN_TRY_HIP(hipEventSynchronize(e[2 + 2 * G]));
        float v = 0.f, gat = 0.f, outer = 0.f;
        GNN_TRY_HIP(hipEventElapsedTime(&v, e[0], e[1]));
        ms[r * GNN_TIMER_STAGES + 0] = v;
        if (t->batched[r]) {
            GNN_TRY_HIP(hipEventElapsedTime(&gat, e[1], e[2]));
            GNN_TRY_HIP(hipEventElapsedTime(&outer, e[2], e[1 + 2 * G]));
        } else {
            for (int gi = 0; gi < G; ++gi) {
                GNN_TRY_HIP(hipEventElapsedTime(&v, e[1 + 2 * gi], e[2 + 2 * gi]));
                gat += v;
                GNN_TRY_HIP(hipEventElapsedTime(&v, e[2 + 2 * gi], e[3 + 2 * gi]));
                outer += v;
            }
        }
        ms[r * GNN_TIMER_STAGES + 1] = gat;
        ms[r * GNN_TIMER_STAGES + 2] = outer;
        GNN_TRY_HIP(hipEventElapsedTime(&v, e[1 + 2 * G], e[2 + 2 * G]));
        ms[r * GNN_TIMER_STAGES + 3] = v;
        float smp = 0.f;
        for (int l = 0; l < t->hops[r]; ++l) {
            GNN_TRY_HIP(hipEventElapsedTime(&v, e[kSampleEvents + 2 * l], e[kSampleEvents + 2 * l + 1]));
            smp += v;
        }
        ms[r * GNN_TIMER_STAGES + 4] = smp;
    }
    return GNN_OK;
}

// Host self-check of the invariant-divisor division used by the kernels (not part of the
// public header): returns the number of mismatches against plain division over a sweep.
int64_t gnn__fastdiv_selfcheck(uint32_t max_divisor) {
    int64_t bad = 0;
    uint64_t x = 88172645463325252ull;
    for (uint32_t dv = 1; dv <= max_divisor; ++dv) {
        const FastDiv f = make_fastdiv(dv);
        for (int t = 0; t < 2000; ++t) {
            x ^= x << 13;
            x ^= x >> 7;
            x ^= x << 17;
            const uint32_t n = t < 4 ? static_cast<uint32_t>(dv * t + (t & 1) - 1u)
                                     : static_cast<uint32_t>(x) & 0x7FFFFFFFu;
            if (fast_div(n, f) != n / dv) ++bad;
        }
        const uint32_t edge[3] = {0x7FFFFFFFu, 0x80000000u, 0xFFFFFFFFu};
        for (uint32_t n : edge)
            if (fast_div(n, f) != n / dv) ++bad;
    }
    return bad;
}

}  // extern "C"
