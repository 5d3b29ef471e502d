// C ABI of the mini-batch library: argument validation, workspace carving, launch sequencing on
// one stream with no host synchronisation, the feature store and the stage timer.
#include <math.h>
#include <string.h>

#include <new>
#include <vector>

#include "common.hpp"

using namespace gnnmb;

struct gnn_feature_store {
    const float *table;  // device-addressable table (mapped pointer for pinned host memory)
    int32_t on_host;
    int64_t num_nodes, d, ld;
    int64_t cache_rows;
    float *cache;   // [cache_rows, ld] in HBM, or NULL
    int32_t *slot;  // [num_nodes] cache slot of each node, -1 if not cached; NULL if no cache
};

struct gnn_timer {
    int32_t n_records;
    int32_t cursor;
    std::vector<hipEvent_t> ev;  // n_records * GNN_TIMER_EVENTS
};

namespace {

#define GNN_TRY_HIP(expr)                                \
    do {                                                 \
        if ((expr) != hipSuccess) return GNN_ERR_HIP;    \
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
    uint32_t *class_count; // [4]
    uint32_t *work;        // [4]
    int32_t *packed;       // [F_max]
    int32_t *lists;        // [4 F_max]
    uint32_t *bsum_c;      // [nb_max]
    uint32_t *bsum_cls;    // [4 nb_max]
    uint32_t *bitmap;      // [W]
    uint32_t *wprefix;     // [W]
    uint32_t *bsum_w;      // [nbw]
    int64_t F_max, nb_max, W, nbw;
    size_t bytes;
};

Workspace carve(int64_t F_max, int64_t num_nodes, void *ws) {
    Workspace w{};
    Carver c{static_cast<char *>(ws)};
    w.F_max = F_max < 1 ? 1 : F_max;
    w.nb_max = (w.F_max + kClassifyTile - 1) / kClassifyTile;
    w.W = (num_nodes + 31) / 32;
    w.nbw = (w.W + kBitmapTile - 1) / kBitmapTile;
    if (w.nbw < 1) w.nbw = 1;
    w.status = c.take<int32_t>(64);
    w.class_count = c.take<uint32_t>(64);
    w.work = c.take<uint32_t>(64);
    w.packed = c.take<int32_t>(w.F_max);
    w.lists = c.take<int32_t>(4 * w.F_max);
    w.bsum_c = c.take<uint32_t>(w.nb_max);
    w.bsum_cls = c.take<uint32_t>(4 * w.nb_max);
    w.bitmap = c.take<uint32_t>(w.W);
    w.wprefix = c.take<uint32_t>(w.W);
    w.bsum_w = c.take<uint32_t>(w.nbw);
    w.bytes = c.off;
    return w;
}

int64_t caps_fmax(const gnn_caps &caps) {
    int64_t f = 1;
    for (int l = 0; l < caps.num_hops; ++l) f = caps.frontier[l] > f ? caps.frontier[l] : f;
    return f;
}

struct Opts {
    int32_t group_max = 256;
    int32_t wave_max = 4096;
    uint32_t flags = 0;
};

gnn_status read_opts(const gnn_options *o, Opts *out) {
    Opts r;
    if (o) {
        if (o->group_max_deg) r.group_max = o->group_max_deg;
        if (o->wave_max_deg) r.wave_max = o->wave_max_deg;
        r.flags = o->flags;
    }
    if (r.group_max < 1 || r.wave_max < r.group_max) return GNN_ERR_INVALID_ARG;
    *out = r;
    return GNN_OK;
}

gnn_status check_graph(const gnn_graph *g) {
    if (!g || g->num_nodes < 1 || g->num_nodes > kInt32Max || g->num_edges < 0) return GNN_ERR_INVALID_ARG;
    if (g->indptr_bytes != 4 && g->indptr_bytes != 8) return GNN_ERR_INVALID_ARG;
    if (g->indptr_bytes == 4 && g->num_edges > kInt32Max) return GNN_ERR_INVALID_ARG;
    if (!g->indptr || (g->num_edges > 0 && !g->indices)) return GNN_ERR_INVALID_ARG;
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

// Caps must chain (frontier[0] = n_seeds, frontier[l] = nodes[l-1]), fit int32, and every array
// a non-empty cap refers to must exist.
gnn_status check_blocks(const gnn_blocks *b, int64_t n_seeds, int32_t K) {
    if (!b || !b->counts) return GNN_ERR_INVALID_ARG;
    const gnn_caps &c = b->caps;
    if (c.num_hops != K || c.n_seeds != n_seeds || c.frontier[0] != n_seeds) return GNN_ERR_INVALID_ARG;
    for (int l = 0; l < K; ++l) {
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

// Sampling and relabel of every hop of one batch; no host synchronisation.
gnn_status run_sample_khop(const gnn_graph &g, const int32_t *seeds, int64_t n_seeds,
                           const int32_t *fanouts, int32_t K, uint64_t seed64, gnn_blocks &out,
                           const Workspace &w, const Opts &o, hipStream_t s) {
    const gnn_caps &c = out.caps;
    for (int l = 0; l < K; ++l) {
        HopArgs h{};
        h.indptr = g.indptr;
        h.indices = g.indices;
        h.num_nodes = g.num_nodes;
        h.front = l == 0 ? seeds : out.hop[l - 1].nodes;
        h.d_F = l == 0 ? nullptr : out.counts + 2 * (l - 1) + 1;
        h.F_cap = c.frontier[l];
        h.ib = g.indptr_bytes;
        h.k = fanouts[l];
        h.hop_seed = mix64(seed64 + kGamma * static_cast<uint64_t>(l + 1));
        h.group_max = o.group_max;
        h.wave_max = o.wave_max;
        h.blk_indptr = out.hop[l].indptr;
        h.blk_gid = out.hop[l].gid;
        h.E_cap = c.edges[l];
        h.d_E = out.counts + 2 * l;
        h.packed = w.packed;
        h.lists = w.lists;
        h.bsum_c = w.bsum_c;
        h.bsum_cls = w.bsum_cls;
        h.class_count = w.class_count;
        h.work = w.work;
        h.status = w.status;
        h.nb = static_cast<int32_t>((h.F_cap + kClassifyTile - 1) / kClassifyTile);
        if (h.nb < 1) h.nb = 1;
        GNN_TRY_HIP(launch_classify(h, s));
        GNN_TRY_HIP(launch_sample(h, s));
        RelabelArgs r{};
        r.keep = h.front;
        r.d_keep = h.d_F;
        r.keep_cap = h.F_cap;
        r.add = h.blk_gid;
        r.d_add = h.d_E;
        r.add_cap = h.E_cap;
        r.id_bound = g.num_nodes;
        r.bitmap = w.bitmap;
        r.wprefix = w.wprefix;
        r.bsum = w.bsum_w;
        r.W = w.W;
        r.nbw = static_cast<int32_t>(w.nbw);
        r.uniq = out.hop[l].nodes;
        r.uniq_cap = c.nodes[l];
        r.d_uniq = out.counts + 2 * l + 1;
        r.add_lid = out.hop[l].lid;
        r.keep_lid = out.hop[l].dst_lid;
        r.status = w.status;
        r.check_dup_keep = l == 0 ? 1 : 0;
        GNN_TRY_HIP(launch_relabel(r, s));
    }
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
    if (caps->num_hops < 1 || caps->num_hops > GNN_MAX_HOPS) return GNN_ERR_INVALID_ARG;
    *out_bytes = carve(caps_fmax(*caps), num_nodes, nullptr).bytes;
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
    if ((st = check_blocks(out, n_seeds, num_hops)) != GNN_OK) return st;
    Opts o;
    if ((st = read_opts(opt, &o)) != GNN_OK) return st;
    if (!ws) return GNN_ERR_INVALID_ARG;
    const Workspace need = carve(caps_fmax(out->caps), g->num_nodes, nullptr);
    if (ws_bytes < need.bytes) return GNN_ERR_CAPACITY;
    const Workspace w = carve(caps_fmax(out->caps), g->num_nodes, ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    GNN_TRY_HIP(launch_fill_i32(w.status, 1, 0, s));
    st = run_sample_khop(*g, seeds, n_seeds, fanouts, num_hops, seed64, *out, w, o, s);
    if (st != GNN_OK) return st;
    return finish(o, w, s);
}

gnn_status gnn_relabel_workspace_size(int64_t id_bound, size_t *out_bytes) {
    if (!out_bytes || id_bound < 1 || id_bound > kInt32Max + 1) return GNN_ERR_INVALID_ARG;
    *out_bytes = carve(1, id_bound, nullptr).bytes;
    return GNN_OK;
}

gnn_status gnn_unique_relabel(const int32_t *keep, int64_t n_keep, const int32_t *add,
                              const int64_t *d_n_add, int64_t n_add, int64_t id_bound,
                              int32_t *uniq, int64_t cap_uniq, int64_t *d_n_uniq,
                              int32_t *add_lid, int32_t *keep_lid, void *ws, size_t ws_bytes,
                              gnn_stream stream) {
    if (n_keep < 0 || n_add < 0 || cap_uniq < 0 || id_bound < 1 || id_bound > kInt32Max + 1)
        return GNN_ERR_INVALID_ARG;
    if ((n_keep > 0 && (!keep || !keep_lid)) || (n_add > 0 && (!add || !add_lid)))
        return GNN_ERR_INVALID_ARG;
    if (!d_n_uniq || (cap_uniq > 0 && !uniq) || !ws) return GNN_ERR_INVALID_ARG;
    if (n_keep > kInt32Max || n_add > kInt32Max) return GNN_ERR_UNSUPPORTED;
    const Workspace need = carve(1, id_bound, nullptr);
    if (ws_bytes < need.bytes) return GNN_ERR_CAPACITY;
    const Workspace w = carve(1, id_bound, ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    GNN_TRY_HIP(launch_fill_i32(w.status, 1, 0, s));
    RelabelArgs r{};
    r.keep = keep;
    r.d_keep = nullptr;
    r.keep_cap = n_keep;
    r.add = add;
    r.d_add = d_n_add;
    r.add_cap = n_add;
    r.id_bound = id_bound;
    r.bitmap = w.bitmap;
    r.wprefix = w.wprefix;
    r.bsum = w.bsum_w;
    r.W = w.W;
    r.nbw = static_cast<int32_t>(w.nbw);
    r.uniq = uniq;
    r.uniq_cap = cap_uniq;
    r.d_uniq = d_n_uniq;
    r.add_lid = add_lid;
    r.keep_lid = keep_lid;
    r.status = w.status;
    r.check_dup_keep = 0;
    GNN_TRY_HIP(launch_relabel(r, s));
    return GNN_OK;
}

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

gnn_status gnn_feature_store_destroy(gnn_feature_store *fs) {
    if (!fs) return GNN_OK;
    if (fs->cache) (void)hipFree(fs->cache);
    if (fs->slot) (void)hipFree(fs->slot);
    delete fs;
    return GNN_OK;
}

gnn_status gnn_gather_features(const gnn_feature_store *fs, const int32_t *ids,
                               const int64_t *d_n, int64_t n, float *out, int64_t ld_out,
                               int64_t *d_hits, int32_t *d_status, gnn_stream stream) {
    if (!fs || n < 0 || ld_out < fs->d) return GNN_ERR_INVALID_ARG;
    if (n > 0 && (!ids || !out)) return GNN_ERR_INVALID_ARG;
    if (n * fs->d > kFlatMax) return GNN_ERR_UNSUPPORTED;
    GNN_TRY_HIP(launch_gather(fs->table, fs->cache, fs->slot, fs->ld, fs->d, fs->num_nodes, ids,
                              d_n, n, out, ld_out, d_hits, d_status,
                              static_cast<hipStream_t>(stream)));
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
    GNN_TRY_HIP(launch_mean(indptr, lid, n_lid, d_n_dst, n_dst, src, ld_src, n_src, d, out,
                            ld_out, d_status, static_cast<hipStream_t>(stream)));
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
    if (batch_ptr[0] != 0) return GNN_ERR_INVALID_ARG;
    Opts o;
    if ((st = read_opts(opt, &o)) != GNN_OK) return st;
    int64_t F_max = 1;
    const int K = num_hops;
    const int64_t d = fs->d;
    for (int gi = 0; gi < group; ++gi) {
        const int64_t ns = batch_ptr[gi + 1] - batch_ptr[gi];
        if (ns < 0 || (ns > 0 && !seeds)) return GNN_ERR_INVALID_ARG;
        gnn_minibatch_out &mo = outs[gi];
        if ((st = check_blocks(&mo.blocks, ns, K)) != GNN_OK) return st;
        if (mo.ld_h < d) return GNN_ERR_INVALID_ARG;
        const gnn_caps &c = mo.blocks.caps;
        if (c.nodes[K - 1] > 0 && !mo.x) return GNN_ERR_INVALID_ARG;
        for (int l = 0; l < K; ++l) {
            const int64_t rows = l == 0 ? ns : c.nodes[l - 1];
            if (rows > 0 && !mo.h[l]) return GNN_ERR_INVALID_ARG;
            if (c.nodes[l] * d > kFlatMax || rows * d > kFlatMax) return GNN_ERR_UNSUPPORTED;
        }
        F_max = caps_fmax(c) > F_max ? caps_fmax(c) : F_max;
    }
    const Workspace need = carve(F_max, g->num_nodes, nullptr);
    if (ws_bytes < need.bytes) return GNN_ERR_CAPACITY;
    const Workspace w = carve(F_max, g->num_nodes, ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t *ev = nullptr;
    if (timer) {
        if (timer->cursor >= timer->n_records) return GNN_ERR_CAPACITY;
        ev = timer->ev.data() + static_cast<size_t>(timer->cursor) * GNN_TIMER_EVENTS;
        timer->cursor += 1;
        GNN_TRY_HIP(hipEventRecord(ev[0], s));
    }
    GNN_TRY_HIP(launch_fill_i32(w.status, 1, 0, s));
    // Stage 1: sampling and relabel of every sub-batch (one shared seed64).
    for (int gi = 0; gi < group; ++gi) {
        const int64_t ns = batch_ptr[gi + 1] - batch_ptr[gi];
        st = run_sample_khop(*g, seeds + batch_ptr[gi], ns, fanouts, K, seed64, outs[gi].blocks,
                             w, o, s);
        if (st != GNN_OK) return st;
    }
    if (ev) GNN_TRY_HIP(hipEventRecord(ev[1], s));
    // Stage 2: feature gather X = rows of V_K.
    for (int gi = 0; gi < group; ++gi) {
        gnn_minibatch_out &mo = outs[gi];
        const gnn_caps &c = mo.blocks.caps;
        GNN_TRY_HIP(launch_gather(fs->table, fs->cache, fs->slot, fs->ld, d, fs->num_nodes,
                                  mo.blocks.hop[K - 1].nodes, mo.blocks.counts + 2 * (K - 1) + 1,
                                  c.nodes[K - 1], mo.x, mo.ld_h, nullptr, w.status, s));
    }
    if (ev) GNN_TRY_HIP(hipEventRecord(ev[2], s));
    // Stage 3: mean aggregation, outermost block first: h_{l-1} from h_l, h_K = X.
    for (int l = K; l >= 1; --l) {
        for (int gi = 0; gi < group; ++gi) {
            gnn_minibatch_out &mo = outs[gi];
            const gnn_caps &c = mo.blocks.caps;
            const float *src = l == K ? mo.x : mo.h[l];
            float *dst = mo.h[l - 1];
            const int64_t *d_n = l == 1 ? nullptr : mo.blocks.counts + 2 * (l - 2) + 1;
            GNN_TRY_HIP(launch_mean(mo.blocks.hop[l - 1].indptr, mo.blocks.hop[l - 1].lid,
                                    c.edges[l - 1], d_n, c.frontier[l - 1], src, mo.ld_h,
                                    c.nodes[l - 1], d, dst, mo.ld_h, w.status, s));
        }
        if (ev && l == K) GNN_TRY_HIP(hipEventRecord(ev[3], s));
    }
    if (ev) GNN_TRY_HIP(hipEventRecord(ev[4], s));
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
    t->ev.assign(static_cast<size_t>(n_records) * GNN_TIMER_EVENTS, nullptr);
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
    GNN_TRY_HIP(hipEventSynchronize(t->ev[static_cast<size_t>(t->cursor) * GNN_TIMER_EVENTS - 1]));
    for (int r = 0; r < t->cursor; ++r) {
        for (int k = 0; k + 1 < GNN_TIMER_EVENTS; ++k) {
            float v = 0.f;
            GNN_TRY_HIP(hipEventElapsedTime(&v, t->ev[r * GNN_TIMER_EVENTS + k],
                                            t->ev[r * GNN_TIMER_EVENTS + k + 1]));
            ms[r * (GNN_TIMER_EVENTS - 1) + k] = v;
        }
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
