/*
 * gnnmb.h -- C ABI of the MI355X (gfx950) sampling-based GNN mini-batch hot path.
 *
 * The path is the per-iteration pipeline that the three source pages share:
 *   GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
 *     Co-Design -- Sec. II.A eq. (1) (mean AGGREGATE over in-neighbours), Sec. II.B with Fig. 1
 *     (layer-wise sampling, one bipartite block per layer), Sec. IV.B (feature and adjacency
 *     caches with pinned host fallback), Sec. IV.C (grouping-based parallel sampler, full vs
 *     random nodes), Sec. IV.D
 *     with Alg. 1 (super-batch degree classifier);
 *   LEO: Enabling Efficient Communication-Computation Pipeline for GNN via Hierarchical Caching --
 *     Sec. 2.2 (sample, extract features, train) and Sec. 2.3 (zero-copy feature reads from pinned
 *     host memory);
 *   FastGL: A GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large Scale --
 *     the sample / ship features / compute iteration and the Fused-Map id remapping.
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless marked "host".  The caller allocates and owns every
 *    input, output and workspace buffer; the library keeps no pointer after a call returns, except
 *    that a feature store borrows its table (an adjacency cache holds copies of its rows).  No
 *    call allocates device memory on the hot path (the stores and caches allocate at set-up).
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream) and return without
 *    waiting.  Outputs are valid once the stream has been synchronised.  Data-dependent sizes stay
 *    in device memory ("counts").
 *  - Host-checkable errors return a negative gnn_status and enqueue nothing.  Errors found on the
 *    device (an id out of range, a duplicate seed, a buffer too small) are written to a status
 *    word in the workspace; read it with gnn_read_device_status.  After any error the output
 *    contents are unspecified.  No exception crosses the ABI and the library never aborts.
 *  - Node ids are int32 (num_nodes < 2^31).  Block-local sizes are int32.
 *  - Concurrent calls on different streams are safe when their workspaces are disjoint.
 *  - Fault injection (for tests of callers' error paths): the environment variable GNN_FAULT,
 *    read once per process, may list "alloc" (every set-up allocation of a feature store cache
 *    or an adjacency cache fails before it is made) and "launch" (every call that enqueues work
 *    fails after its argument checks, before enqueueing anything); both return GNN_ERR_HIP.
 */
#ifndef GNNMB_H
#define GNNMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GNN_MAX_HOPS 8
#define GNN_MAX_GROUP 16 /* sub-batches per super-batch */

typedef int32_t gnn_status;
#define GNN_OK 0
#define GNN_ERR_INVALID_ARG (-1)  /* bad argument, or a duplicate seed (device) */
#define GNN_ERR_CAPACITY (-2)     /* an output or workspace buffer is too small */
#define GNN_ERR_OUT_OF_RANGE (-3) /* a node id outside [0, num_nodes) (device) */
#define GNN_ERR_HIP (-4)          /* a HIP runtime call failed */
#define GNN_ERR_UNSUPPORTED (-5)  /* a size or option the library does not handle */
#define GNN_ERR_INTERNAL (-6)     /* a device-side invariant failed (never expected) */

typedef void *gnn_stream; /* hipStream_t */

/* Flags for gnn_options.flags. */
#define GNN_SYNC 1u /* synchronise the stream at the end of the call and return the device status */
/* How gnn_minibatch relabels the sub-batches of a super-batch (results are identical; at most one
 * may be set; by default the library picks from the sizes):
 *   FULL:    each sub-batch gets a bitmap over all node ids (cheapest when num_nodes is small);
 *   COMPACT: the union of the sub-batches' node sets is relabelled once per hop and each sub-batch
 *            relabels positions in it (cheapest when num_nodes is large). */
#define GNN_SUPERBATCH_FULL 2u
#define GNN_SUPERBATCH_COMPACT 4u
/* How gnn_minibatch gathers X and takes the outermost mean (results are identical; at most one may
 * be set; BATCHED is the default):
 *   INTERLEAVED: per sub-batch, the gather then the mean, which reads X while it is still in the
 *                caches;
 *   BATCHED:     every sub-batch's gather in one launch, then the outermost means in one launch
 *                (one launch's start-up and drain instead of G; G times as many host-link reads
 *                in flight for a host-resident table).  With a table in device memory and no
 *                cache, the outermost means read the table rows and are taken once per node of
 *                the union of the sub-batches' last frontiers: the sub-batches share one seed, so
 *                a node's sampled neighbours and mean are the same in each, and the mean is
 *                stored to the node's row in every sub-batch that holds it. */
#define GNN_GATHER_INTERLEAVED 8u
/* How gnn_sample_khop and gnn_minibatch relabel a short id list (results are identical; at most one
 * may be set; by default the library picks from the sizes, on measured MI355X costs):
 *   SORT:   one workgroup sorts the list in LDS (radix sort, ballot compaction), when the list
 *           fits it (at most 16384 ids on gfx950) and no later kernel reads the bitmap;
 *   BITMAP: always the bitmap over the id range (mark, prefix scan, emit, rank). */
#define GNN_RELABEL_SORT 32u
#define GNN_RELABEL_BITMAP 64u
#define GNN_GATHER_BATCHED 16u
/* How the sampler picks each node's fanout smallest keys among its candidates (results are
 * identical): by default the candidates are ranked by their keys' high 32 bits, and a node whose
 * high words tie at the fanout-th place is ranked again by the full (key, position) order;
 * EXACT_RANK ranks every node by the full order (a check of the default). */
#define GNN_SAMPLE_EXACT_RANK 128u

/*
 * Graph in CSR form by destination: row v lists the sources u of the edges (u, v), which is the
 * neighbourhood N(v) = {u | (u, v) in E} of GARDEN Sec. II.A.  Borrowed, read-only.
 *   indptr: device memory.
 *   indices: device memory, or the device address of pinned host memory (gnn_host_mapped_pointer)
 *     for an adjacency larger than HBM, read in place by the sampler (GARDEN Sec. IV.B: adjacency
 *     served from host memory, with an adjacency cache in GPU memory).
 *   adj_off, adj_rows: an optional HBM adjacency cache (gnn_adjacency_cache_attach sets them;
 *     both NULL: none): row v's neighbours are adj_rows[adj_off[v] ..) when adj_off[v] >= 0.
 * Results do not depend on where the rows are read from.
 */
typedef struct gnn_graph {
    int64_t num_nodes;     /* N */
    int64_t num_edges;     /* |E| = indptr[N] */
    const void *indptr;    /* [N+1], int32 or int64 (indptr_bytes) */
    int32_t indptr_bytes;  /* 4 or 8 */
    const int32_t *indices; /* [num_edges] neighbour ids */
    const int64_t *adj_off;  /* [N] or NULL */
    const int32_t *adj_rows; /* cached rows or NULL */
} gnn_graph;

/*
 * The device address of pinned, mapped host memory (hipHostMalloc), for a graph's indices or a
 * feature table read in place.  Errors: GNN_ERR_INVALID_ARG, GNN_ERR_HIP (not mapped).
 */
gnn_status gnn_host_mapped_pointer(const void *host, const void **out_device);

/*
 * Adjacency cache (GARDEN Sec. IV.B, the adjacency part of the cache allocator): the rows of the
 * nodes hot_order[0..m) (device, distinct ids, hottest first) copied into HBM, m the largest
 * count whose rows hold at most max_entries neighbour ids in all.
 * The graph's indices may be host-resident.  Setup call: allocates adj_off [N] (int64) and the
 * rows with hipMalloc and synchronises.  *out_rows / *out_entries (may be NULL) receive the
 * numbers of rows and ids cached.
 * Errors: GNN_ERR_INVALID_ARG (bad graph, ids out of range or repeated), GNN_ERR_HIP.
 */
typedef struct gnn_adjacency_cache gnn_adjacency_cache;
gnn_status gnn_adjacency_cache_create(const gnn_graph *g, const int32_t *hot_order, int64_t n_hot,
                                      int64_t max_entries, gnn_adjacency_cache **out,
                                      int64_t *out_rows, int64_t *out_entries);
/* Points g->adj_off and g->adj_rows at the cache (same num_nodes), or clears them (c = NULL). */
gnn_status gnn_adjacency_cache_attach(const gnn_adjacency_cache *c, gnn_graph *g);
gnn_status gnn_adjacency_cache_destroy(gnn_adjacency_cache *c);

/* Worst-case element counts per hop, l = 1..K at index l-1. */
typedef struct gnn_caps {
    int32_t num_hops;                /* K */
    int32_t fanouts[GNN_MAX_HOPS];   /* k_l */
    int64_t n_seeds;                 /* |V_0| */
    int64_t frontier[GNN_MAX_HOPS];  /* |V_{l-1}| bound: destinations of block l */
    int64_t edges[GNN_MAX_HOPS];     /* |E_l| bound: sampled edges of block l */
    int64_t nodes[GNN_MAX_HOPS];     /* |V_l| bound: sources of block l */
} gnn_caps;

/*
 * Block l (GARDEN Sec. II.B, Fig. 1): destinations V_{l-1}, sources V_l.  Arrays sized by the caps
 * the caller allocated with (gnn_blocks.caps).
 */
typedef struct gnn_block {
    int32_t *indptr;  /* [frontier+1] destination i owns edges [indptr[i], indptr[i+1]) */
    int32_t *gid;     /* [edges] global id of each sampled neighbour, ascending CSR position
                         within a destination */
    int32_t *lid;     /* [edges] index of gid[e] in nodes (V_l) */
    int32_t *dst_lid; /* [frontier] index of destination i (V_{l-1}[i]) in nodes (V_l) */
    int32_t *nodes;   /* [nodes] V_l: ascending unique global ids of V_{l-1} and gid */
} gnn_block;

typedef struct gnn_blocks {
    gnn_caps caps;                 /* the sizes the arrays below were allocated with */
    gnn_block hop[GNN_MAX_HOPS];   /* hop[l-1] = block l */
    int64_t *counts;               /* [2K] device: counts[2(l-1)] = |E_l|, counts[2(l-1)+1] = |V_l| */
} gnn_blocks;

/* Tuning knobs; results never depend on them.  NULL means defaults (all fields 0). */
typedef struct gnn_options {
    int32_t group_max_deg; /* degree bound of the 16-lane class (default 256) */
    int32_t wave_max_deg;  /* degree bound of the one-wavefront class (default 16384); higher
                              degrees take one workgroup per node */
    uint32_t flags;        /* GNN_SYNC, GNN_SUPERBATCH_*, GNN_GATHER_* */
    int32_t reserved0;
    int64_t *d_hits;       /* gnn_minibatch: device int64 increased by the feature rows read from
                              the HBM caches (static or Dynamic-Cache); NULL: not counted */
    int32_t reserved[2];
} gnn_options;

/* Text for a status code (static storage). */
const char *gnn_status_string(gnn_status s);

/*
 * Seed of batch b of a run seeded with rng_seed (a deterministic per-batch seed; the pages fix no
 * generator, this is output b+1 of a SplitMix64 stream started at rng_seed).  Host function.
 */
uint64_t gnn_batch_seed(uint64_t rng_seed, uint64_t b);

/*
 * Worst-case sizes for K = num_hops hops from n_seeds seeds with the given fanouts (host array
 * [num_hops], each >= 1), on a graph of num_nodes nodes: frontier[0] = n_seeds,
 * edges[l] = frontier[l] * fanouts[l], nodes[l] = min(num_nodes, frontier[l] + edges[l]),
 * frontier[l+1] = nodes[l].  Host function, writes *out (host).  GNN_ERR_INVALID_ARG on bad input,
 * GNN_ERR_UNSUPPORTED if a size does not fit int32.
 */
gnn_status gnn_capacity(int64_t n_seeds, const int32_t *fanouts, int32_t num_hops,
                        int64_t num_nodes, gnn_caps *out);

/*
 * Workspace bytes for gnn_sample_khop / gnn_minibatch with these caps on a graph of num_nodes
 * nodes, for a super-batch of `group` sub-batches whose caps are all <= `caps` (group = 1 for a
 * plain batch).  Writes *out_bytes (host).
 */
gnn_status gnn_workspace_size(const gnn_caps *caps, int64_t num_nodes, int32_t group,
                              size_t *out_bytes);

/*
 * k-hop neighbour sampling and relabel for one batch (GARDEN Sec. II.B, Fig. 1; Sec. IV.C; the
 * draw is the bottom-k of per-edge SplitMix64 keys):
 *   for l = 1..K, destinations V_{l-1} (V_0 = seeds, caller order):
 *     destination i = node v keeps all of row v if deg(v) <= fanouts[l-1] (a "full node"),
 *     otherwise the fanouts[l-1] positions j with the smallest (key(l, v, j), j), where
 *     key(l, v, j) = mix64(s_{l,v} + G*(j+1)), s_{l,v} = mix64(mix64(seed64 + G*l) ^ v),
 *     G = 0x9E3779B97F4A7C15 and mix64 is the SplitMix64 output function;
 *     the chosen neighbours are listed in ascending position;
 *     V_l = ascending unique of V_{l-1} and the sampled ids; lid / dst_lid are ranks in V_l.
 * seeds: [n_seeds] distinct ids in [0, N).  fanouts: host [num_hops].  out: host struct whose
 * device arrays hold at least out->caps; out->caps.n_seeds must equal n_seeds.
 * ws: device workspace of ws_bytes >= gnn_workspace_size(&out->caps, N, 1).
 * Device errors: GNN_ERR_OUT_OF_RANGE (seed outside [0,N)), GNN_ERR_INVALID_ARG (duplicate
 * seed), GNN_ERR_CAPACITY (a count exceeds out->caps).
 */
gnn_status gnn_sample_khop(const gnn_graph *g, const int32_t *seeds, int64_t n_seeds,
                           const int32_t *fanouts, int32_t num_hops, uint64_t seed64,
                           gnn_blocks *out, void *ws, size_t ws_bytes,
                           const gnn_options *opt, gnn_stream stream);

/*
 * Sort-unique relabel of two id lists (FastGL's id remapping; the deduplication of GARDEN Sec. IV.D, Alg. 1):
 *   uniq = ascending unique of keep[0..n_keep) and add[0..n_add);
 *   keep_lid[i] = index of keep[i] in uniq, add_lid[e] = index of add[e] in uniq.
 * Every id must lie in [0, id_bound).  n_add is the length of `add`, or, if d_n_add is not NULL,
 * an upper bound and *d_n_add (device int64) the actual length.  *d_n_uniq (device int64)
 * receives |uniq|.  uniq has room for cap_uniq ids.  ws: device workspace of ws_bytes >=
 * gnn_relabel_workspace_size(id_bound).
 * Device errors: GNN_ERR_OUT_OF_RANGE, GNN_ERR_CAPACITY.
 */
gnn_status gnn_unique_relabel(const int32_t *keep, int64_t n_keep, const int32_t *add,
                              const int64_t *d_n_add, int64_t n_add, int64_t id_bound,
                              int32_t *uniq, int64_t cap_uniq, int64_t *d_n_uniq,
                              int32_t *add_lid, int32_t *keep_lid, void *ws, size_t ws_bytes,
                              gnn_stream stream);

gnn_status gnn_relabel_workspace_size(int64_t id_bound, size_t *out_bytes);

/*
 * gnn_unique_relabel without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same inputs, outputs, results and device errors as gnn_unique_relabel;
 * the first device error (or GNN_OK) goes to *d_status (device int32, cleared by the call; may be
 * NULL, then device errors are dropped).
 * Scratch: a fixed array of GNN_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held until
 * the process ends and shared by every call on that GPU; it keeps the last call's contents, and
 * the call clears what must start at zero.  Calls that overlap on one GPU (other streams, other
 * host threads) race on it and must be serialised by the caller.
 * Host errors: GNN_ERR_UNSUPPORTED when id_bound > GNN_NOALLOC_MAX_IDS (nothing enqueued); the
 * argument checks of gnn_unique_relabel otherwise.
 */
#define GNN_NOALLOC_MAX_IDS 67108864          /* 2^26 */
#define GNN_NOALLOC_SCRATCH_BYTES 25231360    /* 24 MiB + 64 KiB */
gnn_status gnn_unique_relabel_noalloc(const int32_t *keep, int64_t n_keep, const int32_t *add,
                                      const int64_t *d_n_add, int64_t n_add, int64_t id_bound,
                                      int32_t *uniq, int64_t cap_uniq, int64_t *d_n_uniq,
                                      int32_t *add_lid, int32_t *keep_lid, int32_t *d_status,
                                      gnn_stream stream);

/*
 * Feature store: the table of node features (fp32, row-major, row stride ld >= d) in HBM, or in
 * pinned host memory read zero-copy (LEO Sec. 2.3; GARDEN Sec. II.B misses served from pinned
 * host memory), optionally with an HBM hot-row cache (GARDEN Sec. IV.B) holding the rows
 * hot_order[0..cache_rows).
 *   table: device pointer, or (table_on_host = 1) a host pointer allocated pinned and mapped
 *     (hipHostMalloc); borrowed for the store's lifetime.
 *   hot_order: device [cache_rows] distinct ids; may be NULL when cache_rows = 0.
 * Setup call: allocates the cache and the id->slot map with hipMalloc and synchronises.
 * Errors: GNN_ERR_INVALID_ARG, GNN_ERR_HIP (allocation or host mapping failed).
 */
typedef struct gnn_feature_store gnn_feature_store;
gnn_status gnn_feature_store_create(const float *table, int32_t table_on_host, int64_t num_nodes,
                                    int64_t d, int64_t ld, int64_t cache_rows,
                                    const int32_t *hot_order, gnn_feature_store **out);
gnn_status gnn_feature_store_destroy(gnn_feature_store *fs);

/*
 * Dynamic-Cache (GARDEN Sec. IV.B, eq. (5)-(6)): a bounded secondary HBM cache of k_dyn rows, after
 * the static cache's rows, for residual hot rows, i.e. rows that the static cache misses and that
 * recur.  Every gather from the store (gnn_gather_features, and gnn_minibatch once per
 * sub-batch) is one mini-batch t: for each requested row of a node v outside the static cache,
 * Score(v, t) = gamma * Score(v, t-1) + (occurrences of v among the requested rows), eq. (5);
 * every other node's score only decays.  A refresh, once at least t_update mini-batches have been
 * observed since the last one, makes the cache hold the k_dyn nodes of highest score, eq. (6)
 * (ties: the smaller id; only nodes with a positive score; fewer than k_dyn if fewer have one).
 * After max_refreshes refreshes (0: no limit) the cache is frozen and nothing more is observed.
 * Residency: a refresh reserves a row for each node it takes in but copies nothing; the next
 * gather that reads the node's row from the table (a miss) also writes it to the reserved row, and
 * the next refresh due (or, frozen, the next gnn_dyn_cache_update after t_update more
 * mini-batches) makes such rows resident, so a member's row is read from the cache from then on.
 * Results never change: a gather returns the table's rows whichever cache holds them.
 *   gamma: 0 < gamma < 1; k_dyn >= 1 and cache_rows + k_dyn <= num_nodes; t_update >= 1.
 *   flags: GNN_DYN_AUTO -- the gather call that completes an interval refreshes at its end, on its
 *     own stream; else only gnn_dyn_cache_update refreshes.
 * Memory: k_dyn * ld floats of cache and 13 bytes per row of bookkeeping, and 20.25 bytes per
 * node (score, candidate list and key, touched and member bitmaps); the cache is re-allocated
 * (static rows copied).  Setup call: allocates, synchronises the device, and must not overlap
 * any use of the store.
 * Ordering: a refresh rewrites cache rows and slots on its stream; no gather from the store may
 * run concurrently with it on another stream (join the streams around gnn_dyn_cache_update).
 * Observations from several streams may overlap one another.  Calls that use one store are made
 * from one host thread at a time.
 * Errors: GNN_ERR_INVALID_ARG (bad parameters, or already enabled), GNN_ERR_HIP (allocation).
 */
#define GNN_DYN_AUTO 1u
typedef struct gnn_dyn_cache_params {
    double gamma;
    int64_t k_dyn;
    int32_t t_update;
    int32_t max_refreshes;
    uint32_t flags;
} gnn_dyn_cache_params;
gnn_status gnn_feature_store_enable_dynamic(gnn_feature_store *fs, const gnn_dyn_cache_params *p);

/*
 * Refresh of the Dynamic-Cache on `stream` if one is due (see above); *refreshed (host, may be
 * NULL) = 1 if it ran.  Enqueues only; device errors (GNN_ERR_INTERNAL, never expected) go to
 * *d_status when not NULL.  Errors: GNN_ERR_INVALID_ARG (no Dynamic-Cache).
 */
gnn_status gnn_dyn_cache_update(const gnn_feature_store *fs, int32_t *refreshed, int32_t *d_status,
                                gnn_stream stream);

/*
 * Dynamic-Cache counters (host struct).  Synchronises the device for the device-side counts
 * (members, and the last refresh's candidates, admissions and evictions).
 */
typedef struct gnn_dyn_cache_info {
    int64_t steps;           /* mini-batches gathered from the store since enabled */
    int64_t since_refresh;   /* of which after the last refresh */
    int32_t refreshes;
    int32_t due;             /* a refresh would run now */
    int32_t frozen;          /* max_refreshes reached: no more observation */
    int32_t reserved;
    int64_t members;
    int64_t last_candidates;
    int64_t last_admitted;
    int64_t last_evicted;
    int64_t resident;        /* members whose row is filled and used */
    int64_t last_published;  /* rows the last refresh made resident */
} gnn_dyn_cache_info;
gnn_status gnn_dyn_cache_query(const gnn_feature_store *fs, gnn_dyn_cache_info *out);

/*
 * Inspection on `stream`: score[v] = Score(v, t) after the last observed mini-batch t (device
 * double [num_nodes], or NULL) and member[v] = 1 if v is a member whose row is resident, 2 if a
 * member whose row is not filled yet, else 0 (device uint8 [num_nodes], or NULL).
 * Errors: GNN_ERR_INVALID_ARG (no Dynamic-Cache).
 */
gnn_status gnn_dyn_cache_state(const gnn_feature_store *fs, double *score, uint8_t *member,
                               gnn_stream stream);

/*
 * Feature-row gather (GARDEN Sec. II.B "Nfeat-selecting"; LEO Sec. 2.2 feature extraction):
 *   out[i, 0..d) = table row ids[i], bit for bit, for i < n.
 * n is the number of ids, or, if d_n is not NULL, an upper bound and *d_n (device int64) the
 * actual number.  out: device [n, ld_out], ld_out >= d.  With a cache, a row is read from the
 * HBM cache when cached, else from the table; *d_hits (device int64, may be NULL) is increased by
 * the number of cached rows read.
 * Device errors: GNN_ERR_OUT_OF_RANGE (written to *d_status if not NULL).
 */
gnn_status gnn_gather_features(const gnn_feature_store *fs, const int32_t *ids,
                               const int64_t *d_n, int64_t n, float *out, int64_t ld_out,
                               int64_t *d_hits, int32_t *d_status, gnn_stream stream);

/*
 * Match (FastGL: A GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large
 * Scale, "The idea": a new batch's nodes are intersected with the batch still on the GPU and only
 * the remainder is shipped; "What it costs": only the immediately previous batch is used):
 * gnn_gather_features with the previous batch's gathered rows as a second source.
 *   out[i, 0..d) = table row ids[i], bit for bit, for i < n: exactly gnn_gather_features' result.
 *   A row whose id is prev_ids[p] is copied from prev_x row p instead of being read from the
 *   store; match[i] receives p, or -1 for a row read from the store.
 *   prev_ids: device [prev_n] strictly ascending ids (the node lists V_l of gnn_sample_khop and
 *     gnn_minibatch are), *d_prev_n (device int64, may be NULL) the actual count; prev_x: device
 *     [prev_n, ld_prev], row p holding the features of prev_ids[p] (the previous batch's X).
 *   ids need not be sorted; n and d_n as in gnn_gather_features; match: device int32 [n];
 *   d_matched (device int64, may be NULL) is increased by the number of rows copied from prev_x;
 *   d_hits as in gnn_gather_features (rows read from the HBM cache).  prev_x must not overlap out.
 * Errors: GNN_ERR_UNSUPPORTED with a Dynamic-Cache (a copied row is no request to the store) or
 * when the store's cache rows or prev_n reach 2^30; device errors as gnn_gather_features.
 */
gnn_status gnn_gather_features_match(const gnn_feature_store *fs, const int32_t *ids,
                                     const int64_t *d_n, int64_t n, float *out, int64_t ld_out,
                                     const int32_t *prev_ids, const int64_t *d_prev_n,
                                     int64_t prev_n, const float *prev_x, int64_t ld_prev,
                                     int32_t *match, int64_t *d_matched, int64_t *d_hits,
                                     int32_t *d_status, gnn_stream stream);

/*
 * Greedy Reorder, its overlap matrix (FastGL, "What it costs": a full pairwise overlap matrix for
 * each group of sampled batches): overlap[a * B + b] = |L_a ∩ L_b| for a != b and |L_a| for
 * a = b, for B node lists L_a = ids[a][0 .. count_a), each strictly ascending; count_a = *d_n[a]
 * (device int64) when d_n[a] is not NULL, else n[a] (n[a] is always the bound).  ids, d_n, n:
 * host arrays of B entries (d_n may be NULL: every count is n[a]).  overlap: device int64 [B * B].
 * 1 <= B <= GNN_MAX_GROUP.  Enqueued on `stream`; no host synchronisation.
 */
gnn_status gnn_batch_overlap(const int32_t *const *ids, const int64_t *const *d_n, const int64_t *n,
                             int32_t B, int64_t *overlap, gnn_stream stream);

/*
 * Greedy Reorder, the order (FastGL, "The idea": each batch follows the batch it shares the most
 * with; "What it costs": nearest-overlap-first, not optimal).  Host code: order[0] = first, and
 * each next batch is the one not yet placed with the largest overlap[last * B + b] (ties: the
 * smaller b).  overlap: host int64 [B * B] (from gnn_batch_overlap); order: host int32 [B].
 * Errors: GNN_ERR_INVALID_ARG (B < 1, first outside [0, B), NULL arrays).
 */
gnn_status gnn_greedy_order(const int64_t *overlap, int32_t B, int32_t first, int32_t *order);

/*
 * Mean aggregation of one block (GARDEN Sec. II.A eq. (1) with AGGREGATE = mean):
 *   out[i, 0..d) = (1/c_i) * sum_{e in [indptr[i], indptr[i+1])} src[lid[e], 0..d),
 *   c_i = indptr[i+1] - indptr[i]; the zero vector when c_i = 0.  fp32 accumulation in
 *   ascending e, then one division by c_i.
 * n_dst is the number of destinations, or, if d_n_dst is not NULL, an upper bound and *d_n_dst
 * (device int64) the actual number.  indptr: [n_dst+1]; lid: [n_lid] (edge offsets are clamped
 * to n_lid); src: [n_src, ld_src]; out: [n_dst, ld_out].
 * Device errors: GNN_ERR_INTERNAL if a lid lies outside [0, n_src) (written to *d_status if not
 * NULL; that edge then reads row 0).
 */
gnn_status gnn_mean_aggregate(const int32_t *indptr, const int32_t *lid, int64_t n_lid,
                              const int64_t *d_n_dst, int64_t n_dst, const float *src,
                              int64_t ld_src, int64_t n_src, int64_t d, float *out,
                              int64_t ld_out, int32_t *d_status, gnn_stream stream);

/*
 * One GraphSAGE-mean layer over one block (GARDEN Sec. II.A eq. (1)-(2): AGGREGATE = the mean
 * over the sampled neighbours, UPDATE = one dense layer on the node's own previous state
 * concatenated with that mean; the GraphSAGE model of GARDEN Sec. VI.A):
 *   agg[i, 0..d) = the mean of gnn_mean_aggregate over the block (same arithmetic, bit for bit),
 *   out[i, n] = act( sum_{k<d} src[dst_lid[i], k] * W[k, n] + sum_{k<d} agg[i, k] * W[d+k, n]
 *                    + bias[n] ),   act(v) = (relu && v < 0) ? 0 : v.
 * The product runs on the matrix cores in fp32 (fp32 inputs and accumulation; the summation
 * order is the kernel's, not a sequential one).
 * indptr, lid, n_lid, d_n_dst, n_dst, src, ld_src, n_src, d: as for gnn_mean_aggregate.
 * dst_lid: device [n_dst], each destination's row in src (a block's dst_lid; src is then the
 *   block's source node features, e.g. X for the outermost block).
 * W: device fp32, row-major [2d, d_out] (the first d rows multiply the node's own row);
 * bias: device [d_out] or NULL; 1 <= d_out <= 65536.
 * agg: device [n_dst, ld_agg], ld_agg >= d, receives the means (caller-owned; also an output).
 * out: device [n_dst, ld_out], ld_out >= d_out.
 * Device errors: GNN_ERR_INTERNAL if a lid or a dst_lid lies outside [0, n_src) (written to
 * *d_status if not NULL; that row then reads row 0).
 */
gnn_status gnn_sage_layer(const int32_t *indptr, const int32_t *lid, int64_t n_lid,
                          const int32_t *dst_lid, const int64_t *d_n_dst, int64_t n_dst,
                          const float *src, int64_t ld_src, int64_t n_src, int64_t d,
                          const float *W, const float *bias, int64_t d_out, int32_t relu,
                          float *agg, int64_t ld_agg, float *out, int64_t ld_out,
                          int32_t *d_status, gnn_stream stream);

/*
 * The UPDATE of gnn_sage_layer alone, for means computed elsewhere (for instance h_{l-1} of
 * gnn_minibatch, which holds the means of block l):
 *   out[i, n] = act( sum_{k<d} src[dst_lid[i], k] * W[k, n] + sum_{k<d} agg[i, k] * W[d+k, n]
 *                    + bias[n] ),   act(v) = (relu && v < 0) ? 0 : v,
 * for i < n_dst (or < *d_n_dst when d_n_dst is not NULL).  Arguments as for gnn_sage_layer; agg is
 * read, not written.  fp32 matrix-core products and accumulation.
 * Device errors: GNN_ERR_INTERNAL if a dst_lid lies outside [0, n_src).
 */
gnn_status gnn_sage_update(const int32_t *dst_lid, const int64_t *d_n_dst, int64_t n_dst,
                           const float *src, int64_t ld_src, int64_t n_src, int64_t d,
                           const float *agg, int64_t ld_agg, const float *W, const float *bias,
                           int64_t d_out, int32_t relu, float *out, int64_t ld_out,
                           int32_t *d_status, gnn_stream stream);

/*
 * Outputs of one (sub-)batch of gnn_minibatch.
 *   x    = X = h_K: [caps.nodes[K-1], ld_h], row i = feature row of V_K[i];
 *   h[l] = h_l for l = 0..K-1: h_0 is [n_seeds, ld_h] (seed order), h_l is [caps.nodes[l-1],
 *          ld_h] (V_l order).
 */
typedef struct gnn_minibatch_out {
    gnn_blocks blocks;
    float *x;
    float *h[GNN_MAX_HOPS];
    int64_t ld_h;
} gnn_minibatch_out;

/*
 * One mini-batch, or a super-batch of `group` sub-batches (GARDEN Sec. IV.D, Alg. 1), end to end:
 * sampling and relabel for every hop (as gnn_sample_khop), the feature gather of V_K into x, then
 * mean aggregation from h_K = x down to h_0 (UPDATE is the identity; no learnable weights).
 *   seeds: device, the sub-batches' seeds concatenated; batch_ptr: host [group+1] offsets.
 *   All sub-batches use the one seed64, so a node shared by two sub-batches at the same hop has
 *   the same sample in both; each sub-batch's outputs equal a separate run with that seed64.
 *   outs: host [group]; outs[g].blocks.caps.n_seeds = batch_ptr[g+1] - batch_ptr[g].
 *   ws: ws_bytes >= gnn_workspace_size(caps >= every sub-batch's caps, N, group).
 *   timer: NULL, or a timer that records the stage boundaries of this call (gnn_timer_*).
 * Errors: as gnn_sample_khop and gnn_gather_features; GNN_ERR_UNSUPPORTED (host, nothing
 * enqueued) when group > 1 and the super-batch's union block could exceed int32 offsets:
 * max over hops of min(N, group * caps.frontier[l]) * fanouts[l] > 2^31 - 1.
 */
typedef struct gnn_timer gnn_timer;
gnn_status gnn_minibatch(const gnn_graph *g, const gnn_feature_store *fs, const int32_t *seeds,
                         const int64_t *batch_ptr, int32_t group, const int32_t *fanouts,
                         int32_t num_hops, uint64_t seed64, gnn_minibatch_out *outs, void *ws,
                         size_t ws_bytes, const gnn_options *opt, gnn_stream stream,
                         gnn_timer *timer);

/*
 * Device status word of a workspace: synchronises `stream`, returns the first device error
 * recorded by the last call that used ws (GNN_OK if none) in *out (host).
 */
gnn_status gnn_read_device_status(const void *ws, gnn_stream stream, gnn_status *out);

/*
 * Stage timer (HIP events recorded on the call's stream).  A gnn_minibatch call given a timer
 * records one record: events at the call start, at the end of sampling and relabel (all hops),
 * after each sub-batch's feature gather and after its outermost-block mean (these two kernels run
 * back to back per sub-batch), at the end of the call, and around each hop's sampling kernel.
 * gnn_timer_elapsed synchronises on the recorded events and writes GNN_TIMER_STAGES durations in
 * milliseconds per record to ms (host [n_records*GNN_TIMER_STAGES]): sampling+relabel, the
 * gather kernels (summed over sub-batches), the outermost-block mean kernels (summed), the
 * remaining mean blocks, and the sampling kernels alone (summed over hops; part of the first).
 * gnn_timer_reset rewinds to record 0.  Each event costs a few microseconds of stream time.
 */
#define GNN_TIMER_STAGES 5
gnn_status gnn_timer_create(int32_t n_records, gnn_timer **out);
gnn_status gnn_timer_destroy(gnn_timer *t);
gnn_status gnn_timer_reset(gnn_timer *t);
gnn_status gnn_timer_elapsed(gnn_timer *t, int32_t *n_records, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* GNNMB_H */
