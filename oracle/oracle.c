/*
 * oracle.c -- plain, slow, single-threaded CPU reference of the sampling-based GNN mini-batch
 * path: k-hop neighbour sampling, sort-unique relabel, feature-row gather and mean aggregation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no code with the GPU library and includes none of
 * its headers.
 *
 * Sources (the pages are cited by title and section):
 *  - GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
 *    Co-Design, Sec. II.A eq. (1): a node aggregates over N(u) = {v | (v,u) in E}; Sec. II.B and
 *    Fig. 1: layer-wise sampling from the seeds V_0 outwards, each layer's destination set is the
 *    previous node set; Sec. IV.C: a node whose degree is at most the fanout keeps its whole
 *    neighbour list ("full node"), others draw a fixed number of neighbours uniformly, without
 *    reweighting.
 *  - The pages give no random number generator.  The draw is made deterministic with the
 *    SplitMix64 output function (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *    generators", OOPSLA 2014): the keys of node v at hop l are the outputs of a SplitMix64
 *    stream whose state starts at s(l,v); the k positions with the smallest (key, position) are
 *    chosen, which is a uniform k-subset without replacement (bottom-k sampling).
 *
 * Floating point: the mean accumulates in double, in ascending edge order, divides by the count
 * and rounds once to float.
 *
 * The GraphSAGE-mean layer (orc_sage_layer) follows GARDEN Sec. II.A eq. (1)-(2): AGGREGATE is
 * the mean over the sampled neighbours, UPDATE a dense layer on the concatenation of the node's
 * own previous state and that mean, then a ReLU (the layer GraphSAGE defines and GARDEN Sec. VI.A
 * evaluates).  It is computed in double throughout and is not rounded to float.
 *
 * The Dynamic-Cache (orc_dyn_ewma_step, orc_dyn_topk) follows GARDEN Sec. IV.B eq. (5)-(6): an
 * exponentially weighted count of each node's residual accesses, in double, and the K nodes of
 * highest count.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_CAPACITY (-2)
#define ORC_ERR_RANGE (-3)
#define ORC_ERR_NOMEM (-7)

/* SplitMix64 increment: the odd integer nearest 2^64 / golden ratio. */
static const uint64_t ORC_GAMMA = 0x9E3779B97F4A7C15ULL;

/* SplitMix64 output function. */
uint64_t orc_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* One step of a SplitMix64 generator: advance the state by GAMMA and return its output. */
uint64_t orc_splitmix_next(uint64_t *state) {
    *state += ORC_GAMMA;
    return orc_mix64(*state);
}

/* Seed of batch b of a run seeded with rng_seed: output b+1 of the stream started at rng_seed. */
uint64_t orc_batch_seed(uint64_t rng_seed, uint64_t b) {
    return orc_mix64(rng_seed + ORC_GAMMA * (b + 1));
}

/* Seed of hop l (l >= 1) of a batch whose seed is seed64. */
uint64_t orc_hop_seed(uint64_t seed64, int32_t hop) {
    return orc_mix64(seed64 + ORC_GAMMA * (uint64_t)(uint32_t)hop);
}

/* Seed of node v at a hop whose seed is hop_seed. */
uint64_t orc_node_seed(uint64_t hop_seed, int32_t v) {
    return orc_mix64(hop_seed ^ (uint64_t)(uint32_t)v);
}

/* Key of the neighbour at position j (0-based) of a node whose seed is node_seed: output j+1 of
 * the SplitMix64 stream whose state starts at node_seed. */
uint64_t orc_edge_key(uint64_t node_seed, int64_t j) {
    return orc_mix64(node_seed + ORC_GAMMA * (uint64_t)(j + 1));
}

static int64_t row_start(const void *indptr, int ib, int64_t v) {
    return ib == 8 ? ((const int64_t *)indptr)[v] : (int64_t)((const int32_t *)indptr)[v];
}

typedef struct {
    uint64_t key;
    int64_t pos;
} orc_keypos;

static int cmp_keypos(const void *a, const void *b) {
    const orc_keypos *x = (const orc_keypos *)a, *y = (const orc_keypos *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

static int cmp_i64(const void *a, const void *b) {
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

static int cmp_i32(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Positions chosen at one node: all of [0, deg) if deg <= k, else the k positions with the
 * smallest (key, position), listed in ascending position.  Writes min(deg, k) positions to pos.
 */
int orc_select_positions(uint64_t node_seed, int64_t deg, int32_t k, int64_t *pos) {
    if (deg < 0 || k < 1) return ORC_ERR_ARG;
    if (deg <= k) {
        for (int64_t j = 0; j < deg; ++j) pos[j] = j;
        return ORC_OK;
    }
    orc_keypos *all = (orc_keypos *)malloc((size_t)deg * sizeof(orc_keypos));
    if (!all) return ORC_ERR_NOMEM;
    for (int64_t j = 0; j < deg; ++j) {
        all[j].key = orc_edge_key(node_seed, j);
        all[j].pos = j;
    }
    qsort(all, (size_t)deg, sizeof(orc_keypos), cmp_keypos);
    for (int32_t r = 0; r < k; ++r) pos[r] = all[r].pos;
    free(all);
    qsort(pos, (size_t)k, sizeof(int64_t), cmp_i64);
    return ORC_OK;
}

/*
 * One sampling hop.  Destinations are frontier[0..F); destination i is node v = frontier[i].
 * blk_indptr[i+1] - blk_indptr[i] = min(deg(v), k); blk_gid lists the sampled neighbours' global
 * ids, destination by destination, each in ascending CSR position.
 */
int orc_sample_hop(const void *indptr, int32_t ib, const int32_t *indices, int64_t num_nodes,
                   const int32_t *frontier, int64_t F, int32_t k, uint64_t seed64, int32_t hop,
                   int32_t *blk_indptr, int32_t *blk_gid, int64_t cap_edges, int64_t *n_edges) {
    if ((ib != 4 && ib != 8) || k < 1 || F < 0 || hop < 1) return ORC_ERR_ARG;
    const uint64_t hs = orc_hop_seed(seed64, hop);
    int64_t *pos = (int64_t *)malloc(((size_t)k + 1) * sizeof(int64_t));
    if (!pos) return ORC_ERR_NOMEM;
    int64_t e = 0;
    blk_indptr[0] = 0;
    for (int64_t i = 0; i < F; ++i) {
        const int32_t v = frontier[i];
        if (v < 0 || v >= num_nodes) { free(pos); return ORC_ERR_RANGE; }
        const int64_t start = row_start(indptr, ib, v);
        const int64_t deg = row_start(indptr, ib, (int64_t)v + 1) - start;
        const int64_t c = deg <= k ? deg : k;
        if (e + c > cap_edges) { free(pos); return ORC_ERR_CAPACITY; }
        int rc = orc_select_positions(orc_node_seed(hs, v), deg, k, pos);
        if (rc != ORC_OK) { free(pos); return rc; }
        for (int64_t r = 0; r < c; ++r) blk_gid[e + r] = indices[start + pos[r]];
        e += c;
        blk_indptr[i + 1] = (int32_t)e;
    }
    free(pos);
    *n_edges = e;
    return ORC_OK;
}

static int64_t lower_bound_i32(const int32_t *a, int64_t n, int32_t x) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

/*
 * Relabel: uniq = ascending unique of (frontier ++ gid); blk_lid[e] is the index of gid[e] in
 * uniq and dst_lid[i] the index of frontier[i] (both exist, since both lists are in the union).
 */
int orc_relabel(const int32_t *frontier, int64_t F, const int32_t *gid, int64_t E,
                int32_t *uniq, int64_t cap_uniq, int64_t *n_uniq, int32_t *blk_lid,
                int32_t *dst_lid) {
    if (F < 0 || E < 0) return ORC_ERR_ARG;
    int64_t n = F + E;
    int32_t *all = (int32_t *)malloc(((size_t)n + 1) * sizeof(int32_t));
    if (!all) return ORC_ERR_NOMEM;
    memcpy(all, frontier, (size_t)F * sizeof(int32_t));
    memcpy(all + F, gid, (size_t)E * sizeof(int32_t));
    qsort(all, (size_t)n, sizeof(int32_t), cmp_i32);
    int64_t u = 0;
    for (int64_t t = 0; t < n; ++t)
        if (t == 0 || all[t] != all[t - 1]) all[u++] = all[t];
    if (u > cap_uniq) { free(all); return ORC_ERR_CAPACITY; }
    memcpy(uniq, all, (size_t)u * sizeof(int32_t));
    free(all);
    for (int64_t e = 0; e < E; ++e) blk_lid[e] = (int32_t)lower_bound_i32(uniq, u, gid[e]);
    for (int64_t i = 0; i < F; ++i) dst_lid[i] = (int32_t)lower_bound_i32(uniq, u, frontier[i]);
    *n_uniq = u;
    return ORC_OK;
}

/* Gather: out row i = table row ids[i], d floats copied byte for byte. */
int orc_gather(const float *table, int64_t ld, int64_t d, int64_t num_rows, const int32_t *ids,
               int64_t n, float *out, int64_t ld_out) {
    if (d < 0 || ld < d || ld_out < d) return ORC_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= num_rows) return ORC_ERR_RANGE;
        memcpy(out + i * ld_out, table + (int64_t)ids[i] * ld, (size_t)d * sizeof(float));
    }
    return ORC_OK;
}

/*
 * Mean aggregation of one block: out row i = (1/c) * sum of src rows lid[e] for e in
 * [indptr[i], indptr[i+1]), c = indptr[i+1] - indptr[i]; the zero vector when c = 0.
 */
int orc_mean(const int32_t *indptr, const int32_t *lid, int64_t n_dst, const float *src,
             int64_t ld_src, int64_t n_src, int64_t d, float *out, int64_t ld_out) {
    if (d < 0 || ld_src < d || ld_out < d) return ORC_ERR_ARG;
    double *acc = (double *)malloc(((size_t)d + 1) * sizeof(double));
    if (!acc) return ORC_ERR_NOMEM;
    for (int64_t i = 0; i < n_dst; ++i) {
        const int64_t e0 = indptr[i], e1 = indptr[i + 1];
        for (int64_t t = 0; t < d; ++t) acc[t] = 0.0;
        for (int64_t e = e0; e < e1; ++e) {
            const int64_t u = lid[e];
            if (u < 0 || u >= n_src) { free(acc); return ORC_ERR_RANGE; }
            const float *row = src + u * ld_src;
            for (int64_t t = 0; t < d; ++t) acc[t] += (double)row[t];
        }
        const int64_t c = e1 - e0;
        float *o = out + i * ld_out;
        for (int64_t t = 0; t < d; ++t) o[t] = c > 0 ? (float)(acc[t] / (double)c) : 0.0f;
    }
    free(acc);
    return ORC_OK;
}

/*
 * One GraphSAGE-mean layer over one block.  For destination i with sampled edges
 * e in [indptr[i], indptr[i+1]) (count c):
 *   a = [ src row dst_lid[i]  ||  (1/c) * sum_e src row lid[e]  (0 when c = 0) ]   (2d values),
 *   out[i][n] = sum_{k < 2d} a[k] * W[k][n] + (bias ? bias[n] : 0),  then max(0, .) if relu.
 * W is row-major [2d][d_out].  Everything is double; out is [n_dst][d_out] double.  When
 * scale is not NULL it receives sum_k |a[k]| |W[k][n]| + |bias[n]| (the magnitude an error bound
 * of a float evaluation scales with).
 */
int orc_sage_layer(const int32_t *indptr, const int32_t *lid, const int32_t *dst_lid,
                   int64_t n_dst, const float *src, int64_t ld_src, int64_t n_src, int64_t d,
                   const float *W, const float *bias, int64_t d_out, int32_t relu, double *out,
                   double *scale) {
    if (d < 0 || ld_src < d || d_out < 0 || n_dst < 0) return ORC_ERR_ARG;
    const int64_t K = 2 * d;
    double *a = (double *)malloc(((size_t)K + 1) * sizeof(double));
    if (!a) return ORC_ERR_NOMEM;
    for (int64_t i = 0; i < n_dst; ++i) {
        const int64_t self = dst_lid[i];
        if (self < 0 || self >= n_src) { free(a); return ORC_ERR_RANGE; }
        for (int64_t t = 0; t < d; ++t) a[t] = (double)src[self * ld_src + t];
        for (int64_t t = 0; t < d; ++t) a[d + t] = 0.0;
        const int64_t e0 = indptr[i], e1 = indptr[i + 1];
        for (int64_t e = e0; e < e1; ++e) {
            const int64_t u = lid[e];
            if (u < 0 || u >= n_src) { free(a); return ORC_ERR_RANGE; }
            for (int64_t t = 0; t < d; ++t) a[d + t] += (double)src[u * ld_src + t];
        }
        if (e1 > e0)
            for (int64_t t = 0; t < d; ++t) a[d + t] /= (double)(e1 - e0);
        for (int64_t n = 0; n < d_out; ++n) {
            double acc = bias ? (double)bias[n] : 0.0;
            double mag = bias ? (double)(bias[n] < 0 ? -bias[n] : bias[n]) : 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double w = (double)W[k * d_out + n];
                acc += a[k] * w;
                mag += (a[k] < 0 ? -a[k] : a[k]) * (w < 0 ? -w : w);
            }
            out[i * d_out + n] = (relu && acc < 0.0) ? 0.0 : acc;
            if (scale) scale[i * d_out + n] = mag;
        }
    }
    free(a);
    return ORC_OK;
}

/*
 * Dynamic-Cache hotness (GARDEN Sec. IV.B, eq. (5)) for one mini-batch t:
 *   Score(v, t) = gamma * Score(v, t-1) + (number of i in B_t with i = v),
 * where B_t is read as the mini-batch's requested feature rows that the static cache does not
 * hold (the residual accesses the Dynamic-Cache is for); ids[0..n) are the requested rows, with
 * repeats, and is_static[v] != 0 marks static-cache rows (NULL: no static cache).  Every score is
 * scaled by gamma first, then 1 is added once per occurrence.
 */
int orc_dyn_ewma_step(double *score, int64_t num_nodes, double gamma, const int32_t *ids,
                      int64_t n, const uint8_t *is_static) {
    if (num_nodes < 0 || n < 0 || !(gamma > 0.0 && gamma < 1.0)) return ORC_ERR_ARG;
    for (int64_t v = 0; v < num_nodes; ++v) score[v] = gamma * score[v];
    for (int64_t i = 0; i < n; ++i) {
        const int32_t v = ids[i];
        if (v < 0 || v >= num_nodes) return ORC_ERR_RANGE;
        if (is_static && is_static[v]) continue;
        score[v] += 1.0;
    }
    return ORC_OK;
}

typedef struct {
    double score;
    int32_t id;
} orc_scored;

/* Larger score first; equal scores: smaller id first. */
static int cmp_scored(const void *a, const void *b) {
    const orc_scored *x = (const orc_scored *)a, *y = (const orc_scored *)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    return (x->id > y->id) - (x->id < y->id);
}

/*
 * Dynamic-Cache contents (GARDEN Sec. IV.B, eq. (6)): TopK of the scores with K = k.  Only nodes
 * with a positive score take part (a node never requested has nothing to cache); among equal
 * scores the smaller id comes first.  Writes the chosen ids in ascending order to out (room for
 * min(k, num_nodes)) and returns their count (negative: error).
 */
int64_t orc_dyn_topk(const double *score, int64_t num_nodes, int64_t k, int32_t *out) {
    if (num_nodes < 0 || k < 0) return ORC_ERR_ARG;
    int64_t m = 0;
    for (int64_t v = 0; v < num_nodes; ++v) m += score[v] > 0.0;
    orc_scored *all = (orc_scored *)malloc(((size_t)m + 1) * sizeof(orc_scored));
    if (!all) return ORC_ERR_NOMEM;
    m = 0;
    for (int64_t v = 0; v < num_nodes; ++v)
        if (score[v] > 0.0) {
            all[m].score = score[v];
            all[m].id = (int32_t)v;
            ++m;
        }
    qsort(all, (size_t)m, sizeof(orc_scored), cmp_scored);
    const int64_t c = m < k ? m : k;
    for (int64_t i = 0; i < c; ++i) out[i] = all[i].id;
    free(all);
    qsort(out, (size_t)c, sizeof(int32_t), cmp_i32);
    return c;
}
