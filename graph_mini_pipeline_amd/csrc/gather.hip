// Feature-row gather (gfx950): X[i, 0..d) = table row ids[i], bit for bit.
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. II.B ("Nfeat-selecting" is bandwidth-bound; misses of the GPU feature cache are
// served from pinned host memory) and Sec. IV.B (hot feature rows cached in GPU memory); LEO:
// Enabling Efficient Communication-Computation Pipeline for GNN via Hierarchical Caching,
// Sec. 2.3 (GPU kernels read pinned host features directly, zero-copy).
//
// Rows are copied by groups of G lanes (16, 32 or 64 by row length; with 64, a lane owns up to 4
// of the row's 16-byte chunks), so consecutive lanes read consecutive chunks of a row.  A group
// takes G consecutive output rows at a time: lane t loads id t (and its cache slot) once, the ids
// are passed round with cross-lane reads, and the row loads run through a ring of R rows kept in
// flight (a row's chunks are stored as its slot is refilled with the row R places later).  A row
// is read from the HBM hot-row cache when slot[v] >= 0, else from the table (HBM, or pinned host
// memory through its mapped device address).  Bandwidth bound: no arithmetic.  Rows that are not
// 16-byte aligned take a flat (row, element) kernel.  With the Dynamic-Cache on (Sec. IV.B, eq.
// 5), the lane that loads a row's id and slot also records the row's observation when the static
// cache does not hold it.
#include "common.hpp"

namespace gnnmb {

struct GatherArgs {
    const float *table;
    float *cache;   // written only to fill reserved Dynamic-Cache rows
    const int32_t *slot;
    int64_t ld;
    int32_t d;
    int64_t num_rows;
    const int32_t *ids;
    const int64_t *d_n;
    int64_t n_cap;
    float *out;
    int64_t ld_out;
    int64_t *d_hits;
    int32_t *status;
    FastDiv cpr;  // chunks per row
    // scatter (union gather of a super-batch): row r goes to scat_out[s] for every sub-batch s
    // whose relabel bitmap (rank directory scat_rd + s * scat_w) holds the row's key -- its id
    // (scat_by_id) or r itself -- at the key's rank in that bitmap
    const uint2 *scat_rd;
    int64_t scat_w;
    int32_t scat_by_id;
    int32_t scat_g;
    float *scat_out[kMaxGroup];
    int32_t rpu;  // rows per work unit (<= G; G unless the rows are few and fat)
    DynObserve obs;  // Dynamic-Cache observation (obs.score NULL: none), weight obs_w
    double obs_w;
    // Match: output row i is row match[i] of prev (stride ld_prev) when match[i] >= 0 (match NULL:
    // none); such a row has the code -2 - (kPrevCode + match[i])
    const int32_t *match;
    const float *prev;
    int64_t ld_prev;
};

// Row codes of k_gather_rows: c >= 0 table row c; -1 none; -2 - k cache row k (k < kPrevCode) or
// row k - kPrevCode of the previous batch's X (Match).

typedef float f32x4 __attribute__((ext_vector_type(4)));

// A chunk of an output row, stored non-temporally: X is written once and read by the next
// consumer long after, while the table rows just read are read again by the means (which read
// source rows from the table).  Write-back stores left the gathered rows in L2 and the Infinity
// Cache, displacing those rows: dense workload, outermost means 0.188 -> 0.170 ms and the
// three-stream throughput +6% with non-temporal stores (the gather itself then pays for all of its
// writes inside its own time: 0.202 -> 0.229 ms on one stream).
__device__ __forceinline__ void store_x(f32x4 *p, f32x4 v) { __builtin_nontemporal_store(v, p); }

// A source row as a 32-bit code passed between lanes: table row v (v >= 0), cache row s
// (-2 - s), none (-1).  The address is rebuilt from the launch's own table and cache pointers, so
// the row loads stay global loads: a pointer passed between lanes has lost its address space and
// would be read with flat loads, which also count on the LDS counter (a cross-lane read's wait
// would then wait for every row in flight).
__device__ __forceinline__ const float *row_ptr(const float *table, const float *cache, int64_t ld,
                                                int32_t c) {
    return c >= 0 ? table + static_cast<int64_t>(c) * ld
                  : cache + static_cast<int64_t>(-2 - c) * ld;
}
__device__ __forceinline__ const float *row_src(const GatherArgs &g, int32_t c) {
    if (c >= 0) return g.table + static_cast<int64_t>(c) * g.ld;
    const int32_t k = -2 - c;
    return k >= kPrevCode ? g.prev + static_cast<int64_t>(k - kPrevCode) * g.ld_prev
                          : g.cache + static_cast<int64_t>(k) * g.ld;
}

// A row's chunks held by one lane (CH chunks, G lanes apart) written to a reserved Dynamic-Cache
// row: ordinary stores, as the row is read again from there.
template <int CH>
__device__ __forceinline__ void store_cache_row(float *c, const f32x4 (&v)[CH], const bool (&act)[CH],
                                                uint32_t ch0, int G, int d) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        if (!act[q]) continue;
        const int col = static_cast<int>(ch0 + q * G) * 4;
        const int rem = d - col;
        if (rem >= 4) {
            *reinterpret_cast<f32x4 *>(c + col) = v[q];
        } else {
            const float t[4] = {v[q][0], v[q][1], v[q][2], v[q][3]};
            for (int w = 0; w < rem; ++w) c[col + w] = t[w];
        }
    }
}

template <int VEC, int U>
__global__ __launch_bounds__(256) void k_gather(GatherArgs g) {
    using vec_t = typename std::conditional<VEC == 4, f32x4, float>::type;
    const int64_t n = load_count(g.d_n, g.n_cap);
    const uint32_t total = static_cast<uint32_t>(n) * g.cpr.d;
    const uint32_t stride = gridDim.x * 256u * U;
    uint32_t hits = 0;
    for (uint32_t base = blockIdx.x * 256u * U + threadIdx.x; base < total; base += stride) {
        vec_t val[U];
        float *dst[U];
        float *fill[U];   // the reserved Dynamic-Cache row of a pending member, else NULL
        int rem[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t idx = base + u * 256u;
            dst[u] = nullptr;
            fill[u] = nullptr;
            rem[u] = 0;
            if (idx < total) {
                const uint32_t row = fast_div(idx, g.cpr);
                const uint32_t ch = idx - row * g.cpr.d;
                const int32_t v = g.ids[row];
                if (v < 0 || v >= g.num_rows) {
                    set_status(g.status, GNN_ERR_OUT_OF_RANGE);
                    continue;
                }
                const float *src;
                const int32_t pm = g.match ? g.match[row] : -1;
                const int32_t sl = pm < 0 && g.slot ? g.slot[v] : -1;
                if (g.obs.score && ch == 0) dyn_observe(g.obs, v, sl, g.obs_w);
                if (pm >= 0) {
                    src = g.prev + static_cast<int64_t>(pm) * g.ld_prev;
                } else if (sl >= 0) {
                    src = g.cache + static_cast<int64_t>(sl) * g.ld;
                    hits += ch == 0;
                } else {
                    src = g.table + static_cast<int64_t>(v) * g.ld;
                }
                const int col = static_cast<int>(ch) * VEC;
                const int32_t fr = g.obs.filled ? dyn_pending_row(sl) : -1;
                if (fr >= 0) {
                    fill[u] = g.cache + (static_cast<int64_t>(g.obs.static_rows) + fr) * g.ld + col;
                    if (ch == 0) g.obs.filled[fr] = 1;
                }
                dst[u] = g.out + static_cast<int64_t>(row) * g.ld_out + col;
                rem[u] = g.d - col;
                if (VEC == 1 || rem[u] >= VEC) {
                    val[u] = *reinterpret_cast<const vec_t *>(src + col);
                } else {
                    float t[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int q = 0; q < rem[u]; ++q) t[q] = src[col + q];
                    if constexpr (VEC == 4) val[u] = f32x4{t[0], t[1], t[2], t[3]};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (dst[u] == nullptr) continue;
            if (VEC == 1 || rem[u] >= VEC) {
                *reinterpret_cast<vec_t *>(dst[u]) = val[u];
                if (fill[u]) *reinterpret_cast<vec_t *>(fill[u]) = val[u];
            } else if constexpr (VEC == 4) {
                const float t[4] = {val[u][0], val[u][1], val[u][2], val[u][3]};
                for (int q = 0; q < rem[u]; ++q) dst[u][q] = t[q];
                if (fill[u])
                    for (int q = 0; q < rem[u]; ++q) fill[u][q] = t[q];
            }
        }
    }
    if (g.d_hits) {
        hits = wave_sum(hits);
        if (lane_id() == 0 && hits) atomicAdd(reinterpret_cast<unsigned long long *>(g.d_hits),
                                              static_cast<unsigned long long>(hits));
    }
}

template <int G, int CH, int R, bool SCAT>
__global__ __launch_bounds__(256) void k_gather_rows(GatherArgs g) {
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const int64_t n = load_count(g.d_n, g.n_cap);
    const uint32_t cpr = g.cpr.d;
    const uint32_t slabs = (cpr + CH * G - 1) / (CH * G);
    const int rpu = g.rpu;
    const uint32_t units = static_cast<uint32_t>((n + rpu - 1) / rpu) * slabs;
    const uint32_t g0 = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (64 / G) + grp;
    const uint32_t gstride = gridDim.x * 4u * (64 / G);
    uint32_t hits = 0;
    for (uint32_t it = g0; it < units; it += gstride) {
        const uint32_t rb = it / slabs;         // batch of rpu rows
        const uint32_t p = it - rb * slabs;     // slab of the row
        const int64_t r0 = static_cast<int64_t>(rb) * rpu;
        const int nb = static_cast<int>(n - r0 < rpu ? n - r0 : rpu);
        // lane t: id and source row code of output row r0 + t (-1: invalid id), and the reserved
        // Dynamic-Cache row the row also goes to (-1: none)
        int32_t mine = -1;
        int32_t vid = -1;
        int32_t fill = -1;
        if (gl < nb) {
            const int32_t v = g.ids[r0 + gl];
            vid = v;
            const int32_t pm = !SCAT && g.match ? g.match[r0 + gl] : -1;
            if (v < 0 || v >= g.num_rows) {
                set_status(g.status, GNN_ERR_OUT_OF_RANGE);
            } else if (pm >= 0) {
                mine = -2 - (kPrevCode + pm);
            } else {
                const int32_t sl = g.slot ? g.slot[v] : -1;
                if constexpr (!SCAT) {
                    if (g.obs.score && p == 0) dyn_observe(g.obs, v, sl, g.obs_w);
                    if (g.obs.filled) {
                        fill = dyn_pending_row(sl);
                        if (fill >= 0 && p == 0) g.obs.filled[fill] = 1;
                    }
                }
                if (sl >= 0) {
                    mine = -2 - sl;
                    hits += p == 0;
                } else {
                    mine = v;
                }
            }
        }
        // scatter: lane t holds the destination rows (1-based, 0: none) of union row r0 + t
        int32_t dest[kMaxGroup];
        if constexpr (SCAT) {
            const int64_t key = g.scat_by_id ? static_cast<int64_t>(vid) : r0 + gl;
#pragma unroll
            for (int s2 = 0; s2 < kMaxGroup; ++s2) {
                dest[s2] = 0;
                if (s2 < g.scat_g && gl < nb && key >= 0 && (key >> 5) < g.scat_w) {
                    const int32_t r = rdir_rank(g.scat_rd + s2 * g.scat_w, key);
                    if (r >= 0) dest[s2] = r + 1;
                }
            }
        }
        const uint32_t ch0 = p * CH * G + gl;
        bool act[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) act[q] = ch0 + q * G < cpr;
        auto code_of = [&](int r) -> int32_t {
            const int rr = r < nb ? r : 0;
            if constexpr (G == 64) return __builtin_amdgcn_readlane(mine, rr);
            else return __shfl(mine, grp * G + rr, 64);
        };
        f32x4 v[R][CH];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int32_t c = code_of(r);
            const float *row = SCAT ? row_ptr(g.table, g.cache, g.ld, c) : row_src(g, c);   // union rows: no Match
#pragma unroll
            for (int q = 0; q < CH; ++q)
                v[r][q] = (r < nb && c != -1 && act[q])
                              ? *reinterpret_cast<const f32x4 *>(row + static_cast<int64_t>(ch0 + q * G) * 4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int e = 0; e < nb; e += R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int er = e + r;
                auto store_row = [&](float *o) {
#pragma unroll
                    for (int q = 0; q < CH; ++q) {
                        if (!act[q]) continue;
                        const int col = static_cast<int>(ch0 + q * G) * 4;
                        const int rem = g.d - col;
                        if (rem >= 4) {
                            store_x(reinterpret_cast<f32x4 *>(o + col), v[r][q]);
                        } else {
                            const float t[4] = {v[r][q][0], v[r][q][1], v[r][q][2], v[r][q][3]};
                            for (int w = 0; w < rem; ++w) o[col + w] = t[w];
                        }
                    }
                };
                if (er < nb && code_of(er) != -1) {
                    if constexpr (SCAT) {
#pragma unroll
                        for (int s2 = 0; s2 < kMaxGroup; ++s2) {
                            if (s2 >= g.scat_g) break;
                            int32_t pos;
                            if constexpr (G == 64) pos = __builtin_amdgcn_readlane(dest[s2], er);
                            else pos = __shfl(dest[s2], grp * G + er, 64);
                            if (pos > 0) store_row(g.scat_out[s2] + static_cast<int64_t>(pos - 1) * g.ld_out);
                        }
                    } else {
                        store_row(g.out + (r0 + er) * g.ld_out);
                        if (g.obs.filled) {
                            int32_t fr;
                            if constexpr (G == 64) fr = __builtin_amdgcn_readlane(fill, er);
                            else fr = __shfl(fill, grp * G + er, 64);
                            if (fr >= 0)
                                store_cache_row(g.cache + (static_cast<int64_t>(g.obs.static_rows) + fr) * g.ld,
                                                v[r], act, ch0, G, g.d);
                        }
                    }
                }
                const int en = er + R;
                const int32_t c = code_of(en);
                const float *row = SCAT ? row_ptr(g.table, g.cache, g.ld, c) : row_src(g, c);   // union rows: no Match
#pragma unroll
                for (int q = 0; q < CH; ++q)
                    v[r][q] = (en < nb && c != -1 && act[q])
                                  ? *reinterpret_cast<const f32x4 *>(row + static_cast<int64_t>(ch0 + q * G) * 4)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    if (g.d_hits) {
        hits = wave_sum(hits);
        if (lane_id() == 0 && hits) atomicAdd(reinterpret_cast<unsigned long long *>(g.d_hits),
                                              static_cast<unsigned long long>(hits));
    }
}


// ---- all sub-batches of a super-batch in one launch -----------------------------------------------
//
// Row units (G consecutive output rows of one sub-batch, one slab) are numbered over the sub-batches'
// actual row counts, so one launch streams every sub-batch's rows: the start-up and drain of one
// large launch replace those of G small ones, and a host-resident table keeps G times as many
// host-link reads in flight.

template <int G, int CH, int R>
__global__ __launch_bounds__(256) void k_gather_batch(GatherBatchArgs a) {
    __shared__ int64_t s_n[kMaxGroup];
    __shared__ uint32_t s_u0[kMaxGroup + 1];
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const uint32_t cpr = a.cpr;
    const uint32_t slabs = (cpr + CH * G - 1) / (CH * G);
    if (threadIdx.x < static_cast<unsigned>(a.nseg)) {
        const GatherSeg &S = a.seg[threadIdx.x];
        s_n[threadIdx.x] = load_count(S.d_n, S.n_cap);
    }
    __syncthreads();
    // each sub-batch's units start at a multiple of the units one wavefront takes at a time, so
    // a wavefront's units are all in one sub-batch (the padding units have no rows): its fields are
    // read with scalar loads, which do not wait on vector memory
    if (threadIdx.x == 0) {
        uint32_t u = 0;
        for (int sg = 0; sg < a.nseg; ++sg) {
            s_u0[sg] = u;
            const uint32_t nu = static_cast<uint32_t>((s_n[sg] + G - 1) / G) * slabs;
            u += (nu + 64 / G - 1) / (64 / G) * (64 / G);
        }
        s_u0[a.nseg] = u;
    }
    __syncthreads();
    const uint32_t units = s_u0[a.nseg];
    const uint32_t g0 = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (64 / G) + grp;
    const uint32_t gstride = gridDim.x * 4u * (64 / G);
    uint32_t hits = 0;
    for (uint32_t it = g0; it < units; it += gstride) {
        const uint32_t it0 = __builtin_amdgcn_readfirstlane(it);
        int sg = 0;
        while (sg + 1 < a.nseg && s_u0[sg + 1] <= it0) ++sg;
        sg = __builtin_amdgcn_readfirstlane(sg);
        const GatherSeg &S = a.seg[sg];
        const uint32_t li = it - s_u0[sg];
        const uint32_t rb = li / slabs;
        const uint32_t p = li - rb * slabs;
        const int64_t r0 = static_cast<int64_t>(rb) * G;
        const int64_t n = s_n[sg];
        const int nb = static_cast<int>(n - r0 < G ? n - r0 : G);
        // lane t: source row of output row r0 + t (NULL: invalid id), and the reserved Dynamic-Cache
        // row the row also goes to (-1: none)
        int32_t mine = -1;
        int32_t fill = -1;
        if (gl < nb) {
            const int32_t v = S.ids[r0 + gl];
            if (v < 0 || v >= a.num_rows) {
                set_status(a.status, GNN_ERR_OUT_OF_RANGE);
            } else {
                const int32_t sl = a.slot ? a.slot[v] : -1;
                if (a.obs.score && p == 0) dyn_observe(a.obs, v, sl, S.obs_w);
                if (a.obs.filled) {
                    fill = dyn_pending_row(sl);
                    if (fill >= 0 && p == 0) a.obs.filled[fill] = 1;
                }
                hits += sl >= 0 && p == 0;
                mine = sl >= 0 ? -2 - sl : v;
            }
        }
        const uint32_t ch0 = p * CH * G + gl;
        bool act[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) act[q] = ch0 + q * G < cpr;
        auto code_of = [&](int r) -> int32_t {
            const int rr = r < nb ? r : 0;
            if constexpr (G == 64) return __builtin_amdgcn_readlane(mine, rr);
            else return __shfl(mine, grp * G + rr, 64);
        };
        f32x4 v[R][CH];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int32_t c = code_of(r);
            const float *row = row_ptr(a.table, a.cache, a.ld, c);
#pragma unroll
            for (int q = 0; q < CH; ++q)
                v[r][q] = (r < nb && c != -1 && act[q])
                              ? *reinterpret_cast<const f32x4 *>(row + static_cast<int64_t>(ch0 + q * G) * 4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int e = 0; e < nb; e += R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int er = e + r;
                if (er < nb && code_of(er) != -1) {
                    float *o = S.out + (r0 + er) * a.ld_out;
#pragma unroll
                    for (int q = 0; q < CH; ++q) {
                        if (!act[q]) continue;
                        const int col = static_cast<int>(ch0 + q * G) * 4;
                        const int rem = a.d - col;
                        if (rem >= 4) {
                            store_x(reinterpret_cast<f32x4 *>(o + col), v[r][q]);
                        } else {
                            const float t[4] = {v[r][q][0], v[r][q][1], v[r][q][2], v[r][q][3]};
                            for (int w = 0; w < rem; ++w) o[col + w] = t[w];
                        }
                    }
                    if (a.obs.filled) {
                        int32_t fr;
                        if constexpr (G == 64) fr = __builtin_amdgcn_readlane(fill, er);
                        else fr = __shfl(fill, grp * G + er, 64);
                        if (fr >= 0)
                            store_cache_row(a.cache + (static_cast<int64_t>(a.obs.static_rows) + fr) * a.ld,
                                            v[r], act, ch0, G, a.d);
                    }
                }
                const int en = er + R;
                const int32_t c = code_of(en);
                const float *row = row_ptr(a.table, a.cache, a.ld, c);
#pragma unroll
                for (int q = 0; q < CH; ++q)
                    v[r][q] = (en < nb && c != -1 && act[q])
                                  ? *reinterpret_cast<const f32x4 *>(row + static_cast<int64_t>(ch0 + q * G) * 4)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    if (a.d_hits) {
        hits = wave_sum(hits);
        if (lane_id() == 0 && hits) atomicAdd(reinterpret_cast<unsigned long long *>(a.d_hits),
                                              static_cast<unsigned long long>(hits));
    }
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// rows per work unit of the union gather (measured with 16, 8 and 4 rows: dense gather 232, 214
// and 205 us)
constexpr int kUnionRowsPerUnit = 4;

// rows in flight per group: 8 with 64 lanes, 4 with 16 or 32 (measured best on 602-, 128-, 100-
// and 64-float rows)
template <bool SCAT>
void launch_rows(const GatherArgs &g, int G, int CH, dim3 grid, hipStream_t s) {
    if (G == 16) hipLaunchKernelGGL((k_gather_rows<16, 1, 4, SCAT>), grid, dim3(256), 0, s, g);
    else if (G == 32) hipLaunchKernelGGL((k_gather_rows<32, 1, 4, SCAT>), grid, dim3(256), 0, s, g);
    else if (CH == 1) hipLaunchKernelGGL((k_gather_rows<64, 1, 8, SCAT>), grid, dim3(256), 0, s, g);
    else if (CH == 2) hipLaunchKernelGGL((k_gather_rows<64, 2, 8, SCAT>), grid, dim3(256), 0, s, g);
    else if (CH == 3) hipLaunchKernelGGL((k_gather_rows<64, 3, 8, SCAT>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((k_gather_rows<64, 4, 8, SCAT>), grid, dim3(256), 0, s, g);
}

hipError_t launch_gather(const float *table, float *cache, const int32_t *slot, int64_t ld,
                         int64_t d, int64_t num_rows, const int32_t *ids, const int64_t *d_n,
                         int64_t n_cap, float *out, int64_t ld_out, int64_t *d_hits,
                         int32_t *status, hipStream_t s, const DynObserve *obs, double obs_w,
                         const int32_t *match, const float *prev, int64_t ld_prev) {
    if (n_cap <= 0 || d <= 0) return hipSuccess;
    const bool v4 = ld % 4 == 0 && ld_out % 4 == 0 && aligned16(table) && aligned16(out) &&
                    (cache == nullptr || aligned16(cache)) &&
                    (match == nullptr || (ld_prev % 4 == 0 && aligned16(prev)));
    const int vec = v4 ? 4 : 1;
    const int64_t cpr = (d + vec - 1) / vec;
    GatherArgs g{table, cache, slot, ld, static_cast<int32_t>(d), num_rows, ids, d_n, n_cap,
                 out, ld_out, d_hits, status, make_fastdiv(static_cast<uint32_t>(cpr)),
                 nullptr, 0, 0, 0, {}, 0, {}, 0.0};
    if (obs) {
        g.obs = *obs;
        g.obs_w = obs_w;
    }
    g.match = match;
    g.prev = prev;
    g.ld_prev = ld_prev;
    if (!v4) {
        constexpr int U = 4;
        hipLaunchKernelGGL((k_gather<1, U>), dim3(grid_for(n_cap * cpr, 256 * U, 2048)), dim3(256),
                           0, s, g);
        return hipGetLastError();
    }
    const int G = cpr <= 16 ? 16 : (cpr <= 32 ? 32 : 64);
    const int CH = G < 64 ? 1 : static_cast<int>((cpr + 63) / 64 < 4 ? (cpr + 63) / 64 : 4);
    const int64_t slabs = (cpr + CH * G - 1) / (CH * G);
    const int64_t units = (n_cap + G - 1) / G * slabs;
    if (units > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    g.rpu = G;
    const dim3 grid(grid_for(units, 4 * (64 / G), 8192));
    launch_rows<false>(g, G, CH, grid, s);
    return hipGetLastError();
}

hipError_t launch_gather_union(const float *table, int64_t ld, int64_t d, int64_t num_rows,
                               const int32_t *ids, const int64_t *d_n, int64_t n_cap,
                               const uint2 *rd, int64_t words, int by_id,
                               int G_sb, float *const *outs, int64_t ld_out, int32_t *status,
                               hipStream_t s) {
    if (G_sb < 1 || G_sb > kMaxGroup) return hipErrorInvalidValue;
    bool v4 = ld % 4 == 0 && ld_out % 4 == 0 && aligned16(table);
    for (int sg = 0; sg < G_sb; ++sg) v4 = v4 && aligned16(outs[sg]);
    if (!v4) return hipErrorInvalidValue;   // the caller gathers per sub-batch instead
    if (n_cap <= 0 || d <= 0) return hipSuccess;
    const int64_t cpr = (d + 3) / 4;
    GatherArgs g{table, nullptr, nullptr, ld, static_cast<int32_t>(d), num_rows, ids, d_n, n_cap,
                 nullptr, ld_out, nullptr, status, make_fastdiv(static_cast<uint32_t>(cpr)),
                 rd, words, by_id, G_sb, {}, 0, {}, 0.0};
    for (int sg = 0; sg < G_sb; ++sg) g.scat_out[sg] = outs[sg];
    const int G = cpr <= 16 ? 16 : (cpr <= 32 ? 32 : 64);
    const int CH = G < 64 ? 1 : static_cast<int>((cpr + 63) / 64 < 4 ? (cpr + 63) / 64 : 4);
    // each union row is stored several times: units of kUnionRowsPerUnit rows keep enough
    // workgroups in flight for the union's (fewer) rows
    g.rpu = kUnionRowsPerUnit < G ? kUnionRowsPerUnit : G;
    const int64_t slabs = (cpr + CH * G - 1) / (CH * G);
    const int64_t units = (n_cap + g.rpu - 1) / g.rpu * slabs;
    if (units > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const dim3 grid(grid_for(units, 4 * (64 / G), 8192));
    launch_rows<true>(g, G, CH, grid, s);
    return hipGetLastError();
}

hipError_t launch_gather_batch(GatherBatchArgs a, int64_t rows_cap, hipStream_t s) {
    if (a.nseg <= 0 || a.d <= 0 || rows_cap <= 0) return hipSuccess;
    bool v4 = a.ld % 4 == 0 && a.ld_out % 4 == 0 && aligned16(a.table) &&
              (a.cache == nullptr || aligned16(a.cache));
    for (int sg = 0; sg < a.nseg; ++sg) v4 = v4 && (a.seg[sg].n_cap == 0 || aligned16(a.seg[sg].out));
    if (!v4) {
        // rows not 16-byte aligned: the flat kernel, one launch per sub-batch
        for (int sg = 0; sg < a.nseg; ++sg) {
            const GatherSeg &S = a.seg[sg];
            const hipError_t e = launch_gather(a.table, a.cache, a.slot, a.ld, a.d, a.num_rows, S.ids,
                                               S.d_n, S.n_cap, S.out, a.ld_out, a.d_hits, a.status, s,
                                               &a.obs, S.obs_w);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int64_t cpr = (a.d + 3) / 4;
    a.cpr = static_cast<uint32_t>(cpr);
    const int G = cpr <= 16 ? 16 : (cpr <= 32 ? 32 : 64);
    const int CH = G < 64 ? 1 : static_cast<int>((cpr + 63) / 64 < 4 ? (cpr + 63) / 64 : 4);
    const int64_t slabs = (cpr + CH * G - 1) / (CH * G);
    // each sub-batch: its rounded-up row units and up to 64 / G - 1 padding units
    const int64_t units = (rows_cap + G - 1) / G * slabs + a.nseg * (slabs + 64 / G);
    if (units > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const dim3 grid(grid_for(units, 4 * (64 / G), 8192));
    if (G == 16) hipLaunchKernelGGL((k_gather_batch<16, 1, 4>), grid, dim3(256), 0, s, a);
    else if (G == 32) hipLaunchKernelGGL((k_gather_batch<32, 1, 4>), grid, dim3(256), 0, s, a);
    else if (CH == 1) hipLaunchKernelGGL((k_gather_batch<64, 1, 8>), grid, dim3(256), 0, s, a);
    else if (CH == 2) hipLaunchKernelGGL((k_gather_batch<64, 2, 8>), grid, dim3(256), 0, s, a);
    else if (CH == 3) hipLaunchKernelGGL((k_gather_batch<64, 3, 8>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_gather_batch<64, 4, 8>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

// Setup: cache[r] = table row hot[r]; slot[hot[r]] = r.
__global__ __launch_bounds__(256) void k_cache_fill(const float *table, int64_t ld, int64_t d,
                                                   int64_t num_rows, const int32_t *hot,
                                                   int64_t rows, float *cache, int32_t *slot,
                                                   int32_t *status) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int32_t v = hot[r];
        if (v < 0 || v >= num_rows) {
            if (threadIdx.x == 0) set_status(status, GNN_ERR_OUT_OF_RANGE);
            continue;
        }
        for (int64_t t = threadIdx.x; t < d; t += blockDim.x)
            cache[r * ld + t] = table[static_cast<int64_t>(v) * ld + t];
        if (threadIdx.x == 0) slot[v] = static_cast<int32_t>(r);
    }
}

hipError_t launch_cache_fill(const float *table, int64_t ld, int64_t d, int64_t num_rows,
                             const int32_t *hot, int64_t rows, float *cache, int32_t *slot,
                             int32_t *status, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_cache_fill, dim3(grid_for(rows, 1, 65536)), dim3(256), 0, s, table, ld,
                       d, num_rows, hot, rows, cache, slot, status);
    return hipGetLastError();
}

}  // namespace gnnmb
