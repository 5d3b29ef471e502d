// Shared device/host helpers of the gfx950 mini-batch library (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gnnmb.h"

namespace gnnmb {

// SplitMix64 increment (odd integer nearest 2^64 / golden ratio).
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

// SplitMix64 output function (Steele, Lea, Flood, OOPSLA 2014).  The pages fix no generator; this
// hash makes the neighbour draw deterministic and counter-based.
__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

// Division of n < 2^32 by a fixed divisor with one multiply-high and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI 1994, round-up variant):
// s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1, q = (mulhi(n, m) + n) >> s.
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t m = (((1ull << 32) * ((1ull << s) - d)) / d) + 1;
    return FastDiv{d, static_cast<uint32_t>(m), s};
}

__host__ __device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
    const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> 32);
    return static_cast<uint32_t>((static_cast<uint64_t>(t) + n) >> f.s);
}

// First device error wins; later ones are dropped.  A NULL status word drops every error.
__device__ __forceinline__ void set_status(int32_t *st, int32_t code) {
    if (st != nullptr) atomicCAS(st, 0, code);
}

__device__ __forceinline__ int64_t load_count(const int64_t *d_n, int64_t cap) {
    if (d_n == nullptr) return cap;
    const int64_t n = *d_n;
    return n < 0 ? 0 : (n < cap ? n : cap);
}

__device__ __forceinline__ int64_t row_ptr(const void *indptr, int ib, int64_t v) {
    return ib == 8 ? static_cast<const int64_t *>(indptr)[v]
                   : static_cast<int64_t>(static_cast<const int32_t *>(indptr)[v]);
}

// Orders LDS traffic between lanes of one wavefront (compiler code-motion barrier plus
// wavefront-scope fences; LDS operations of one wavefront execute in order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x & 63u); }

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const T t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Exclusive scan over a workgroup of NT threads; `smem` holds NT/64 entries.  Every thread of
// the workgroup must call it.  Returns the exclusive prefix; *total receives the block total.
template <typename T, int NT>
__device__ __forceinline__ T block_exclusive_scan(T v, T *total, T *smem) {
    constexpr int NW = NT / 64;
    const int lane = lane_id();
    const int w = static_cast<int>(threadIdx.x >> 6);
    const T inc = wave_inclusive_scan(v);
    if (lane == 63) smem[w] = inc;
    __syncthreads();
    T before = T(0), tot = T(0);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const T s = smem[i];
        if (i < w) before += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + inc - v;
}

// ---- single-pass scans (decoupled look-back) ----------------------------------------------------
//
// A scan over tiles in one launch: each workgroup takes a ticket (an atomic counter, so tiles are
// handed out in the order workgroups start and every lower tile belongs to a workgroup that is
// running or done), publishes its tile's aggregate, sums its predecessors' published words back
// to the nearest inclusive prefix, and publishes its own inclusive prefix.  A tile only waits for
// lower tiles, which publish their aggregates without waiting, so every wait ends.  Each tile's
// state and value share one 64-bit word written and read with agent-scope atomics, so no other
// memory ordering is needed across the chip's L2 caches.  Words and ticket start at zero (the
// call's first kernel clears them).
constexpr uint64_t kLbAggregate = 1ull << 62;
constexpr uint64_t kLbInclusive = 2ull << 62;

__device__ __forceinline__ void lb_publish(uint64_t *word, uint64_t state, uint32_t value) {
    __hip_atomic_store(word, state | value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The sum of the values of tiles 0 .. t-1 of a chain of words; called by all 64 lanes of one
// wavefront, returns the same value on every lane.  Each round reads the 256 nearest unsummed
// predecessors at once (lane L the four at distances 4L .. 4L+3), so that a chain of up to 256
// tiles needs one round trip to the coherent memory once its words are published.
constexpr int kLbPerLane = 4;
__device__ __forceinline__ uint32_t lb_exclusive(const uint64_t *words, int64_t t) {
    const int lane = lane_id();
    uint32_t prefix = 0;
    int64_t end = t;
    while (end > 0) {
        uint64_t f[kLbPerLane];
#pragma unroll
        for (int q = 0; q < kLbPerLane; ++q) {
            const int64_t j = end - 1 - (kLbPerLane * lane + q);
            f[q] = kLbInclusive;            // before tile 0: an inclusive prefix of 0
            if (j >= 0) {
                do {
                    f[q] = __hip_atomic_load(&words[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } while ((f[q] >> 62) == 0);
            }
        }
        // the nearest inclusive word of this lane (kLbPerLane: none), and the lanes that have one
        int near = kLbPerLane;
#pragma unroll
        for (int q = kLbPerLane - 1; q >= 0; --q)
            if ((f[q] >> 62) == 2) near = q;
        const uint64_t incl = __ballot(near < kLbPerLane);
        const int k = incl ? __ffsll(static_cast<long long>(incl)) - 1 : 64;
        // sum every word up to and including the nearest inclusive one (all of them if none)
        uint32_t v = 0;
#pragma unroll
        for (int q = 0; q < kLbPerLane; ++q)
            if (lane < k || (lane == k && q <= near)) v += static_cast<uint32_t>(f[q]);
        prefix += wave_sum(v);
        if (incl) break;
        end -= 64 * kLbPerLane;
    }
    return prefix;
}

// Thread 0 of the workgroup takes the next ticket of `ticket`; every thread gets it.
__device__ __forceinline__ uint32_t lb_ticket(uint32_t *ticket, uint32_t *s_slot) {
    if (threadIdx.x == 0) *s_slot = atomicAdd(ticket, 1u);
    __syncthreads();
    return *s_slot;
}

// Per-launch chains of look-back words, carved from the workspace's arena (cleared at the start of
// every call), handed out in launch order on the host.
struct LbSlice {
    uint64_t *words;    // one per tile
    uint32_t *ticket;   // ticket counter (a relabel: one per bitmap)
};

// ---- launch helpers (host) ----------------------------------------------------------------------

inline unsigned grid_for(int64_t items, int per_block, unsigned max_blocks) {
    int64_t b = (items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > static_cast<int64_t>(max_blocks)) b = max_blocks;
    return static_cast<unsigned>(b);
}

// Degree classes of the sampler.
enum : int32_t { kFull = 0, kGroup = 1, kWave = 2, kBlock = 3, kNumClasses = 4 };

// Degree buckets of the one-wavefront class, and the classification's per-block columns (edges,
// then FULL, GROUP, the buckets and BLOCK).
constexpr int kWaveBuckets = 6;
constexpr int kCols = 4 + kWaveBuckets;
constexpr int kCats = 3 + kWaveBuckets;       // FULL, GROUP, WAVE buckets, BLOCK
// Per-hop slots of the classification totals in the workspace (kCols used).
constexpr int kTotalsStride = 16;

// Candidate capacities per class (LDS) and the fanout each supports (capacity >= 4 * fanout).
// A sampler workgroup holds kBlockCap candidates of 12 bytes (key, position): 3328 of them keep it
// under 40 KB, so four workgroups (32 wavefronts, the register-file limit) fit one CU's 160 KB.
constexpr int kGroupLanes = 16;
constexpr int kGroupCap = 104;
constexpr int kWaveCap = 416;
constexpr int kBlockThreads = 512;
constexpr int kBlockCap = 3328;
constexpr int kMaxFanout = kBlockCap / 4;

// One sampling hop.
struct HopArgs {
    const void *indptr;
    const int32_t *indices;     // device, or pinned host memory read in place
    const int64_t *adj_off;     // optional HBM adjacency cache: row v at adj_rows + adj_off[v]
    const int32_t *adj_rows;
    int64_t num_nodes;
    const int32_t *front;   // destinations V_{l-1}
    const int64_t *d_F;     // device count of front (NULL: F_cap)
    int64_t F_cap;
    int32_t ib;             // indptr bytes
    int32_t k;              // fanout
    uint64_t hop_seed;
    int32_t group_max, wave_max;
    int32_t exact_rank;     // rank every node's candidates by (key, position), skipping the
                            // ranking by the keys' high words
    int32_t *blk_indptr;    // [F_cap+1]
    int32_t *blk_gid;       // [E_cap]
    int64_t E_cap;
    int64_t *d_E;           // receives |E_l|
    int32_t *lists;         // [kCats * F_cap] one work-list per category (FULL, GROUP, the WAVE
                            // degree buckets largest first, BLOCK), each at a multiple of F_cap
    uint32_t *totals;       // [kCols] |E_l| then the category sizes (zero before the hop)
    uint32_t *clear_ptr;    // words the classification clears (the relabel bitmap of this hop)
    int64_t clear_n;
    uint32_t *inv_mask;     // optional [F]: zeroed over the frontier by the classification
    uint32_t *mark;         // optional bitmap over node ids: the sampler sets the bit of every
                            // id it emits (a super-batch's accumulated union, compact relabel)
    // optional: the grid first zeroes zero_g regions of zero_stride words (and their byte maps of
    // 8 zero_stride words, when given) over the first ceil(bound / 32) words, bound = *zero_da +
    // *zero_db capped at 32 zero_stride: the sub-batch bitmaps that this hop's distribution marks
    uint32_t *zero_words;
    uint32_t *zero_bytes;
    int64_t zero_stride;
    int32_t zero_g;
    const int64_t *zero_da;
    const int64_t *zero_db;
    int32_t *status;
    int32_t nb;             // classify tiles (workgroups)
    LbSlice lb;             // look-back words of the classification: nb tiles (zero)
};

// Largest super-batch (sub-batches per call).
constexpr int kMaxGroup = GNN_MAX_GROUP;

// An id list to relabel: marked into bitmap `bitmap`; if lid is not NULL, lid[i] receives the
// rank of ids[i] in that bitmap's unique list.  Lists of pass 1 are marked first, alone, and a
// repeated id among them is reported as a duplicate.
struct IdList {
    const int32_t *ids;
    const int64_t *d_n;  // device count (NULL: cap)
    int64_t cap;
    int32_t *lid;
    int32_t bitmap;
    int32_t pass;        // 1: marked first, repeats reported; 0: marked; 2: ranked only
};

// The sorted unique list of one bitmap.
struct BitmapOut {
    int32_t *uniq;
    int64_t uniq_cap;
    int64_t *d_uniq;
    int32_t *pos;        // optional: the bit positions themselves (equal to uniq unless mapped)
};

struct RelabelArgs {
    IdList list[2 * kMaxGroup];
    int32_t nlist;
    BitmapOut out[kMaxGroup];
    int32_t nbm;              // bitmaps (one per BitmapOut)
    int64_t id_bound;
    const int64_t *d_bound;   // optional device bound on the ids (at most id_bound); bitmap words
                              // at or past it are ignored, whatever they hold
    const int32_t *id_map;    // optional: bit position p stands for id id_map[p] in uniq
    uint8_t *bytes;           // optional [nbm * W * 32], zero: lists of pass 0 set byte[id] = 1
                              // (plain stores) and the popcount pass packs bytes into the bitmap
    uint32_t *bitmap;         // [nbm * W]
    uint2 *rdir;              // [nbm * W] rank directory, written by the emit pass: entry w holds
                              // the set bits before word w and word w itself, so that an id's rank
                              // is one 8-byte load
    uint32_t *bsum;           // [nbm * nbw] tile popcounts (bitmaps of many tiles)
    int64_t W;
    int32_t nbw;              // tiles per bitmap
    uint32_t *clear_ptr;      // optional region zeroed by the emit pass
    int64_t clear_n;
    int32_t *status;
    int32_t bitmap_cleared;   // the bitmaps are already zero on this stream
    LbSlice lb;               // look-back words of the emit pass: nbm * nbw tiles (zero)
    int32_t sort_sets_bits;   // the sort path (short lists) also sets the unique ids' bits in the
                              // bitmap (which it otherwise leaves untouched)
    int32_t bitmap_read_after; // later kernels rank ids in the bitmap and its word prefixes: the
                               // bitmap path is required
    int32_t force;            // 0: the path by size; 1: sort whenever eligible; 2: the bitmap
};

// Short lists are relabelled by one workgroup that sorts them in LDS (relabel.hip) instead of
// through the bitmap; whether launch_relabel takes that path for these arguments.
bool relabel_sorts(const RelabelArgs &a);

// Rank of bit v in a bitmap by its rank directory (entry w: set bits before word w, word w), or
// -1 when the bit is clear.
__device__ __forceinline__ int32_t rdir_rank(const uint2 *rd, int64_t v) {
    const uint2 e = rd[v >> 5];
    const uint32_t bit = 1u << (v & 31);
    return (e.y & bit) ? static_cast<int32_t>(e.x + __popc(e.y & (bit - 1u))) : -1;
}

__device__ __forceinline__ int64_t relabel_bound(const RelabelArgs &a) {
    if (a.d_bound == nullptr) return a.id_bound;
    const int64_t b = *a.d_bound;
    return b < 0 ? 0 : (b < a.id_bound ? b : a.id_bound);
}

// Destinations per tile of the super-batch distribution: one per thread of its workgroup.  512
// measured best of 128 .. 1024 (sampling stage outside the sampler per super-batch, 256 -> 512:
// 111M-node 0.413 -> 0.397 ms, mid 0.321 -> 0.314, dense unchanged): half as many tiles wait in
// each sub-batch's look-back chain.
constexpr int kDistTile = 512;

// One sub-batch of a super-batch hop: its destinations and the block it receives.
struct DistSub {
    const int32_t *front;
    const int64_t *d_F;
    int64_t F_cap;
    const int32_t *upos;  // [F] position of each destination in the union frontier U_l, or NULL:
                          // the rank of front[i] in the union bitmap
    int32_t *f_pos;       // [F] out (with upos): position of each destination in U_{l+1}
    int32_t *blk_indptr;
    int32_t *blk_gid;
    int32_t *e_pos;       // [E_cap] out (with upos): position of each sampled id in U_{l+1}
    int64_t E_cap;
    int64_t *d_E;
    int32_t tile0;  // first tile of this sub-batch in the launch
    int32_t ntile;
};

struct DistArgs {
    DistSub sub[kMaxGroup];
    int32_t G;
    int32_t ntiles;
    const uint2 *rdir0;        // union bitmap's rank directory (destinations without upos)
    int64_t id_bound;
    const int32_t *u_indptr;   // union block
    const int32_t *u_gid;
    int64_t uE_cap;
    const int64_t *d_U;        // |U_l|
    int64_t U_cap;
    const int64_t *d_U1;       // |U_{l+1}|
    int64_t U1_cap;
    LbSlice lb;                // look-back words, one per tile (sub-batch g's chain at tile0),
                               // and one ticket counter per sub-batch
    int32_t *status;
    int32_t *inv;              // optional out [U_cap * G]: inv[r * G + g] = 1 + the position of
                               // union node r among sub-batch g's destinations, written where
    uint32_t *inv_mask;        // inv_mask[r] (zero before) gets bit g: entries without it are stale
    // optional (compact relabel): the sub-batch relabel's marks, made here: sub-batch g's bitmap
    // at mark_words + g * mark_stride (zero before), or its byte map at mark_bytes + 32 g
    // mark_stride; destinations at hop 0 are seeds, marked with a duplicate check
    uint32_t *mark_words;
    uint8_t *mark_bytes;
    int64_t mark_stride;
    int32_t mark_dup;
    // compact relabel: U_l (global ids) and the rank directory of U_{l+1}'s node-id bitmap; a
    // position in U_{l+1} is a rank in that bitmap
    const int32_t *Ul;
    const uint2 *rdir1;
};

constexpr int kClassifyThreads = 256;
constexpr int kClassifyItems = 2;   // nodes per thread: two keep enough wavefronts in flight for the row-pointer loads
constexpr int kClassifyTile = kClassifyThreads * kClassifyItems;
constexpr int kBitmapThreads = 256;
// Bitmap words per thread of the popcount and emit passes: 4 keeps more workgroups in flight than
// 8 (sampling stage -2 to -5% on every workload); 2 helps small id ranges and costs large ones.
constexpr int kBitmapWordsPerThread = 4;
constexpr int kBitmapTile = kBitmapThreads * kBitmapWordsPerThread;

// ---- Dynamic-Cache observation (GARDEN, Sec. IV.B, eq. 5) ---------------------------------------
//
// Each mini-batch t adds its weight w_t = W * gamma^-t to the scaled score S(v) of every node v
// whose row it requests and the static cache does not hold, so S(v) = w_t * Score(v, t) at any
// step t: all scores decay by the same factor per step, none has to be touched to decay, and the
// order of the S(v) is the order of the Score(v, t).  Observed nodes are marked in the touched
// bitmap, which also holds the current Dynamic-Cache members (set at each refresh).
//
// Slots: s >= 0 -- the row is in cache row s; -1 -- not cached; s <= -2 -- a Dynamic-Cache member
// whose row (-2 - s of the Dynamic-Cache region) is reserved but not filled yet.  Such a row is
// read from the table, and the gather that reads it also writes it to the reserved row and marks
// it filled (fill on miss: taking a node in moves no row by itself); the next refresh, after
// which no gather of before it still runs, makes filled rows resident (slot >= 0).
struct DynObserve {
    double *score;        // [num_rows] scaled scores; NULL: no observation
    uint32_t *touched;    // [ceil(num_rows / 32)]
    int32_t static_rows;  // cache slots below this one hold the static cache
    uint8_t *filled;      // [k_dyn] reserved rows written by a gather; NULL: no Dynamic-Cache
};

// The reserved Dynamic-Cache row of a pending member's slot value, else -1.
__device__ __forceinline__ int32_t dyn_pending_row(int32_t sl) { return sl <= -2 ? -2 - sl : -1; }

// Observation of the requested row of node v (0 <= v < num_rows) whose cache slot is sl.
__device__ __forceinline__ void dyn_observe(const DynObserve &o, int32_t v, int32_t sl, double w) {
    if (sl >= 0 && sl < o.static_rows) return;   // a static-cache hit: not residual
    unsafeAtomicAdd(o.score + v, w);
    uint32_t *word = o.touched + (v >> 5);
    const uint32_t bit = 1u << (v & 31);
    if (!(*word & bit)) atomicOr(word, bit);
}

// Device state of a Dynamic-Cache refresh (eq. 6): the top-k selection's radix digits, the
// candidate count and the free-row stack.  Written by the refresh kernels only.
constexpr int kDynBins = 2048;   // 11-bit digits
struct DynState {
    int64_t n_cand;       // candidates of this refresh (touched nodes and members)
    int64_t remaining;    // rank still to place within the digits chosen so far
    uint32_t hi_prefix, hi_mask;   // digits chosen so far of the k-th largest key (high word),
    uint32_t lo_prefix, lo_mask;   // (low word), then among keys equal to it, of the largest
    uint32_t id_prefix, id_mask;   // id taken
    int64_t n_admit;      // nodes entering the cache in this refresh
    int64_t n_evict;      // members leaving it
    int64_t n_evict_resident;      // of which resident
    int64_t n_published;  // filled rows made resident by this refresh
    int64_t n_resident;   // members resident after it (the others wait for their fill)
    int64_t free_top;     // rows on the free-row stack
    int64_t members;      // rows in use after the refresh
    int64_t refreshes;
    uint32_t hist[kDynBins];
};

// Kernel launchers (each returns hipGetLastError()).
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t value, hipStream_t s);
hipError_t launch_classify(HopArgs a, hipStream_t s);
hipError_t launch_sample(const HopArgs &a, hipStream_t s);
hipError_t launch_relabel(RelabelArgs a, hipStream_t s);
// Look-back words a launch_relabel call needs in a.lb, besides its nbm ticket counters.
int64_t relabel_lb_words(const RelabelArgs &a);
hipError_t launch_dist(const DistArgs &a, hipStream_t s);

// Match: each id's position in the previous batch's (ascending) node list, or -1.  The gather
// codes such a row past the cache rows, so cache rows and list positions stay below kPrevCode.
constexpr int32_t kPrevCode = 1 << 30;
constexpr int64_t kPrevCodeBound = kPrevCode;
struct MatchArgs {
    const int32_t *ids;
    const int64_t *d_n;
    int64_t n_cap;
    const int32_t *prev_ids;
    const int64_t *d_prev_n;
    int64_t prev_cap;
    int32_t *match;        // [n_cap] out
    int64_t *d_matched;    // optional: += rows found
};
hipError_t launch_match(const MatchArgs &a, hipStream_t s);

// Overlap matrix of B ascending node lists: pairs (pa[y], pb[y]), pa < pb, one grid row each.
constexpr int64_t kOverlapChunk = 4096;   // elements of L_a per workgroup
struct OverlapArgs {
    const int32_t *ids[kMaxGroup];
    const int64_t *d_n[kMaxGroup];
    int64_t cap[kMaxGroup];
    int32_t B;
    int32_t npairs;
    uint8_t pa[kMaxGroup * (kMaxGroup - 1) / 2];
    uint8_t pb[kMaxGroup * (kMaxGroup - 1) / 2];
    unsigned long long *out;   // [B * B]
};
hipError_t launch_overlap(const OverlapArgs &a, hipStream_t s);

// The first union level of a super-batch as the concatenation of its sub-batches' seeds.
struct SeedConcatArgs {
    const int32_t *seeds[kMaxGroup];
    int64_t off[kMaxGroup + 1];   // sub-batch g's seeds go to positions off[g] .. off[g+1] - 1
    int32_t G;
    int32_t *U0;                  // [off[G]] out
    int64_t *d_U0;                // out: off[G]
    int32_t *upos;                // out: upos[g * P + i] = off[g] + i
    int64_t P;
    uint32_t *bitmap;             // node-id bitmap: each valid seed's bit is set
    int64_t num_nodes;
};
hipError_t launch_seed_concat(const SeedConcatArgs &a, hipStream_t s);
hipError_t launch_gather(const float *table, float *cache, const int32_t *slot, int64_t ld,
                         int64_t d, int64_t num_rows, const int32_t *ids, const int64_t *d_n,
                         int64_t n_cap, float *out, int64_t ld_out, int64_t *d_hits,
                         int32_t *status, hipStream_t s, const DynObserve *obs = nullptr,
                         double obs_w = 0.0, const int32_t *match = nullptr,
                         const float *prev = nullptr, int64_t ld_prev = 0);
// One sub-batch of a batched gather: out[r] = row ids[r] for r < n (n = *d_n, or n_cap); obs_w:
// its Dynamic-Cache observation weight.
struct GatherSeg {
    const int32_t *ids;
    const int64_t *d_n;
    int64_t n_cap;
    float *out;
    double obs_w;
};

struct GatherBatchArgs {
    GatherSeg seg[kMaxGroup];
    int32_t nseg;
    const float *table;
    float *cache;      // written only to fill reserved Dynamic-Cache rows
    const int32_t *slot;
    int64_t ld;
    int32_t d;
    int64_t num_rows;
    int64_t ld_out;
    int32_t *status;
    uint32_t cpr;      // set by the launcher
    DynObserve obs;    // obs.score NULL: no observation
    int64_t *d_hits;   // rows read from the cache are added here (NULL: not counted)
};

// Gather of up to kMaxGroup sub-batches in one launch (rows_cap: the sub-batches' total row
// capacity).  Rows that are not 16-byte aligned take the flat kernel, one launch per sub-batch.
hipError_t launch_gather_batch(GatherBatchArgs a, int64_t rows_cap, hipStream_t s);

// One mean-aggregation block: destinations [0, n) (n = *d_n, or n_cap if d_n is NULL) with
// edges indptr / lid (lid has e_cap entries), sources src [n_src rows], output out.
struct MeanJob {
    const int32_t *indptr;
    const int32_t *lid;
    int64_t e_cap;
    const int64_t *d_n;
    int64_t n_cap;
    const float *src;
    int64_t n_src;
    float *out;
};
constexpr int kMaxMeanSegs = 16;
// All jobs share d and the row strides; up to kMaxMeanSegs jobs go into one launch.  max_c is a
// typical (or the largest) edge count per destination; it only picks the load depth.
hipError_t launch_mean(const MeanJob *jobs, int njobs, int64_t ld_src, int64_t ld_out, int64_t d,
                       int32_t max_c, int32_t *status, hipStream_t s);
// One block whose destinations are the union of G sub-batches' destinations: destination r's mean
// is stored to row inv[r * G + g] - 1 of outs[g] for every g whose bit is set in inv_mask[r] (job.out
// is not used; entries without their bit are never used).
hipError_t launch_mean_scatter(const MeanJob &job, const int32_t *inv, const uint32_t *inv_mask,
                               int G, float *const *outs, int64_t ld_src, int64_t ld_out, int64_t d,
                               int32_t *status, hipStream_t s);
// The dense UPDATE of a GraphSAGE-mean layer: out = act([src[dst_lid] || agg] W + bias) on the
// matrix cores (fp32); rows beyond *d_n (when given) are skipped.
hipError_t launch_sage_update(const int32_t *dst_lid, const int64_t *d_n, int64_t n_cap,
                              const float *src, int64_t ld_src, int64_t n_src, const float *agg,
                              int64_t ld_agg, int64_t d, const float *W, const float *bias,
                              int64_t d_out, int32_t relu, float *out, int64_t ld_out,
                              int32_t *status, hipStream_t s);
// Gather of the union of a super-batch's gathered node sets: union row r < *d_n (global id
// ids[r]) is read once and stored to every sub-batch g whose relabel bitmap (bm + g * words, word
// prefixes wp + g * words) holds the row's key -- the id when by_id, else r -- at the key's rank
// in that bitmap.
// Rows must be 16-byte aligned (ld and ld_out multiples of 4, aligned bases): otherwise
// hipErrorInvalidValue is returned and nothing is launched.
// Adjacency cache set-up: deg[i] = degree of hot[i]; then rows of the selected nodes copied to
// rows + off[i] and adj_off[node[i]] = off[i].
hipError_t launch_adj_degrees(const void *indptr, int32_t ib, const int32_t *hot, int64_t n,
                              int64_t *deg, hipStream_t s);
hipError_t launch_adj_fill(const void *indptr, int32_t ib, const int32_t *indices,
                           const int32_t *node, const int64_t *off, int64_t n, int32_t *rows,
                           int64_t *adj_off, hipStream_t s);
hipError_t launch_gather_union(const float *table, int64_t ld, int64_t d, int64_t num_rows,
                               const int32_t *ids, const int64_t *d_n, int64_t n_cap,
                               const uint2 *rd, int64_t words, int by_id,
                               int G, float *const *outs, int64_t ld_out, int32_t *status,
                               hipStream_t s);
hipError_t launch_cache_fill(const float *table, int64_t ld, int64_t d, int64_t num_rows,
                             const int32_t *hot, int64_t rows, float *cache, int32_t *slot,
                             int32_t *status, hipStream_t s);

// Dynamic-Cache (GARDEN, Sec. IV.B, eq. 6).  Set-up: free rows 0..k-1 on the stack, no row held
// or filled, state zero.
hipError_t launch_dyn_init(DynState *st, int32_t *free_rows, int32_t *row_node, uint8_t *filled,
                           int64_t k, hipStream_t s);
// score[v] *= factor for every node (factor a power of two: exact for normal numbers).
hipError_t launch_dyn_rescale(double *score, int64_t n, double factor, hipStream_t s);
// One refresh: filled rows become resident; then the k_dyn touched nodes of largest scaled score
// (ties: smaller id first) become the members; members left out lose their slot and row, nodes
// taken in get a reserved row (filled by a later gather).  The touched bitmap is left holding
// exactly the members.  publish_only: only the first step (a frozen cache).
struct DynRefreshArgs {
    DynState *st;
    double *score;
    uint32_t *touched;
    uint32_t *member;     // [ceil(num_rows / 32)] Dynamic-Cache members
    int64_t num_rows;
    uint32_t *cand;       // [num_rows] candidate ids, bit 31 set for members
    uint32_t *key_hi;     // [num_rows] high and low words of the bits of their scaled scores
    uint32_t *key_lo;
    int32_t *free_rows;   // [k_dyn] free-row stack
    int32_t *admit;       // [k_dyn] nodes taken in
    int32_t *row_node;    // [k_dyn] member holding each row, -1 if free
    uint8_t *filled;      // [k_dyn rounded up to 4]
    int64_t k_dyn;
    int32_t static_rows;
    int32_t *slot;
    int32_t *status;
};
hipError_t launch_dyn_refresh(const DynRefreshArgs &a, bool publish_only, hipStream_t s);
// Inspection: out_score[v] = score[v] * scale and out_member[v] = 1 for resident Dynamic-Cache
// members, 2 for members waiting for their fill, else 0 (either output may be NULL).
hipError_t launch_dyn_state(const double *score, int64_t n, double scale, const int32_t *slot,
                            int32_t static_rows, double *out_score, uint8_t *out_member,
                            hipStream_t s);

}  // namespace gnnmb
