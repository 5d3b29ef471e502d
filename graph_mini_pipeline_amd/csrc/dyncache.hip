// Dynamic-Cache refresh (gfx950).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. IV.B, eq. (5)-(6): a bounded secondary feature cache for residual hot rows
// (requested rows that the static cache misses), ranked by an exponentially weighted moving
// average of each node's accesses and refreshed every T_update mini-batches with the K_dyn nodes
// of highest score.
//
// Candidates.  The gather kernels add each mini-batch's weight to the scaled score S(v) of every
// residual row they read and mark v in the touched bitmap; a refresh leaves exactly its members
// marked.  A node marked in neither way ranked below every member at the previous refresh and its
// score has not changed since, while each member's only grew, so the top K_dyn of all nodes are
// among the marked ones: the refresh ranks those alone.
//
// Selection.  Radix select, most significant digit first, over the candidates' keys (the bit
// patterns of non-negative doubles order as the doubles do): 8 passes of 8-bit digits find the
// K_dyn-th largest key tau and how many of the K_dyn take that key; 4 passes over the ids of the
// candidates whose key is tau find the largest id taken, iota.  Members: key > tau, or key == tau
// and id <= iota, i.e. the first K_dyn in the order (score descending, id ascending); every
// candidate when there are no more than K_dyn.
//
// Residency.  A member left out gives its row back to a free-row stack and its slot becomes -1;
// a node taken in pops a row, its table row is copied there, then its slot is set.  The kernels
// run in order on one stream, so a gather issued before the refresh on that stream reads the old
// rows and one issued after it the new ones.
#include "common.hpp"

namespace gnnmb {

constexpr int kDynThreads = 256;
constexpr int kDynWords = 16;   // touched-bitmap words per thread of the compaction
constexpr int kDynItems = 8;    // candidates per thread of the apply step
constexpr int kDynKeyPasses = 8;
constexpr int kDynPasses = kDynKeyPasses + 4;

static unsigned grid_of(int64_t items, int64_t per_block, int64_t max_grid) {
    int64_t g = (items + per_block - 1) / per_block;
    g = g < 1 ? 1 : (g > max_grid ? max_grid : g);
    return static_cast<unsigned>(g);
}

__global__ __launch_bounds__(256) void k_dyn_init(DynState *st, int32_t *free_rows, int64_t k) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (int64_t r = i; r < k; r += static_cast<int64_t>(gridDim.x) * blockDim.x)
        free_rows[r] = static_cast<int32_t>(k - 1 - r);   // row 0 on top
    if (blockIdx.x == 0) {
        st->hist[threadIdx.x] = 0;
        if (threadIdx.x == 0) {
            st->n_cand = 0;
            st->remaining = 0;
            st->key_prefix = 0;
            st->key_mask = 0;
            st->id_prefix = 0;
            st->id_mask = 0;
            st->n_admit = 0;
            st->n_evict = 0;
            st->free_top = k;
            st->members = 0;
            st->refreshes = 0;
        }
    }
}

__global__ __launch_bounds__(256) void k_dyn_rescale(double *score, int64_t n, double factor) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const double x = score[i];
        if (x != 0.0) score[i] = x * factor;
    }
}

// Clears the counters and digits of one refresh (one workgroup of 256 threads).
__global__ __launch_bounds__(256) void k_dyn_begin(DynState *st, int64_t k) {
    st->hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        st->n_cand = 0;
        st->remaining = k;
        st->key_prefix = 0;
        st->key_mask = 0;
        st->id_prefix = 0;
        st->id_mask = 0;
        st->n_admit = 0;
        st->n_evict = 0;
    }
}

// Candidates: the marked nodes, with the bit patterns of their scores; the bitmap is cleared as
// it is read.  Each workgroup takes kDynThreads * kDynWords words and reserves its candidates'
// positions with one atomic add, so the list is in no particular order.
__global__ __launch_bounds__(256) void k_dyn_compact(DynRefreshArgs a, int64_t words) {
    __shared__ uint32_t s_red[kDynThreads / 64];
    __shared__ unsigned long long s_base;
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kDynThreads * kDynWords + threadIdx.x;
    uint32_t w[kDynWords];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kDynWords; ++j) {
        const int64_t wi = w0 + static_cast<int64_t>(j) * kDynThreads;
        w[j] = wi < words ? a.touched[wi] : 0u;
        cnt += __popc(w[j]);
    }
    uint32_t tot;
    const uint32_t excl = block_exclusive_scan<uint32_t, kDynThreads>(cnt, &tot, s_red);
    if (threadIdx.x == 0)
        s_base = tot ? atomicAdd(reinterpret_cast<unsigned long long *>(&a.st->n_cand),
                                 static_cast<unsigned long long>(tot))
                     : 0ull;
    __syncthreads();
    int64_t pos = static_cast<int64_t>(s_base) + excl;
#pragma unroll
    for (int j = 0; j < kDynWords; ++j) {
        uint32_t x = w[j];
        if (x == 0u) continue;
        const int64_t wi = w0 + static_cast<int64_t>(j) * kDynThreads;
        a.touched[wi] = 0u;
        while (x) {
            const int b = __ffs(x) - 1;
            x &= x - 1u;
            const int64_t v = wi * 32 + b;
            if (v >= a.num_rows || pos >= a.num_rows) {   // no bit is set past the nodes
                set_status(a.status, GNN_ERR_INTERNAL);
                continue;
            }
            a.cand[pos] = static_cast<int32_t>(v);
            a.keys[pos] = static_cast<uint64_t>(__double_as_longlong(a.score[v]));
            ++pos;
        }
    }
}

// Histogram of one digit over the candidates that agree with the digits chosen so far: passes
// 0..7 the key's bytes from the most significant, passes 8..11 the id's bytes among the keys
// equal to tau.  Nothing to do when every candidate is taken.
__global__ __launch_bounds__(256) void k_dyn_hist(DynRefreshArgs a, int pass) {
    __shared__ uint32_t h[256];
    const int64_t n = a.st->n_cand < a.num_rows ? a.st->n_cand : a.num_rows;
    if (n <= a.k_dyn) return;
    h[threadIdx.x] = 0u;
    __syncthreads();
    const uint64_t kp = a.st->key_prefix, km = a.st->key_mask;
    const uint32_t ip = a.st->id_prefix, im = a.st->id_mask;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kDynThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kDynThreads + threadIdx.x; i < n; i += stride) {
        const uint64_t key = a.keys[i];
        if ((key & km) != kp) continue;
        uint32_t bin;
        if (pass < kDynKeyPasses) {
            bin = static_cast<uint32_t>(key >> (56 - 8 * pass)) & 255u;
        } else {
            const uint32_t id = static_cast<uint32_t>(a.cand[i]);
            if ((id & im) != ip) continue;
            bin = (id >> (24 - 8 * (pass - kDynKeyPasses))) & 255u;
        }
        atomicAdd(&h[bin], 1u);
    }
    __syncthreads();
    if (h[threadIdx.x]) atomicAdd(&a.st->hist[threadIdx.x], h[threadIdx.x]);
}

// The digit of one pass (one workgroup): key bytes are taken largest first, id bytes smallest
// first; the bin where the running count reaches the rank still to place is the digit, and the
// rank left is the rank within it.  The histogram is cleared for the next pass.
__global__ __launch_bounds__(256) void k_dyn_pick(DynRefreshArgs a, int pass) {
    __shared__ uint32_t s_red[kDynThreads / 64];
    __shared__ int64_t s_rem;
    DynState *st = a.st;
    if (st->n_cand <= a.k_dyn) return;
    const bool by_key = pass < kDynKeyPasses;
    const int bin = by_key ? 255 - static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x);
    if (threadIdx.x == 0) s_rem = st->remaining;
    const uint32_t c = st->hist[bin];
    __syncthreads();
    const int64_t rem = s_rem;
    uint32_t tot;
    const uint32_t before = block_exclusive_scan<uint32_t, kDynThreads>(c, &tot, s_red);
    if (static_cast<int64_t>(before) < rem && rem <= static_cast<int64_t>(before) + c) {
        st->remaining = rem - before;
        if (by_key) {
            const int sh = 56 - 8 * pass;
            st->key_prefix |= static_cast<uint64_t>(bin) << sh;
            st->key_mask |= 0xFFull << sh;
        } else {
            const int sh = 24 - 8 * (pass - kDynKeyPasses);
            st->id_prefix |= static_cast<uint32_t>(bin) << sh;
            st->id_mask |= 0xFFu << sh;
        }
    }
    if (threadIdx.x == 0 && static_cast<int64_t>(tot) < rem) set_status(a.status, GNN_ERR_INTERNAL);
    st->hist[bin] = 0u;
}

// Members of the new cache marked again in the bitmap; members left out lose their slot and push
// their row onto the free stack; nodes taken in are listed.  One reservation per workgroup for
// each list.
__global__ __launch_bounds__(256) void k_dyn_apply(DynRefreshArgs a) {
    __shared__ uint32_t s_red[kDynThreads / 64];
    __shared__ unsigned long long s_abase, s_ebase;
    const DynState *st = a.st;
    const int64_t n = st->n_cand < a.num_rows ? st->n_cand : a.num_rows;
    const bool all = n <= a.k_dyn;
    const uint64_t tau = st->key_prefix;
    const uint32_t iota = st->id_prefix;
    const int64_t free_top = st->free_top;
    constexpr int64_t kPerBlock = static_cast<int64_t>(kDynThreads) * kDynItems;
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kPerBlock; i0 < n;
         i0 += static_cast<int64_t>(gridDim.x) * kPerBlock) {
        int32_t v[kDynItems], row[kDynItems];
        int kind[kDynItems];   // 0: unchanged, 1: taken in, 2: left out
        uint32_t na = 0, ne = 0;
#pragma unroll
        for (int j = 0; j < kDynItems; ++j) {
            const int64_t i = i0 + threadIdx.x + static_cast<int64_t>(j) * kDynThreads;
            kind[j] = 0;
            v[j] = -1;
            row[j] = -1;
            if (i >= n) continue;
            const int32_t u = a.cand[i];
            if (u < 0 || u >= a.num_rows) {
                set_status(a.status, GNN_ERR_INTERNAL);
                continue;
            }
            const uint64_t key = a.keys[i];
            const bool sel = all || key > tau || (key == tau && static_cast<uint32_t>(u) <= iota);
            const int32_t sl = a.slot[u];
            const bool member = sl >= a.static_rows;
            v[j] = u;
            if (sel) {
                atomicOr(a.touched + (u >> 5), 1u << (u & 31));
                if (!member) {
                    kind[j] = 1;
                    ++na;
                }
            } else if (member) {
                kind[j] = 2;
                row[j] = sl - a.static_rows;
                a.slot[u] = -1;
                ++ne;
            }
        }
        uint32_t ta, te;
        const uint32_t ea = block_exclusive_scan<uint32_t, kDynThreads>(na, &ta, s_red);
        const uint32_t ee = block_exclusive_scan<uint32_t, kDynThreads>(ne, &te, s_red);
        if (threadIdx.x == 0) {
            s_abase = ta ? atomicAdd(reinterpret_cast<unsigned long long *>(&a.st->n_admit),
                                     static_cast<unsigned long long>(ta))
                         : 0ull;
            s_ebase = te ? atomicAdd(reinterpret_cast<unsigned long long *>(&a.st->n_evict),
                                     static_cast<unsigned long long>(te))
                         : 0ull;
        }
        __syncthreads();
        int64_t pa = static_cast<int64_t>(s_abase) + ea;
        int64_t pe = free_top + static_cast<int64_t>(s_ebase) + ee;
#pragma unroll
        for (int j = 0; j < kDynItems; ++j) {
            if (kind[j] == 1) {
                if (pa < a.k_dyn) a.admit[pa] = v[j];
                else set_status(a.status, GNN_ERR_INTERNAL);
                ++pa;
            } else if (kind[j] == 2) {
                if (pe < a.k_dyn && row[j] >= 0 && row[j] < a.k_dyn) a.free_rows[pe] = row[j];
                else set_status(a.status, GNN_ERR_INTERNAL);
                ++pe;
            }
        }
        __syncthreads();   // s_abase / s_ebase are rewritten by the next round
    }
}

// Nodes taken in: one wavefront per node pops row top - 1 - i of the free stack, copies the
// node's table row into it, then sets the node's slot.
__global__ __launch_bounds__(256) void k_dyn_admit(DynRefreshArgs a) {
    const DynState *st = a.st;
    const int64_t na = st->n_admit;
    const int64_t top = st->free_top + st->n_evict;
    const int lane = lane_id();
    const int64_t wstride = static_cast<int64_t>(gridDim.x) * (kDynThreads / 64);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * (kDynThreads / 64) + (threadIdx.x >> 6);
         i < na; i += wstride) {
        if (i >= top || top > a.k_dyn) {   // more nodes than free rows: cannot happen
            if (lane == 0) set_status(a.status, GNN_ERR_INTERNAL);
            continue;
        }
        const int32_t v = a.admit[i];
        const int32_t r = a.free_rows[top - 1 - i];
        if (v < 0 || v >= a.num_rows || r < 0 || r >= a.k_dyn) {
            if (lane == 0) set_status(a.status, GNN_ERR_INTERNAL);
            continue;
        }
        const float *src = a.table + static_cast<int64_t>(v) * a.ld;
        float *dst = a.cache + (static_cast<int64_t>(a.static_rows) + r) * a.ld;
        for (int64_t c = lane; c < a.d; c += 64) dst[c] = src[c];
        if (lane == 0) a.slot[v] = a.static_rows + r;
    }
}

__global__ void k_dyn_finish(DynState *st, int64_t k, int32_t *status) {
    int64_t top = st->free_top + st->n_evict - st->n_admit;
    if (top < 0 || top > k) {
        set_status(status, GNN_ERR_INTERNAL);
        top = top < 0 ? 0 : k;
    }
    st->free_top = top;
    st->members = k - top;
    st->refreshes += 1;
}

__global__ __launch_bounds__(256) void k_dyn_state(const double *score, int64_t n, double scale,
                                                   const int32_t *slot, int32_t static_rows,
                                                   double *out_score, uint8_t *out_member) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        if (out_score) out_score[i] = score[i] * scale;
        if (out_member) out_member[i] = slot[i] >= static_rows ? 1 : 0;
    }
}

hipError_t launch_dyn_init(DynState *st, int32_t *free_rows, int64_t k, hipStream_t s) {
    hipLaunchKernelGGL(k_dyn_init, dim3(grid_of(k, 256, 4096)), dim3(256), 0, s, st, free_rows, k);
    return hipGetLastError();
}

hipError_t launch_dyn_rescale(double *score, int64_t n, double factor, hipStream_t s) {
    hipLaunchKernelGGL(k_dyn_rescale, dim3(grid_of(n, 256 * 8, 8192)), dim3(256), 0, s, score, n,
                       factor);
    return hipGetLastError();
}

hipError_t launch_dyn_refresh(const DynRefreshArgs &a, hipStream_t s) {
    if (a.k_dyn < 1 || a.num_rows < 1) return hipErrorInvalidValue;
    const int64_t words = (a.num_rows + 31) / 32;
    hipLaunchKernelGGL(k_dyn_begin, dim3(1), dim3(kDynThreads), 0, s, a.st, a.k_dyn);
    hipLaunchKernelGGL(k_dyn_compact, dim3(grid_of(words, kDynThreads * kDynWords, 1 << 30)),
                       dim3(kDynThreads), 0, s, a, words);
    const unsigned hg = grid_of(a.num_rows, kDynThreads * 16, 1024);
    for (int pass = 0; pass < kDynPasses; ++pass) {
        hipLaunchKernelGGL(k_dyn_hist, dim3(hg), dim3(kDynThreads), 0, s, a, pass);
        hipLaunchKernelGGL(k_dyn_pick, dim3(1), dim3(kDynThreads), 0, s, a, pass);
    }
    hipLaunchKernelGGL(k_dyn_apply, dim3(grid_of(a.num_rows, kDynThreads * kDynItems, 2048)),
                       dim3(kDynThreads), 0, s, a);
    hipLaunchKernelGGL(k_dyn_admit, dim3(grid_of(a.k_dyn, kDynThreads / 64, 4096)),
                       dim3(kDynThreads), 0, s, a);
    hipLaunchKernelGGL(k_dyn_finish, dim3(1), dim3(1), 0, s, a.st, a.k_dyn, a.status);
    return hipGetLastError();
}

hipError_t launch_dyn_state(const double *score, int64_t n, double scale, const int32_t *slot,
                            int32_t static_rows, double *out_score, uint8_t *out_member,
                            hipStream_t s) {
    if (!out_score && !out_member) return hipSuccess;
    hipLaunchKernelGGL(k_dyn_state, dim3(grid_of(n, 256 * 8, 8192)), dim3(256), 0, s, score, n,
                       scale, slot, static_rows, out_score, out_member);
    return hipGetLastError();
}

}  // namespace gnnmb
