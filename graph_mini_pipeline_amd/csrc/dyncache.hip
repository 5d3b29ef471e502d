// Dynamic-Cache refresh (gfx950).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. IV.B, eq. (5)-(6): a bounded secondary feature cache for residual hot rows
// (requested rows that the static cache misses), ranked by an exponentially weighted moving
// average of each node's accesses and refreshed every T_update mini-batches with the K_dyn nodes
// of highest score.
//
// Candidates.  The gather kernels add each mini-batch's weight to the scaled score S(v) of every
// residual row they read and mark v in the touched bitmap; the members are marked in a bitmap of
// their own.  A node in neither ranked below every member at the previous refresh and its score
// has not changed since, while each member's only grew, so the top K_dyn of all nodes are among
// the nodes in either bitmap: the refresh ranks those alone.  The compaction lists them (with the
// high and low words of their keys, read with many loads in flight) and clears the touched bitmap.
//
// Selection.  Radix select, most significant digit first, over the candidates' keys (the bit
// patterns of non-negative doubles order as the doubles do): 6 passes of 11-bit digits (three on
// the high word, which alone is read until it is fixed, three on the low word) find the K_dyn-th
// largest key tau and how many of the K_dyn take that key; 3 passes over the ids of the
// candidates whose key is tau find the largest id taken, iota.  Members: key > tau, or key == tau
// and id <= iota, i.e. the first K_dyn in the order (score descending, id ascending); every
// candidate when there are no more than K_dyn.  A digit that every lane of a wavefront shares
// (the high digits mostly are) is counted with one LDS atomic per wavefront.  Only the candidates
// whose membership changes are then touched: the rest keep their slot, row and member bit.
//
// Residency.  A member left out gives its row back to a free-row stack and its slot becomes -1;
// a node taken in pops a row, which its slot reserves (slot -2 - row).  Nothing is copied: the
// next gather that reads the node's row from the table (a miss either way) also writes it to the
// reserved row and marks the row filled, and a refresh first makes every filled row resident.
// Copying the rows in at the refresh instead (as eq. (6) might be read) moved as many rows over
// the host link as the misses it then saved on the billion-edge workload, where few misses
// recur.  A refresh runs after every gather issued before it and before every gather issued
// after it (one stream, or streams joined around it), so no gather sees a row change under it,
// and a filled row is resident only once the gather that wrote it has finished.
#include "common.hpp"

namespace gnnmb {

constexpr int kDynThreads = 256;
constexpr int kDynWords = 16;   // bitmap words per thread of the compaction
constexpr int kDynItems = 8;    // candidates per thread of the apply step

// Digits of the passes: word 0 the key's high word (bit 31, the sign, is 0), 1 its low word,
// 2 the id; each as shift and width.
struct DynDigit {
    int word, shift, bits;
};
constexpr int kDynPasses = 9;
__host__ __device__ constexpr DynDigit dyn_digit(int p) {
    return p == 0 ? DynDigit{0, 20, 11} : p == 1 ? DynDigit{0, 9, 11} : p == 2 ? DynDigit{0, 0, 9}
         : p == 3 ? DynDigit{1, 21, 11} : p == 4 ? DynDigit{1, 10, 11} : p == 5 ? DynDigit{1, 0, 10}
         : p == 6 ? DynDigit{2, 20, 11} : p == 7 ? DynDigit{2, 9, 11} : DynDigit{2, 0, 9};
}

static unsigned grid_of(int64_t items, int64_t per_block, int64_t max_grid) {
    int64_t g = (items + per_block - 1) / per_block;
    g = g < 1 ? 1 : (g > max_grid ? max_grid : g);
    return static_cast<unsigned>(g);
}

__global__ __launch_bounds__(256) void k_dyn_init(DynState *st, int32_t *free_rows, int32_t *row_node,
                                                  uint8_t *filled, int64_t k) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t k4 = (k + 3) / 4 * 4;
    for (int64_t r = i; r < k4; r += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        if (r < k) {
            free_rows[r] = static_cast<int32_t>(k - 1 - r);   // row 0 on top
            row_node[r] = -1;
        }
        filled[r] = 0;
    }
    if (blockIdx.x == 0) {
        for (int b = threadIdx.x; b < kDynBins; b += blockDim.x) st->hist[b] = 0;
        if (threadIdx.x == 0) {
            st->n_cand = 0;
            st->remaining = 0;
            st->hi_prefix = st->hi_mask = st->lo_prefix = st->lo_mask = 0;
            st->id_prefix = st->id_mask = 0;
            st->n_admit = st->n_evict = st->n_evict_resident = 0;
            st->n_published = st->n_resident = 0;
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

// Clears the counters and digits of one refresh (the histogram is left zero by the picks); of a
// publish-only pass, just its count.
__global__ void k_dyn_begin(DynState *st, int64_t k, int publish_only) {
    st->n_published = 0;
    if (publish_only) return;
    st->n_cand = 0;
    st->remaining = k;
    st->hi_prefix = st->hi_mask = st->lo_prefix = st->lo_mask = 0;
    st->id_prefix = st->id_mask = 0;
    st->n_admit = st->n_evict = st->n_evict_resident = 0;
}

// Filled rows of pending members become resident; their flags are cleared (a resident row is
// never marked again), four rows per flag word.
__global__ __launch_bounds__(256) void k_dyn_publish(DynRefreshArgs a) {
    __shared__ uint32_t s_red[kDynThreads / 64];
    uint32_t n = 0;
    const int64_t nw = (a.k_dyn + 3) / 4;
    uint32_t *fw = reinterpret_cast<uint32_t *>(a.filled);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kDynThreads;
    for (int64_t w = static_cast<int64_t>(blockIdx.x) * kDynThreads + threadIdx.x; w < nw; w += stride) {
        const uint32_t f = fw[w];
        if (f == 0u) continue;
        fw[w] = 0u;
        for (int q = 0; q < 4; ++q) {
            const int64_t r = w * 4 + q;
            if (((f >> (8 * q)) & 0xFFu) == 0u || r >= a.k_dyn) continue;
            const int32_t v = a.row_node[r];
            if (v < 0 || v >= a.num_rows) continue;
            if (a.slot[v] == -2 - static_cast<int32_t>(r)) {
                a.slot[v] = a.static_rows + static_cast<int32_t>(r);
                ++n;
            }
        }
    }
    uint32_t tot;
    (void)block_exclusive_scan<uint32_t, kDynThreads>(n, &tot, s_red);
    if (threadIdx.x == 0 && tot)
        atomicAdd(reinterpret_cast<unsigned long long *>(&a.st->n_published),
                  static_cast<unsigned long long>(tot));
}

// Candidates: the nodes marked in the touched or the member bitmap (bit 31 of the entry: a
// member), then the two words of their keys; the touched bitmap is cleared as it is read.  Each
// workgroup takes kDynThreads * kDynWords words and reserves its positions with one atomic add,
// so the list is in no particular order.
__global__ __launch_bounds__(256) void k_dyn_compact(DynRefreshArgs a, int64_t words) {
    __shared__ uint32_t s_red[kDynThreads / 64];
    __shared__ unsigned long long s_base;
    __shared__ uint32_t s_tot;
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kDynThreads * kDynWords + threadIdx.x;
    uint32_t w[kDynWords], m[kDynWords];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kDynWords; ++j) {
        const int64_t wi = w0 + static_cast<int64_t>(j) * kDynThreads;
        uint32_t t = 0u;
        m[j] = 0u;
        if (wi < words) {
            t = a.touched[wi];
            m[j] = a.member[wi];
        }
        w[j] = t | m[j];
        cnt += __popc(w[j]);
        if (t) a.touched[wi] = 0u;
    }
    uint32_t tot;
    const uint32_t excl = block_exclusive_scan<uint32_t, kDynThreads>(cnt, &tot, s_red);
    if (threadIdx.x == 0) {
        s_base = tot ? atomicAdd(reinterpret_cast<unsigned long long *>(&a.st->n_cand),
                                 static_cast<unsigned long long>(tot))
                     : 0ull;
        s_tot = tot;
    }
    __syncthreads();
    const int64_t base = static_cast<int64_t>(s_base);
    int64_t pos = base + excl;
#pragma unroll
    for (int j = 0; j < kDynWords; ++j) {
        uint32_t x = w[j];
        const int64_t wi = w0 + static_cast<int64_t>(j) * kDynThreads;
        while (x) {
            const int b = __ffs(x) - 1;
            x &= x - 1u;
            const int64_t v = wi * 32 + b;
            if (v >= a.num_rows || pos >= a.num_rows) {   // no bit is set past the nodes
                set_status(a.status, GNN_ERR_INTERNAL);
                continue;
            }
            a.cand[pos] = static_cast<uint32_t>(v) | (((m[j] >> b) & 1u) << 31);
            ++pos;
        }
    }
    __syncthreads();   // the block's entries are read back below by other threads
    const int64_t end = base + s_tot < a.num_rows ? base + s_tot : a.num_rows;
    constexpr int L = 4;
    for (int64_t i0 = base + threadIdx.x; i0 < end; i0 += L * kDynThreads) {
        uint64_t key[L];
#pragma unroll
        for (int q = 0; q < L; ++q) {
            const int64_t i = i0 + static_cast<int64_t>(q) * kDynThreads;
            key[q] = i < end ? static_cast<uint64_t>(__double_as_longlong(
                                   a.score[a.cand[i] & 0x7FFFFFFFu]))
                             : 0ull;
        }
#pragma unroll
        for (int q = 0; q < L; ++q) {
            const int64_t i = i0 + static_cast<int64_t>(q) * kDynThreads;
            if (i >= end) continue;
            a.key_hi[i] = static_cast<uint32_t>(key[q] >> 32);
            a.key_lo[i] = static_cast<uint32_t>(key[q]);
        }
    }
}

// Histogram of one digit over the candidates that agree with the digits chosen so far.  The low
// word and the id are read only for candidates that agree on what precedes them.  Nothing to do
// when every candidate is taken.
__global__ __launch_bounds__(256) void k_dyn_hist(DynRefreshArgs a, int pass) {
    __shared__ uint32_t h[kDynBins];
    const int64_t n = a.st->n_cand < a.num_rows ? a.st->n_cand : a.num_rows;
    if (n <= a.k_dyn) return;
    for (int b = threadIdx.x; b < kDynBins; b += kDynThreads) h[b] = 0u;
    __syncthreads();
    const DynDigit dg = dyn_digit(pass);
    const uint32_t hp = a.st->hi_prefix, hm = a.st->hi_mask;
    const uint32_t lp = a.st->lo_prefix, lm = a.st->lo_mask;
    const uint32_t ip = a.st->id_prefix, im = a.st->id_mask;
    const uint32_t dmask = (1u << dg.bits) - 1u;
    const int lane = lane_id();
    const int64_t wave0 = (static_cast<int64_t>(blockIdx.x) * kDynThreads + (threadIdx.x & ~63u));
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kDynThreads;
    for (int64_t i0 = wave0; i0 < n; i0 += stride) {   // wavefront-uniform bound
        const int64_t i = i0 + lane;
        bool match = i < n;
        uint32_t x = 0u;
        if (match) {
            x = a.key_hi[i];
            match = (x & hm) == hp;
        }
        if (dg.word >= 1 && match) {
            x = a.key_lo[i];
            match = (x & lm) == lp;
        }
        if (dg.word == 2 && match) {
            x = a.cand[i] & 0x7FFFFFFFu;
            match = (x & im) == ip;
        }
        const uint32_t bin = (x >> dg.shift) & dmask;
        const uint64_t mk = __ballot(match);
        if (mk == 0ull) continue;
        const int src = __ffsll(static_cast<unsigned long long>(mk)) - 1;
        const uint32_t b0 = __shfl(bin, src, 64);
        const uint64_t same = __ballot(match && bin == b0);
        if (same == mk) {
            if (lane == src) atomicAdd(&h[b0], static_cast<uint32_t>(__popcll(mk)));
        } else if (match) {
            atomicAdd(&h[bin], 1u);
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < kDynBins; b += kDynThreads)
        if (h[b]) atomicAdd(&a.st->hist[b], h[b]);
}

// The digit of one pass (one workgroup): key digits are taken largest first, id digits smallest
// first; the bin where the running count reaches the rank still to place is the digit, and the
// rank left is the rank within it.  The histogram is cleared for the next pass.
__global__ __launch_bounds__(256) void k_dyn_pick(DynRefreshArgs a, int pass) {
    constexpr int PER = kDynBins / kDynThreads;
    __shared__ uint32_t s_red[kDynThreads / 64];
    __shared__ int64_t s_rem;
    DynState *st = a.st;
    if (st->n_cand <= a.k_dyn) return;
    const DynDigit dg = dyn_digit(pass);
    const bool desc = dg.word < 2;
    if (threadIdx.x == 0) s_rem = st->remaining;
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int j = static_cast<int>(threadIdx.x) * PER + q;   // scan order
        const int bin = desc ? kDynBins - 1 - j : j;
        c[q] = st->hist[bin];
        sum += c[q];
    }
    __syncthreads();
    const int64_t rem = s_rem;
    uint32_t tot;
    const uint32_t before = block_exclusive_scan<uint32_t, kDynThreads>(sum, &tot, s_red);
    int64_t run = before;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int j = static_cast<int>(threadIdx.x) * PER + q;
        const uint32_t bin = static_cast<uint32_t>(desc ? kDynBins - 1 - j : j);
        if (run < rem && rem <= run + c[q]) {
            st->remaining = rem - run;
            const uint32_t dm = ((1u << dg.bits) - 1u) << dg.shift;
            if (dg.word == 0) {
                st->hi_prefix |= bin << dg.shift;
                st->hi_mask |= dm;
            } else if (dg.word == 1) {
                st->lo_prefix |= bin << dg.shift;
                st->lo_mask |= dm;
            } else {
                st->id_prefix |= bin << dg.shift;
                st->id_mask |= dm;
            }
        }
        run += c[q];
        if (c[q]) st->hist[bin] = 0u;
    }
    if (threadIdx.x == 0 && static_cast<int64_t>(tot) < rem) set_status(a.status, GNN_ERR_INTERNAL);
}

// Membership changes: a member left out loses its slot, row and member bit and pushes its row
// onto the free stack; a node taken in is listed.  One reservation per workgroup for each list;
// candidates whose membership stays are not touched.
__global__ __launch_bounds__(256) void k_dyn_apply(DynRefreshArgs a) {
    __shared__ uint32_t s_red[kDynThreads / 64];
    __shared__ unsigned long long s_abase, s_ebase;
    const DynState *st = a.st;
    const int64_t n = st->n_cand < a.num_rows ? st->n_cand : a.num_rows;
    const bool all = n <= a.k_dyn;
    const uint64_t tau = (static_cast<uint64_t>(st->hi_prefix) << 32) | st->lo_prefix;
    const uint32_t iota = st->id_prefix;
    const int64_t free_top = st->free_top;
    constexpr int64_t kPerBlock = static_cast<int64_t>(kDynThreads) * kDynItems;
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kPerBlock; i0 < n;
         i0 += static_cast<int64_t>(gridDim.x) * kPerBlock) {
        int32_t v[kDynItems], row[kDynItems];
        int kind[kDynItems];   // 0: unchanged, 1: taken in, 2: left out
        uint32_t na = 0, ne = 0, nres = 0;
#pragma unroll
        for (int j = 0; j < kDynItems; ++j) {
            const int64_t i = i0 + threadIdx.x + static_cast<int64_t>(j) * kDynThreads;
            kind[j] = 0;
            v[j] = -1;
            row[j] = -1;
            if (i >= n) continue;
            const uint32_t e = a.cand[i];
            const int32_t u = static_cast<int32_t>(e & 0x7FFFFFFFu);
            const bool member = (e >> 31) != 0u;
            if (u >= a.num_rows) {
                set_status(a.status, GNN_ERR_INTERNAL);
                continue;
            }
            bool sel = all;
            if (!sel) {
                const uint64_t key = (static_cast<uint64_t>(a.key_hi[i]) << 32) | a.key_lo[i];
                sel = key > tau || (key == tau && static_cast<uint32_t>(u) <= iota);
            }
            v[j] = u;
            if (sel && !member) {
                kind[j] = 1;
                ++na;
            } else if (!sel && member) {
                const int32_t sl = a.slot[u];
                const bool resident = sl >= a.static_rows;
                const int32_t r = resident ? sl - a.static_rows : (sl <= -2 ? -2 - sl : -1);
                if (r < 0 || r >= a.k_dyn) {
                    set_status(a.status, GNN_ERR_INTERNAL);
                    continue;
                }
                kind[j] = 2;
                row[j] = r;
                a.slot[u] = -1;
                a.row_node[r] = -1;
                atomicAnd(a.member + (u >> 5), ~(1u << (u & 31)));
                ++ne;
                nres += resident;
            }
        }
        uint32_t ta, te, tr;
        const uint32_t ea = block_exclusive_scan<uint32_t, kDynThreads>(na, &ta, s_red);
        const uint32_t ee = block_exclusive_scan<uint32_t, kDynThreads>(ne, &te, s_red);
        (void)block_exclusive_scan<uint32_t, kDynThreads>(nres, &tr, s_red);
        if (threadIdx.x == 0) {
            if (tr) atomicAdd(reinterpret_cast<unsigned long long *>(&a.st->n_evict_resident),
                              static_cast<unsigned long long>(tr));
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
                if (pe < a.k_dyn) a.free_rows[pe] = row[j];
                else set_status(a.status, GNN_ERR_INTERNAL);
                ++pe;
            }
        }
        __syncthreads();   // s_abase / s_ebase are rewritten by the next round
    }
}

// Nodes taken in: node i pops row top - 1 - i of the free stack, which its slot then reserves
// (not filled yet), and gets its member bit.
__global__ __launch_bounds__(256) void k_dyn_admit(DynRefreshArgs a) {
    const DynState *st = a.st;
    const int64_t na = st->n_admit;
    const int64_t top = st->free_top + st->n_evict;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kDynThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kDynThreads + threadIdx.x; i < na;
         i += stride) {
        if (i >= top || top > a.k_dyn) {   // more nodes than free rows: cannot happen
            set_status(a.status, GNN_ERR_INTERNAL);
            continue;
        }
        const int32_t v = a.admit[i];
        const int32_t r = a.free_rows[top - 1 - i];
        if (v < 0 || v >= a.num_rows || r < 0 || r >= a.k_dyn) {
            set_status(a.status, GNN_ERR_INTERNAL);
            continue;
        }
        a.row_node[r] = v;
        a.filled[r] = 0;
        a.slot[v] = -2 - r;
        atomicOr(a.member + (v >> 5), 1u << (v & 31));
    }
}

__global__ void k_dyn_finish(DynState *st, int64_t k, int32_t *status, int publish_only) {
    st->n_resident += st->n_published;
    if (publish_only) return;
    st->n_resident -= st->n_evict_resident;
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
        if (out_member) out_member[i] = slot[i] >= static_rows ? 1 : (slot[i] <= -2 ? 2 : 0);
    }
}

hipError_t launch_dyn_init(DynState *st, int32_t *free_rows, int32_t *row_node, uint8_t *filled,
                           int64_t k, hipStream_t s) {
    hipLaunchKernelGGL(k_dyn_init, dim3(grid_of(k, 256, 4096)), dim3(256), 0, s, st, free_rows,
                       row_node, filled, k);
    return hipGetLastError();
}

hipError_t launch_dyn_rescale(double *score, int64_t n, double factor, hipStream_t s) {
    hipLaunchKernelGGL(k_dyn_rescale, dim3(grid_of(n, 256 * 8, 8192)), dim3(256), 0, s, score, n,
                       factor);
    return hipGetLastError();
}

hipError_t launch_dyn_refresh(const DynRefreshArgs &a, bool publish_only, hipStream_t s) {
    if (a.k_dyn < 1 || a.num_rows < 1 || a.num_rows > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const int64_t words = (a.num_rows + 31) / 32;
    hipLaunchKernelGGL(k_dyn_begin, dim3(1), dim3(1), 0, s, a.st, a.k_dyn, publish_only ? 1 : 0);
    hipLaunchKernelGGL(k_dyn_publish, dim3(grid_of((a.k_dyn + 3) / 4, kDynThreads * 4, 2048)),
                       dim3(kDynThreads), 0, s, a);
    if (!publish_only) {
        hipLaunchKernelGGL(k_dyn_compact, dim3(grid_of(words, kDynThreads * kDynWords, 1 << 30)),
                           dim3(kDynThreads), 0, s, a, words);
        const unsigned hg = grid_of(a.num_rows, kDynThreads * 16, 1024);
        for (int pass = 0; pass < kDynPasses; ++pass) {
            hipLaunchKernelGGL(k_dyn_hist, dim3(hg), dim3(kDynThreads), 0, s, a, pass);
            hipLaunchKernelGGL(k_dyn_pick, dim3(1), dim3(kDynThreads), 0, s, a, pass);
        }
        hipLaunchKernelGGL(k_dyn_apply, dim3(grid_of(a.num_rows, kDynThreads * kDynItems, 2048)),
                           dim3(kDynThreads), 0, s, a);
        hipLaunchKernelGGL(k_dyn_admit, dim3(grid_of(a.k_dyn, kDynThreads, 4096)),
                           dim3(kDynThreads), 0, s, a);
    }
    hipLaunchKernelGGL(k_dyn_finish, dim3(1), dim3(1), 0, s, a.st, a.k_dyn, a.status,
                       publish_only ? 1 : 0);
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
