// Sort-unique relabel over the id universe (gfx950).
//
// Defines V_l = ascending unique of V_{l-1} and the sampled ids (GARDEN: Efficient GPU-Accelerated
// Billion-Scale GNN Training via Caching-Sampling-Batching Co-Design, Sec. II.B / Fig. 1: the
// destinations of a layer are part of its sources) and the local ids of both lists.  FastGL: A
// GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large Scale (Fused-Map)
// builds the map with atomic hash inserts, whose first-come local ids vary from run to run; here
// the order is ascending global id, so the result is a pure function of the input.
//
// Method: a counting sort with one bucket per id.  A bitmap of id_bound bits marks every id
// (atomicOr; the final bitmap does not depend on the order of the ors), a two-level scan of the
// per-word popcounts gives each word the number of set bits before it, set bits are written out in
// order (this is the sorted unique list), and the rank of id v is
//   prefix[v >> 5] + popcount(word[v >> 5] & ((1 << (v & 31)) - 1)).
// Work is O(id_bound / 32) words plus O(list length); every output position comes from a scan.
//
// One launch sequence serves several bitmaps at once: each id list names the bitmap it marks.
// The ids may also be positions in a sorted list of global ids (id_map): then the bitmap covers
// only that list, the emitted ids are id_map[position] (still ascending), and a device count
// bounds the live part of the bitmap, so that a super-batch relabels each sub-batch in the
// compact space of the super-batch's own sorted node set instead of the whole id range.
#include "common.hpp"

namespace gnnmb {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *p, int64_t n, uint32_t value) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = value;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *p, int64_t n, int32_t value) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = value;
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 256 * 4, 2048)), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3(grid_for(n, 256 * 4, 2048)), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

// Marks the ids of the lists of the given pass.  In pass 1 (the seed lists, marked before
// anything else) an id whose bit is already set is a duplicate within that list's bitmap.  The
// whole grid walks each list up to its actual (device) length, list after list: capacities can
// be many times the actual lengths.
// The lists' actual lengths (then the outputs' sizes), read once per workgroup with one load
// per list in flight, and their exclusive prefix: items of the lists are numbered in list order,
// so the grid spreads over the actual items of all lists at once.  Each list starts at a multiple
// of 64, so the items of one wavefront belong to one list (the padding items are skipped): the
// list's fields are then read with scalar loads, which do not wait on vector memory.
__device__ __forceinline__ void list_lengths(const RelabelArgs &a, int64_t *s_len, int64_t *s_off) {
    const int nl = a.nlist + a.nbm;
    if (threadIdx.x < static_cast<unsigned>(a.nlist))
        s_len[threadIdx.x] = load_count(a.list[threadIdx.x].d_n, a.list[threadIdx.x].cap);
    else if (threadIdx.x < static_cast<unsigned>(nl))
        s_len[threadIdx.x] = load_count(a.out[threadIdx.x - a.nlist].d_uniq,
                                        a.out[threadIdx.x - a.nlist].uniq_cap);
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t run = 0;
        for (int l = 0; l < nl; ++l) {
            s_off[l] = run;
            run += (s_len[l] + 63) & ~int64_t{63};
        }
        s_off[nl] = run;
    }
    __syncthreads();
}

// The list (among the first n of them) holding item t: the last l with s_off[l] <= t, the same
// for every active lane of the wavefront (found from the first one).
__device__ __forceinline__ int item_list(const int64_t *s_off, int n, int64_t t) {
    const int64_t t0 = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(t >> 32))) << 32) |
                       __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(t));
    int lo = 0, hi = n;  // s_off[lo] <= t0 < s_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= t0) lo = mid;
        else hi = mid;
    }
    return __builtin_amdgcn_readfirstlane(lo);
}

// Marks the ids of the lists of the given pass.  In pass 1 (the seed lists, marked before
// anything else) an id whose bit is already set is a duplicate within that list's bitmap.
// Only the lists' actual items are visited (capacities can be many times the actual lengths).
__global__ __launch_bounds__(256) void k_mark(RelabelArgs a, int32_t pass) {
    __shared__ int64_t s_len[3 * kMaxGroup];
    __shared__ int64_t s_off[3 * kMaxGroup + 1];
    list_lengths(a, s_len, s_off);
    const int64_t bound = relabel_bound(a);
    const int64_t total = s_off[a.nlist];
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int l = item_list(s_off, a.nlist, t);
        const IdList &L = a.list[l];
        if (L.pass != pass || t - s_off[l] >= s_len[l]) continue;
        const int32_t v = L.ids[t - s_off[l]];
        if (v < 0 || v >= bound) {
            set_status(a.status, GNN_ERR_OUT_OF_RANGE);
            continue;
        }
        const uint32_t bit = 1u << (v & 31);
        uint32_t *word = &a.bitmap[static_cast<int64_t>(L.bitmap) * a.W + (v >> 5)];
        if (a.bytes) a.bytes[static_cast<int64_t>(L.bitmap) * a.W * 32 + v] = 1;  // idempotent
        if (pass == 1) {
            const uint32_t old = atomicOr(word, bit);
            if (old & bit) set_status(a.status, GNN_ERR_INVALID_ARG);
        } else if (!a.bytes) {
            atomicOr(word, bit);  // result unused: the atomic is posted, the lane does not wait
        }
    }
}

// Words of each bitmap that can hold a set bit.
__device__ __forceinline__ int64_t live_words(const RelabelArgs &a) {
    if (a.d_bound == nullptr) return a.W;
    const int64_t w = (relabel_bound(a) + 31) >> 5;
    return w < a.W ? w : a.W;
}

// Per-tile popcounts; tile t covers kBitmapTile words of bitmap t / nbw.  Also zeroes the
// optional clear region (a bitmap no longer needed by this stream).
__global__ __launch_bounds__(kBitmapThreads) void k_popc_tiles(RelabelArgs a) {
    __shared__ uint32_t red[kBitmapThreads / 64];
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < a.clear_n;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x)
        a.clear_ptr[t] = 0u;
    const int bm = static_cast<int>(blockIdx.x) / a.nbw;
    const int lt = static_cast<int>(blockIdx.x) - bm * a.nbw;
    const uint32_t *words = a.bitmap + static_cast<int64_t>(bm) * a.W;
    const int64_t w0 = static_cast<int64_t>(lt) * kBitmapTile +
                       static_cast<int64_t>(threadIdx.x) * kBitmapWordsPerThread;
    const int64_t Wl = live_words(a);
    uint32_t c = 0;
    if (a.bytes) {
        // word w = the 32 bytes of ids 32w .. 32w+31 (each 0 or 1), packed
        uint32_t *wout = a.bitmap + static_cast<int64_t>(bm) * a.W;
        const uint8_t *bytes = a.bytes + static_cast<int64_t>(bm) * a.W * 32;
#pragma unroll
        for (int q = 0; q < kBitmapWordsPerThread; ++q) {
            const int64_t w = w0 + q;
            if (w >= Wl) break;
            const uint4 *p = reinterpret_cast<const uint4 *>(bytes + w * 32);
            const uint4 lo = p[0], hi = p[1];
            const uint32_t x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k)   // 4 bytes (0/1) -> 4 bits: products land on distinct bits
                word |= ((((x[k] & 0x01010101u) * 0x00204081u) >> 21) & 0xFu) << (4 * k);
            wout[w] = word;
            c += __popc(word);
        }
    } else {
#pragma unroll
        for (int q = 0; q < kBitmapWordsPerThread; ++q)
            if (w0 + q < Wl) c += __popc(words[w0 + q]);
    }
    c = wave_sum(c);
    if (lane_id() == 0) red[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int i = 0; i < kBitmapThreads / 64; ++i) s += red[i];
        a.bsum[blockIdx.x] = s;
    }
}

// Many tiles: workgroup b scans the tile popcounts of bitmap b in place and writes its size.
__global__ __launch_bounds__(1024) void k_popc_scan(RelabelArgs a) {
    __shared__ uint32_t smem[16];
    const int bm = blockIdx.x;
    uint32_t *bs = a.bsum + static_cast<int64_t>(bm) * a.nbw;
    const int nb = a.nbw;
    const int per = (nb + 1023) / 1024;
    const int b0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int t = 0; t < per; ++t)
        if (b0 + t < nb) local += bs[b0 + t];
    uint32_t total;
    uint32_t run = block_exclusive_scan<uint32_t, 1024>(local, &total, smem);
    for (int t = 0; t < per; ++t) {
        if (b0 + t < nb) {
            const uint32_t x = bs[b0 + t];
            bs[b0 + t] = run;
            run += x;
        }
    }
    if (threadIdx.x == 0) {
        const BitmapOut &o = a.out[bm];
        *o.d_uniq = total;
        if (static_cast<int64_t>(total) > o.uniq_cap) set_status(a.status, GNN_ERR_CAPACITY);
    }
}

// Word prefixes and the sorted unique ids.  With few tiles (pre_scanned = 0) each workgroup sums
// the popcounts of the tiles of its bitmap before it, and the bitmap's first tile writes its size.
__global__ __launch_bounds__(kBitmapThreads) void k_emit(RelabelArgs a, int32_t pre_scanned) {
    __shared__ uint32_t s_red[2][kBitmapThreads / 64];
    __shared__ uint32_t s_base;
    const int bm = static_cast<int>(blockIdx.x) / a.nbw;
    const int lt = static_cast<int>(blockIdx.x) - bm * a.nbw;
    const BitmapOut &o = a.out[bm];
    const uint32_t *bs = a.bsum + static_cast<int64_t>(bm) * a.nbw;
    if (pre_scanned) {
        if (threadIdx.x == 0) s_base = bs[lt];
    } else {
        uint32_t before = 0, all = 0;
        for (int b = threadIdx.x; b < a.nbw; b += blockDim.x) {
            const uint32_t x = bs[b];
            all += x;
            if (b < lt) before += x;
        }
        before = wave_sum(before);
        all = wave_sum(all);
        if (lane_id() == 0) {
            s_red[0][threadIdx.x >> 6] = before;
            s_red[1][threadIdx.x >> 6] = all;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t b0 = 0, tot = 0;
            for (int i = 0; i < kBitmapThreads / 64; ++i) {
                b0 += s_red[0][i];
                tot += s_red[1][i];
            }
            s_base = b0;
            if (lt == 0) {
                *o.d_uniq = tot;
                if (static_cast<int64_t>(tot) > o.uniq_cap) set_status(a.status, GNN_ERR_CAPACITY);
            }
        }
    }
    __syncthreads();
    const uint32_t *words = a.bitmap + static_cast<int64_t>(bm) * a.W;
    uint32_t *wpre = a.wprefix + static_cast<int64_t>(bm) * a.W;
    const int64_t tile0 = static_cast<int64_t>(lt) * kBitmapTile;
    const int64_t Wl = live_words(a);
    if (tile0 >= Wl) return;  // whole workgroup: nothing live
    // Round q: thread t takes word tile0 + q * kBitmapThreads + t, so the ids that neighbouring
    // lanes write sit a few entries apart and one store instruction touches few cache lines.
    // The rounds' wavefront scans run two at a time on 16-bit halves (a wavefront's popcount
    // total is at most 2048), and one barrier publishes every (round, wavefront) total.
    constexpr int Q = kBitmapWordsPerThread;
    constexpr int NW = kBitmapThreads / 64;
    static_assert(Q % 2 == 0, "rounds are scanned in pairs");
    __shared__ uint32_t s_tot[Q * NW];
    const int wv = static_cast<int>(threadIdx.x >> 6);
    uint32_t wd[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t w = tile0 + static_cast<int64_t>(q) * kBitmapThreads + threadIdx.x;
        wd[q] = w < Wl ? words[w] : 0u;
    }
    uint32_t inc[Q];
#pragma unroll
    for (int q = 0; q < Q; q += 2) {
        const uint32_t pair =
            wave_inclusive_scan<uint32_t>(__popc(wd[q]) | (static_cast<uint32_t>(__popc(wd[q + 1])) << 16));
        inc[q] = pair & 0xFFFFu;
        inc[q + 1] = pair >> 16;
    }
    if (lane_id() == 63) {
#pragma unroll
        for (int q = 0; q < Q; ++q) s_tot[q * NW + wv] = inc[q];
    }
    __syncthreads();
    uint32_t base = s_base;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const uint32_t v = s_tot[q * NW + i];
            if (i < wv) before += v;
            tot += v;
        }
        const int64_t w = tile0 + static_cast<int64_t>(q) * kBitmapThreads + threadIdx.x;
        uint32_t run = base + before + inc[q] - __popc(wd[q]);
        base += tot;
        if (w >= Wl) continue;
        wpre[w] = run;
        uint32_t bits = wd[q];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            if (static_cast<int64_t>(run) < o.uniq_cap) {
                const int32_t p = static_cast<int32_t>(w * 32 + b);
                o.uniq[run] = p;  // mapped through id_map by k_rank
                if (o.pos) o.pos[run] = p;
            }
            ++run;
        }
    }
}

// Ranks of every list that asks for them, in its bitmap's unique list; with an id map, also
// replaces each emitted position by its id (a separate pass keeps the dependent loads out of the
// emit loop, which writes one set bit after another).  The grid spreads over the actual items of
// the lists (and outputs), numbered in list order.
__global__ __launch_bounds__(256) void k_rank(RelabelArgs a) {
    __shared__ int64_t s_len[3 * kMaxGroup];
    __shared__ int64_t s_off[3 * kMaxGroup + 1];
    list_lengths(a, s_len, s_off);
    const int64_t bound = relabel_bound(a);
    // items: the lists' ids, then (with an id map) the outputs' positions
    const int nl = a.id_map ? a.nlist + a.nbm : a.nlist;
    const int64_t total = s_off[nl];
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int l = item_list(s_off, nl, t);
        const int64_t i = t - s_off[l];
        if (i >= s_len[l]) continue;
        if (l >= a.nlist) {
            const BitmapOut &o = a.out[l - a.nlist];
            const int32_t p = o.uniq[i];
            o.uniq[i] = p >= 0 && p < bound ? a.id_map[p] : -1;
            continue;
        }
        const IdList &L = a.list[l];
        if (L.lid == nullptr) continue;
        const int32_t v = L.ids[i];
        int32_t r = -1;
        if (v >= 0 && v < bound) {
            const int64_t w = static_cast<int64_t>(L.bitmap) * a.W + (v >> 5);
            r = static_cast<int32_t>(a.wprefix[w] + __popc(a.bitmap[w] & ((1u << (v & 31)) - 1u)));
        }
        L.lid[i] = r;
    }
}

// Tiles per bitmap at or below which k_emit computes its own offsets.
constexpr int kSelfScanMaxTiles = 512;

hipError_t launch_relabel(RelabelArgs a, hipStream_t s) {
    int64_t total = 0;
    bool any_rank = false, any_pass1 = false;
    for (int l = 0; l < a.nlist; ++l) {
        total += a.list[l].cap;
        any_rank |= a.list[l].lid != nullptr;
        any_pass1 |= a.list[l].pass == 1;
    }
    int64_t outs = 0;
    for (int b = 0; b < a.nbm; ++b) outs += a.out[b].uniq_cap;
    if (!a.bitmap_cleared) {
        hipError_t e = launch_fill_u32(a.bitmap, static_cast<int64_t>(a.nbm) * a.W, 0u, s);
        if (e != hipSuccess) return e;
    }
    if (total > 0) {
        const unsigned grid = grid_for(total, 256, 4096);
        if (any_pass1) hipLaunchKernelGGL(k_mark, dim3(grid), dim3(256), 0, s, a, 1);
        hipLaunchKernelGGL(k_mark, dim3(grid), dim3(256), 0, s, a, 0);
    }
    hipLaunchKernelGGL(k_popc_tiles, dim3(a.nbm * a.nbw), dim3(kBitmapThreads), 0, s, a);
    const int pre = a.nbw > kSelfScanMaxTiles ? 1 : 0;
    if (pre) hipLaunchKernelGGL(k_popc_scan, dim3(a.nbm), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(k_emit, dim3(a.nbm * a.nbw), dim3(kBitmapThreads), 0, s, a, pre);
    const int64_t rank_items = (any_rank ? total : 0) + (a.id_map ? outs : 0);
    if (rank_items > 0)
        hipLaunchKernelGGL(k_rank, dim3(grid_for(rank_items, 256, 4096)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
