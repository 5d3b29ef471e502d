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

// Words up to the first 16-byte boundary one at a time, then 16-byte stores, then the tail.
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t *p, int64_t n, uint32_t value) {
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t head = static_cast<int64_t>((16u - (reinterpret_cast<uintptr_t>(p) & 15u)) & 15u) / 4;
    head = head < n ? head : n;
    if (t0 < head) p[t0] = value;
    const int64_t nq = (n - head) / 4;
    uint4 *q = reinterpret_cast<uint4 *>(p + head);
    const uint4 v = make_uint4(value, value, value, value);
    for (int64_t i = t0; i < nq; i += stride) q[i] = v;
    const int64_t done = head + 4 * nq;
    if (t0 < n - done) p[done + t0] = value;
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

// Word prefixes and the sorted unique ids of a bitmap of many tiles, after k_popc_tiles (and
// k_popc_scan): each workgroup sums the popcounts of the tiles of its bitmap before it (or reads
// their scanned prefix), and the bitmap's first tile writes its size.
__global__ __launch_bounds__(kBitmapThreads) void k_emit_tiles(RelabelArgs a, int32_t pre_scanned) {
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
    uint2 *rdir = a.rdir + static_cast<int64_t>(bm) * a.W;
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
        rdir[w] = make_uint2(run, wd[q]);
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

// The words of round q of one tile for thread t: word tile0 + q * kBitmapThreads + t (packed from
// the byte maps first, when given, and stored to the bitmap).
template <int Q>
__device__ __forceinline__ void tile_words(const RelabelArgs &a, int bm, int64_t tile0, int64_t Wl,
                                           uint32_t (&wd)[Q]) {
    uint32_t *words = a.bitmap + static_cast<int64_t>(bm) * a.W;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t w = tile0 + static_cast<int64_t>(q) * kBitmapThreads + threadIdx.x;
        uint32_t word = 0;
        if (w < Wl) {
            if (a.bytes) {
                // word w = the 32 bytes of ids 32w .. 32w+31 (each 0 or 1), packed
                const uint4 *p = reinterpret_cast<const uint4 *>(
                    a.bytes + static_cast<int64_t>(bm) * a.W * 32 + w * 32);
                const uint4 lo = p[0], hi = p[1];
                const uint32_t x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int k = 0; k < 8; ++k)   // 4 bytes (0/1) -> 4 bits: products land on distinct bits
                    word |= ((((x[k] & 0x01010101u) * 0x00204081u) >> 21) & 0xFu) << (4 * k);
                words[w] = word;
            } else {
                word = words[w];
            }
        }
        wd[q] = word;
    }
}

// Word prefixes and the sorted unique ids of bitmaps of few tiles, in one pass: tile t (by ticket)
// of bitmap t / nbw packs its words (from the byte maps when given), counts its set bits, takes
// the count of set bits before it by look-back over the earlier tiles of the same bitmap, then
// writes every word's prefix and the ids of its set bits in order; the last tile holding live
// words writes the number of ids.  Tiles past the live words have nothing to do and nobody waits
// for them.  The grid also zeroes the optional clear region (a bitmap no longer needed by this
// stream).  One launch instead of three (k_popc_tiles, k_popc_scan, k_emit_tiles); a look-back
// round covers 256 tiles, and each round costs a round trip to the chip-coherent memory, so long
// bitmaps keep the three launches.
__global__ __launch_bounds__(kBitmapThreads) void k_emit(RelabelArgs a) {
    constexpr int Q = kBitmapWordsPerThread;
    constexpr int NW = kBitmapThreads / 64;
    static_assert(Q % 2 == 0, "rounds are scanned in pairs");
    __shared__ uint32_t s_tot[Q * NW];
    __shared__ uint32_t s_ticket, s_base;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < a.clear_n;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x)
        a.clear_ptr[t] = 0u;
    // Workgroup b serves bitmap b / nbw; those beyond the bitmap's live tiles leave before taking
    // a ticket.  The live ones take tickets 0 .. last from their bitmap's own counter (tickets of
    // one counter are handed out one at a time), and ticket t is tile t.
    const int bm = static_cast<int>(blockIdx.x / static_cast<unsigned>(a.nbw));
    const int64_t Wl = live_words(a);
    const int64_t last = Wl > 0 ? (Wl - 1) / kBitmapTile : 0;   // last tile with live words
    if (static_cast<int64_t>(blockIdx.x) - static_cast<int64_t>(bm) * a.nbw > last) return;
    const int64_t lt = lb_ticket(a.lb.ticket + bm, &s_ticket);
    const int64_t tile0 = lt * kBitmapTile;
    const BitmapOut &o = a.out[bm];
    const int wv = static_cast<int>(threadIdx.x >> 6);
    uint32_t wd[Q];
    tile_words<Q>(a, bm, tile0, Wl, wd);
    // Round q: thread t takes word tile0 + q * 256 + t, so the ids that neighbouring lanes write
    // sit a few entries apart and one store instruction touches few cache lines.  The rounds'
    // wavefront scans run two at a time on 16-bit halves (a wavefront's popcount total is at most
    // 2048), and one barrier publishes every (round, wavefront) total.
    uint32_t inc[Q];
#pragma unroll
    for (int q = 0; q < Q; q += 2) {
        const uint32_t pair = wave_inclusive_scan<uint32_t>(
            __popc(wd[q]) | (static_cast<uint32_t>(__popc(wd[q + 1])) << 16));
        inc[q] = pair & 0xFFFFu;
        inc[q + 1] = pair >> 16;
    }
    if (lane_id() == 63) {
#pragma unroll
        for (int q = 0; q < Q; ++q) s_tot[q * NW + wv] = inc[q];
    }
    __syncthreads();
    if (wv == 0) {
        uint32_t agg = 0;
        for (int i = lane_id(); i < Q * NW; i += 64) agg += s_tot[i];
        agg = wave_sum(agg);
        uint64_t *chain = a.lb.words + static_cast<int64_t>(bm) * a.nbw;
        uint32_t before = 0;
        if (lt == 0) {
            if (lane_id() == 0) lb_publish(&chain[0], kLbInclusive, agg);
        } else {
            if (lane_id() == 0) lb_publish(&chain[lt], kLbAggregate, agg);
            before = lb_exclusive(chain, lt);
            if (lane_id() == 0) lb_publish(&chain[lt], kLbInclusive, before + agg);
        }
        if (lane_id() == 0) {
            s_base = before;
            if (lt == last) {
                const uint32_t tot = before + agg;
                *o.d_uniq = tot;
                if (static_cast<int64_t>(tot) > o.uniq_cap) set_status(a.status, GNN_ERR_CAPACITY);
            }
        }
    }
    __syncthreads();
    uint32_t base = s_base;
    uint2 *rdir = a.rdir + static_cast<int64_t>(bm) * a.W;
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
        rdir[w] = make_uint2(run, wd[q]);
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
            const uint2 e = a.rdir[static_cast<int64_t>(L.bitmap) * a.W + (v >> 5)];
            r = static_cast<int32_t>(e.x + __popc(e.y & ((1u << (v & 31)) - 1u)));
        }
        L.lid[i] = r;
    }
}

// ---- short lists: an LDS-staged radix sort in one workgroup --------------------------------------
//
// For lists far shorter than the id range, passes over id_bound / 32 bitmap words cost more than
// sorting the ids themselves.  One workgroup of kSortThreads loads every list's ids as keys
// id << 1 | (1 for an id of a pass-1 list), so that a pass-1 id given twice becomes two equal keys,
// and sorts them with a least-significant-digit radix sort of kSortBits-bit digits between two LDS
// buffers.  The sort is stable: each thread holds a run of consecutive keys, counts its digits,
// and the counts are scanned over the threads in digit-major order.  The first key of every id is
// kept with wavefront ballots (the unique ids, in order, compacted by the ballot's popcounts and a
// prefix over the wavefronts' counts), and every list item is ranked by binary search in the
// unique ids, which stay in LDS.
constexpr int kSortThreads = 1024;
constexpr int kSortBits = 4;
constexpr uint32_t kSortNone = 0xFFFFFFFFu;   // an out-of-range id: sorts last, never kept

// v[q] for a per-lane q, with masks rather than an indexed (memory) access.
__device__ __forceinline__ uint64_t pick4(const uint64_t (&v)[4], int q) {
    const uint64_t m0 = 0ull - static_cast<uint64_t>(q == 0), m1 = 0ull - static_cast<uint64_t>(q == 1);
    const uint64_t m2 = 0ull - static_cast<uint64_t>(q == 2), m3 = 0ull - static_cast<uint64_t>(q == 3);
    return (v[0] & m0) | (v[1] & m1) | (v[2] & m2) | (v[3] & m3);
}

// Exclusive scan over the workgroup of four 64-bit words (16 digit counts of 16 bits each).
__device__ __forceinline__ void block_scan4(const uint64_t (&v)[4], uint64_t (&before)[4],
                                            uint64_t (&total)[4], uint64_t (*smem)[4]) {
    constexpr int NW = kSortThreads / 64;
    const int lane = lane_id();
    const int w = static_cast<int>(threadIdx.x >> 6);
    uint64_t inc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) inc[q] = wave_inclusive_scan<uint64_t>(v[q]);
    if (lane == 63) {
#pragma unroll
        for (int q = 0; q < 4; ++q) smem[w][q] = inc[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint64_t b = 0, t = 0;
        for (int i = 0; i < NW; ++i) {
            const uint64_t x = smem[i][q];
            if (i < w) b += x;
            t += x;
        }
        before[q] = b + inc[q] - v[q];
        total[q] = t;
    }
    __syncthreads();
}

template <int CAP>
__global__ __launch_bounds__(kSortThreads) void k_relabel_sort(RelabelArgs a, int32_t key_bits) {
    constexpr int NW = kSortThreads / 64;
    constexpr int MAXCH = CAP / 64;           // 64-key chunks of a full buffer
    __shared__ uint32_t s_keys[2][CAP];
    __shared__ uint64_t s_scan[NW][4];
    __shared__ uint32_t s_cnt[MAXCH];
    __shared__ int64_t s_len[2 * kMaxGroup];
    __shared__ int64_t s_off[2 * kMaxGroup + 1];
    __shared__ uint32_t s_nu;
    if (threadIdx.x < static_cast<unsigned>(a.nlist))
        s_len[threadIdx.x] = load_count(a.list[threadIdx.x].d_n, a.list[threadIdx.x].cap);
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t run = 0;
        for (int l = 0; l < a.nlist; ++l) {
            s_off[l] = run;
            run += s_len[l];
        }
        s_off[a.nlist] = run;
    }
    __syncthreads();
    const int64_t n = s_off[a.nlist] < CAP ? s_off[a.nlist] : CAP;   // the host checked the caps
    // keys per thread for this list length, and the slots sorted (n rounded up; the rest hold
    // keys that sort last)
    const int per = static_cast<int>((n + kSortThreads - 1) / kSortThreads) > 0
                        ? static_cast<int>((n + kSortThreads - 1) / kSortThreads) : 1;
    const int m = per * kSortThreads;
    const int64_t bound = a.id_bound;
    for (int64_t t = threadIdx.x; t < m; t += kSortThreads) {
        uint32_t key = kSortNone;
        if (t < n) {
            int l = 0;
            while (l + 1 < a.nlist && s_off[l + 1] <= t) ++l;
            const int32_t v = a.list[l].ids[t - s_off[l]];
            if (v < 0 || v >= bound) set_status(a.status, GNN_ERR_OUT_OF_RANGE);
            else key = (static_cast<uint32_t>(v) << 1) | (a.list[l].pass == 1 ? 1u : 0u);
        }
        s_keys[0][t] = key;
    }
    __syncthreads();
    // Radix passes: thread t holds keys [t per, (t + 1) per) of the current buffer.
    int cur = 0;
    static_assert(kSortBits == 4, "16 digit counts of 16 bits in four 64-bit words");
    for (int bit = 0; bit < key_bits; bit += kSortBits) {
        const uint32_t *src = s_keys[cur] + threadIdx.x * per;
        uint64_t c[4] = {0, 0, 0, 0};   // this thread's digit counts
        for (int i = 0; i < per; ++i) {
            const int d = static_cast<int>((src[i] >> bit) & 15u);
            const uint64_t one = 1ull << (16 * (d & 3));
            const int q = d >> 2;
            c[0] += q == 0 ? one : 0;
            c[1] += q == 1 ? one : 0;
            c[2] += q == 2 ? one : 0;
            c[3] += q == 3 ? one : 0;
        }
        uint64_t before[4], tot[4];
        block_scan4(c, before, tot, s_scan);
        // start of each digit's run for this thread: the keys of smaller digits (all threads) plus
        // the keys of this digit on earlier threads, kept in the same packed fields
        uint64_t start[4] = {0, 0, 0, 0};
        uint32_t run = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            start[b >> 2] |= static_cast<uint64_t>(run) << (16 * (b & 3));
            run += static_cast<uint32_t>((tot[b >> 2] >> (16 * (b & 3))) & 0xFFFF);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) start[q] += before[q];   // no field exceeds CAP < 2^16
        for (int i = 0; i < per; ++i) {   // in order: equal digits keep their order (stable)
            const uint32_t key = src[i];
            const int d = static_cast<int>((key >> bit) & 15u);
            const int q = d >> 2, f = 16 * (d & 3);
            const uint32_t pos = static_cast<uint32_t>((pick4(start, q) >> f) & 0xFFFF);
            const uint64_t one = 1ull << f;
            start[0] += q == 0 ? one : 0;
            start[1] += q == 1 ? one : 0;
            start[2] += q == 2 ? one : 0;
            start[3] += q == 3 ? one : 0;
            s_keys[cur ^ 1][pos] = key;
        }
        __syncthreads();
        cur ^= 1;
    }
    // The first key of every id: wavefront ballots over 64 consecutive sorted keys at a time.
    const uint32_t *sk = s_keys[cur];
    uint32_t *su = s_keys[cur ^ 1];   // the unique ids, ascending
    const int w = static_cast<int>(threadIdx.x >> 6);
    const int lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
    auto first_of = [&](int64_t idx, bool report) {
        const uint32_t key = sk[idx];
        const uint32_t prev = idx > 0 ? sk[idx - 1] : kSortNone;
        const bool valid = idx < n && key != kSortNone;
        if (report && valid && idx > 0 && key == prev && (key & 1u))
            set_status(a.status, GNN_ERR_INVALID_ARG);   // an id given twice in a pass-1 list
        return valid && (idx == 0 || (key >> 1) != (prev >> 1));
    };
    const int nch = per * NW;   // chunk j * NW + w holds sorted keys [64 (j NW + w), + 64)
    for (int j = 0; j < per; ++j) {
        const uint64_t mk = __ballot(first_of(static_cast<int64_t>(j) * kSortThreads + threadIdx.x, true));
        if (lane == 0) s_cnt[j * NW + w] = static_cast<uint32_t>(__popcll(mk));
    }
    __syncthreads();
    if (w == 0) {   // exclusive prefix of the chunk counts: lane L takes chunks [L cpl, (L+1) cpl)
        const int cpl = (nch + 63) / 64;
        uint32_t sum = 0;
        for (int q = 0; q < cpl; ++q) {
            const int ch = lane * cpl + q;
            if (ch < nch) sum += s_cnt[ch];
        }
        const uint32_t inc = wave_inclusive_scan<uint32_t>(sum);
        uint32_t r = inc - sum;
        for (int q = 0; q < cpl; ++q) {
            const int ch = lane * cpl + q;
            if (ch < nch) {
                const uint32_t v = s_cnt[ch];
                s_cnt[ch] = r;
                r += v;
            }
        }
        if (lane == 63) s_nu = inc;
    }
    __syncthreads();
    const uint32_t nu = s_nu;
    const BitmapOut &o = a.out[0];
    for (int j = 0; j < per; ++j) {
        const int64_t idx = static_cast<int64_t>(j) * kSortThreads + threadIdx.x;
        const bool f = first_of(idx, false);
        const uint64_t mk = __ballot(f);
        if (f) {
            const uint32_t u = s_cnt[j * NW + w] + static_cast<uint32_t>(__popcll(mk & below));
            const int32_t id = static_cast<int32_t>(sk[idx] >> 1);
            su[u] = static_cast<uint32_t>(id);
            if (static_cast<int64_t>(u) < o.uniq_cap) o.uniq[u] = id;
            if (a.sort_sets_bits) atomicOr(&a.bitmap[id >> 5], 1u << (id & 31));
        }
    }
    if (threadIdx.x == 0) {
        *o.d_uniq = nu;
        if (static_cast<int64_t>(nu) > o.uniq_cap) set_status(a.status, GNN_ERR_CAPACITY);
    }
    __syncthreads();
    // Ranks: binary search of every list item in the unique ids.
    for (int64_t t = threadIdx.x; t < n; t += kSortThreads) {
        int l = 0;
        while (l + 1 < a.nlist && s_off[l + 1] <= t) ++l;
        const IdList &L = a.list[l];
        if (L.lid == nullptr) continue;
        const int32_t v = L.ids[t - s_off[l]];
        int32_t r = -1;
        if (v >= 0 && v < bound) {
            uint32_t lo = 0, hi = nu;
            while (lo < hi) {
                const uint32_t mid = (lo + hi) >> 1;
                if (su[mid] < static_cast<uint32_t>(v)) lo = mid + 1;
                else hi = mid;
            }
            r = static_cast<int32_t>(lo);
        }
        L.lid[t - s_off[l]] = r;
    }
}

constexpr int kSortCapLarge = 16384;   // 128 KB of keys: needs the large LDS of gfx950 workgroups
constexpr int kSortCapSmall = 8192;    // 64 KB

// Keys one sort workgroup can hold on the current device (the larger variant when its LDS fits).
int64_t sort_capacity() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kSortCapSmall;
    if (cached[dev] == 0) {
        int lds = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            lds = 0;
        cached[dev] = lds >= 2 * kSortCapLarge * 4 + 8192 ? kSortCapLarge : kSortCapSmall;
    }
    return cached[dev];
}

// The sort path pays when its cost, ~42 us + ~7.7 ns per key (one workgroup), is below the
// bitmap path's, ~25 us + ~4.6 us per million bitmap words (passes spread over the chip):
// measured on MI355X with gnn_unique_relabel over lists of 256 .. 16384 ids and id ranges of 2^20
// .. 2^30, both paths forced.  Sort when the bitmap has at least kSortBaseWords plus
// kSortWordsPerKey words per listed id (short lists over id ranges of ~130M ids and more).
constexpr int64_t kSortBaseWords = 3700000;
constexpr int64_t kSortWordsPerKey = 1700;

bool relabel_sorts(const RelabelArgs &a) {
    if (a.force == 2 || a.bitmap_read_after) return false;
    if (a.nbm != 1 || a.bytes || a.id_map || a.d_bound || a.out[0].pos) return false;
    if (a.id_bound > (1LL << 30)) return false;   // keys id << 1 | flag below 2^31
    if (a.nlist < 1 || a.nlist > 2 * kMaxGroup) return false;
    int64_t n = 0;
    for (int l = 0; l < a.nlist; ++l) {
        if (a.list[l].pass == 2) return false;
        n += a.list[l].cap;
    }
    if (n > sort_capacity()) return false;
    if (a.force == 1) return true;
    return a.W >= kSortBaseWords + kSortWordsPerKey * n;
}

// Tiles per bitmap at or below which k_emit_tiles computes its own offsets.
constexpr int kSelfScanMaxTiles = 512;

// Bitmaps of at most this many tiles take the single-pass k_emit (at most four look-back rounds);
// longer ones the three launches, whose passes are each spread over every tile at once.
constexpr int kSinglePassMaxTiles = 1024;
bool emit_single_pass(const RelabelArgs &a) { return a.nbw <= kSinglePassMaxTiles; }

// Look-back words of one relabel launch (single pass only): one per tile of every bitmap (the
// launch also takes one ticket counter per bitmap).
int64_t relabel_lb_words(const RelabelArgs &a) {
    return emit_single_pass(a) ? static_cast<int64_t>(a.nbm) * a.nbw : 0;
}

hipError_t launch_relabel(RelabelArgs a, hipStream_t s) {
    if (relabel_sorts(a)) {
        int key_bits = 1;   // the pass flag, then the id's bits
        while ((1LL << (key_bits - 1)) < a.id_bound) ++key_bits;
        if (sort_capacity() == kSortCapLarge)
            hipLaunchKernelGGL(k_relabel_sort<kSortCapLarge>, dim3(1), dim3(kSortThreads), 0, s, a, key_bits);
        else
            hipLaunchKernelGGL(k_relabel_sort<kSortCapSmall>, dim3(1), dim3(kSortThreads), 0, s, a, key_bits);
        return hipGetLastError();
    }
    int64_t total = 0;
    bool any_rank = false, any_pass[3] = {false, false, false};
    for (int l = 0; l < a.nlist; ++l) {
        total += a.list[l].cap;
        any_rank |= a.list[l].lid != nullptr;
        if (a.list[l].pass >= 0 && a.list[l].pass < 3) any_pass[a.list[l].pass] = true;
    }
    int64_t outs = 0;
    for (int b = 0; b < a.nbm; ++b) outs += a.out[b].uniq_cap;
    if (!a.bitmap_cleared) {
        hipError_t e = launch_fill_u32(a.bitmap, static_cast<int64_t>(a.nbm) * a.W, 0u, s);
        if (e != hipSuccess) return e;
    }
    if (total > 0) {
        const unsigned grid = grid_for(total, 256, 4096);
        if (any_pass[1]) hipLaunchKernelGGL(k_mark, dim3(grid), dim3(256), 0, s, a, 1);
        if (any_pass[0]) hipLaunchKernelGGL(k_mark, dim3(grid), dim3(256), 0, s, a, 0);
    }
    if (emit_single_pass(a)) {
        hipLaunchKernelGGL(k_emit, dim3(a.nbm * a.nbw), dim3(kBitmapThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(k_popc_tiles, dim3(a.nbm * a.nbw), dim3(kBitmapThreads), 0, s, a);
        const int pre = a.nbw > kSelfScanMaxTiles ? 1 : 0;
        if (pre) hipLaunchKernelGGL(k_popc_scan, dim3(a.nbm), dim3(1024), 0, s, a);
        hipLaunchKernelGGL(k_emit_tiles, dim3(a.nbm * a.nbw), dim3(kBitmapThreads), 0, s, a, pre);
    }
    const int64_t rank_items = (any_rank ? total : 0) + (a.id_map ? outs : 0);
    if (rank_items > 0)
        hipLaunchKernelGGL(k_rank, dim3(grid_for(rank_items, 256, 4096)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
