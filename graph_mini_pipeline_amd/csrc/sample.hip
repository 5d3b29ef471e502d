// Frontier degree classification and degree-grouped k-hop neighbour sampling (gfx950, wave64).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. IV.C: a "full node" (degree <= fanout) keeps its whole neighbour list; other
// nodes draw `fanout` neighbours; lanes are grouped so that the threads of a group run identical
// logic, and high-degree nodes take a separate path.  Sec. IV.D, Alg. 1: classification by a flag
// and an exclusive scan turns placement into index arithmetic, with no atomics.
//
// Here the draw is the bottom-k of per-edge SplitMix64 keys: node v at hop l keeps the k positions
// with the smallest (key, position), key(j) = mix64(s_{l,v} + G*(j+1)).  Keys depend only on
// (seed, hop, node, position), so no adjacency is read to choose; only the k chosen neighbour ids
// are read.  Selection is exact: a threshold tau is chosen so that the expected number of keys
// <= tau is a little above k; the keys <= tau (candidates) are compacted to LDS; if fewer than k or
// more than the LDS capacity survive, tau is bisected and the pass repeated.  Once
// k <= count <= capacity the k smallest candidates are exactly the k smallest keys of the row.
//
// Classes (per hop, per frontier node v of degree deg, fanout k):
//   FULL   deg <= k                one lane per node copies the row
//   GROUP  k < deg <= group_max   16 lanes per node (4 nodes per wavefront)
//   WAVE   group_max < deg <= wave_max   one wavefront per node
//   BLOCK  deg > wave_max          one 512-thread workgroup per node
// Random classes fetch work dynamically from a per-class counter; results do not depend on the
// order in which nodes are processed.
#include <math.h>

#include "common.hpp"

namespace gnnmb {

// ---- classification: count, scan, scatter ------------------------------------------------------

__device__ __forceinline__ int32_t node_class(int64_t deg, int k, int group_max, int wave_max) {
    if (deg <= k) return kFull;
    if (deg <= group_max && k * 4 <= kGroupCap) return kGroup;
    if (deg <= wave_max && k * 4 <= kWaveCap) return kWave;
    return kBlock;
}

__global__ __launch_bounds__(kClassifyThreads) void k_classify_count(HopArgs a) {
    __shared__ uint32_t red[5][kClassifyThreads / 64];
    const int64_t F = load_count(a.d_F, a.F_cap);
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kClassifyTile +
                         static_cast<int64_t>(threadIdx.x) * kClassifyItems;
    uint32_t csum = 0, cc[4] = {0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        const int64_t i = base + q;
        if (i < F) {
            const int32_t v = a.front[i];
            int64_t deg = 0;
            if (v < 0 || v >= a.num_nodes) {
                set_status(a.status, GNN_ERR_OUT_OF_RANGE);
            } else {
                deg = row_ptr(a.indptr, a.ib, v + 1) - row_ptr(a.indptr, a.ib, v);
            }
            const int32_t c = deg <= a.k ? static_cast<int32_t>(deg) : a.k;
            const int32_t cls = node_class(deg, a.k, a.group_max, a.wave_max);
            a.packed[i] = (c << 2) | cls;
            csum += static_cast<uint32_t>(c);
            cc[cls] += 1;
        }
    }
    const int lane = lane_id(), w = threadIdx.x >> 6;
    uint32_t vals[5] = {csum, cc[0], cc[1], cc[2], cc[3]};
#pragma unroll
    for (int t = 0; t < 5; ++t) {
        const uint32_t s = wave_sum(vals[t]);
        if (lane == 0) red[t][w] = s;
    }
    __syncthreads();
    if (threadIdx.x < 5) {
        uint32_t s = 0;
        for (int i = 0; i < kClassifyThreads / 64; ++i) s += red[threadIdx.x][i];
        if (threadIdx.x == 0) a.bsum_c[blockIdx.x] = s;
        else a.bsum_cls[(threadIdx.x - 1) * a.nb + blockIdx.x] = s;
    }
}

// One workgroup scans the per-block sums (edge counts and the four class counts) in place.
__global__ __launch_bounds__(1024) void k_classify_scan(HopArgs a) {
    __shared__ uint32_t smem[16];
    const int nb = a.nb;
    const int per = (nb + 1023) / 1024;
    for (int col = 0; col < 5; ++col) {
        uint32_t *arr = col == 0 ? a.bsum_c : a.bsum_cls + static_cast<int64_t>(col - 1) * nb;
        const int b0 = threadIdx.x * per;
        uint32_t local = 0;
        for (int t = 0; t < per; ++t)
            if (b0 + t < nb) local += arr[b0 + t];
        uint32_t total;
        uint32_t run = block_exclusive_scan<uint32_t, 1024>(local, &total, smem);
        for (int t = 0; t < per; ++t) {
            if (b0 + t < nb) {
                const uint32_t x = arr[b0 + t];
                arr[b0 + t] = run;
                run += x;
            }
        }
        if (threadIdx.x == 0) {
            if (col == 0) {
                const int64_t F = load_count(a.d_F, a.F_cap);
                a.blk_indptr[F] = static_cast<int32_t>(total);
                *a.d_E = total;
                if (static_cast<int64_t>(total) > a.E_cap) set_status(a.status, GNN_ERR_CAPACITY);
            } else {
                a.class_count[col - 1] = total;
                a.work[col - 1] = 0;
            }
        }
    }
}

__global__ __launch_bounds__(kClassifyThreads) void k_classify_scatter(HopArgs a) {
    __shared__ uint32_t sm_c[kClassifyThreads / 64];
    __shared__ uint64_t sm_k[kClassifyThreads / 64];
    const int64_t F = load_count(a.d_F, a.F_cap);
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kClassifyTile +
                         static_cast<int64_t>(threadIdx.x) * kClassifyItems;
    int32_t pk[kClassifyItems];
    uint32_t csum = 0;
    uint64_t kc = 0;  // four 16-bit class counters
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        const int64_t i = base + q;
        pk[q] = i < F ? a.packed[i] : -1;
        if (pk[q] >= 0) {
            csum += static_cast<uint32_t>(pk[q] >> 2);
            kc += 1ull << (16 * (pk[q] & 3));
        }
    }
    uint32_t ctot;
    uint64_t ktot;
    uint32_t coff = block_exclusive_scan<uint32_t, kClassifyThreads>(csum, &ctot, sm_c);
    uint64_t koff = block_exclusive_scan<uint64_t, kClassifyThreads>(kc, &ktot, sm_k);
    coff += a.bsum_c[blockIdx.x];
#pragma unroll
    for (int q = 0; q < kClassifyItems; ++q) {
        if (pk[q] < 0) continue;
        const int64_t i = base + q;
        const int32_t cls = pk[q] & 3;
        a.blk_indptr[i] = static_cast<int32_t>(coff);
        coff += static_cast<uint32_t>(pk[q] >> 2);
        const uint32_t r = static_cast<uint32_t>((koff >> (16 * cls)) & 0xFFFF);
        koff += 1ull << (16 * cls);
        const uint32_t pos = a.bsum_cls[static_cast<int64_t>(cls) * a.nb + blockIdx.x] + r;
        a.lists[static_cast<int64_t>(cls) * a.F_cap + pos] = static_cast<int32_t>(i);
    }
}

// ---- FULL: one lane per node --------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_sample_full(HopArgs a) {
    const int64_t n = a.class_count[kFull];
    const int32_t *list = a.lists;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int32_t i = list[t];
        const int32_t v = a.front[i];
        if (v < 0 || v >= a.num_nodes) continue;
        const int64_t s = row_ptr(a.indptr, a.ib, v);
        const int64_t deg = row_ptr(a.indptr, a.ib, v + 1) - s;
        const int64_t o = a.blk_indptr[i];
        for (int64_t j = 0; j < deg; ++j)
            if (o + j < a.E_cap) a.blk_gid[o + j] = a.indices[s + j];
    }
}

// ---- threshold selection helpers ----------------------------------------------------------------

// Threshold whose expected number of keys <= tau among deg uniform keys is ~ k + 3 sqrt(k) + 6.
__device__ __forceinline__ uint64_t initial_tau(int64_t deg, int k) {
    const double mu = static_cast<double>(k) + 3.0 * sqrt(static_cast<double>(k)) + 6.0;
    const double p = mu / static_cast<double>(deg);
    if (p >= 1.0) return ~0ull;
    const double t = p * 18446744073709551616.0;
    if (t >= 18446744073709549568.0) return ~0ull;
    return static_cast<uint64_t>(t);
}

// Next threshold after a pass that collected `cnt` keys <= tau.  Returns false when done (k <=
// cnt <= cap) and sets *fail when no threshold can separate the keys (identical keys only).
__device__ __forceinline__ bool next_tau(int cnt, int k, int cap, uint64_t &tau, uint64_t &lo,
                                         uint64_t &hi, bool &has_lo, bool &has_hi, bool &fail) {
    if (cnt < k) {
        has_lo = true;
        lo = tau;
        if (has_hi) tau = lo + (hi - lo) / 2;
        else tau = tau >= (~0ull >> 2) ? ~0ull : ((tau << 2) | 3ull);
    } else if (cnt > cap) {
        has_hi = true;
        hi = tau;
        const uint64_t l = has_lo ? lo : 0ull;
        tau = l + (hi - l) / 2;
    } else {
        return false;
    }
    if (has_lo && has_hi && hi - lo <= 1) {
        fail = true;
        return false;
    }
    return true;
}

// ---- GROUP and WAVE: G lanes per node -----------------------------------------------------------

template <int G, int CAP>
__global__ __launch_bounds__(256) void k_sample_lanes(HopArgs a, int32_t cls) {
    constexpr int NG = 64 / G;       // nodes per wavefront
    constexpr int SLOTS = 4 * NG;    // nodes per workgroup
    __shared__ uint64_t s_key[SLOTS][CAP];
    __shared__ int32_t s_pos[SLOTS][CAP];
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const int slot = static_cast<int>(threadIdx.x >> 6) * NG + grp;
    const uint64_t gmask = G == 64 ? ~0ull : (((1ull << G) - 1ull) << (grp * G));
    const uint64_t below = (1ull << lane) - 1ull;  // lanes below this one
    const int64_t n = a.class_count[cls];
    const int32_t *list = a.lists + static_cast<int64_t>(cls) * a.F_cap;
    const int k = a.k;
    for (;;) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&a.work[cls], static_cast<uint32_t>(NG));
        base = __shfl(base, 0, 64);
        if (static_cast<int64_t>(base) >= n) break;
        const int64_t item = static_cast<int64_t>(base) + grp;
        if (item < n) {
            const int32_t i = list[item];
            const int32_t v = a.front[i];
            const int64_t start = row_ptr(a.indptr, a.ib, v);
            const int64_t deg = row_ptr(a.indptr, a.ib, v + 1) - start;
            const int64_t out0 = a.blk_indptr[i];
            const uint64_t ns = mix64(a.hop_seed ^ static_cast<uint64_t>(static_cast<uint32_t>(v)));
            uint64_t tau = initial_tau(deg, k), lo = 0, hi = 0;
            bool has_lo = false, has_hi = false, fail = false;
            int cnt = 0;
            for (int it = 0; it < 128; ++it) {
                cnt = 0;
                uint64_t z = ns + kGamma * static_cast<uint64_t>(gl + 1);
                const uint64_t step = kGamma * static_cast<uint64_t>(G);
                for (int64_t j0 = 0; j0 < deg; j0 += G) {
                    const int64_t j = j0 + gl;
                    const uint64_t key = mix64(z);
                    z += step;
                    const bool p = j < deg && key <= tau;
                    const uint64_t m = __ballot(p) & gmask;
                    if (p) {
                        const int pos = cnt + __popcll(m & below);
                        if (pos < CAP) {
                            s_key[slot][pos] = key;
                            s_pos[slot][pos] = static_cast<int32_t>(j);
                        }
                    }
                    cnt += __popcll(m);
                }
                if (!next_tau(cnt, k, CAP, tau, lo, hi, has_lo, has_hi, fail)) break;
            }
            if (fail || cnt < k || cnt > CAP) {
                if (gl == 0) set_status(a.status, GNN_ERR_INTERNAL);
                cnt = 0;
            }
            wave_lds_sync();
            // Candidates sit in ascending position; keep those of rank < k among (key, pos).
            int outc = 0;
            for (int c0 = 0; c0 < cnt; c0 += G) {
                const int c = c0 + gl;
                bool sel = false;
                int32_t jc = 0;
                if (c < cnt) {
                    const uint64_t kc = s_key[slot][c];
                    jc = s_pos[slot][c];
                    int r = 0;
                    for (int t = 0; t < cnt; ++t) {
                        const uint64_t kt = s_key[slot][t];
                        const int32_t jt = s_pos[slot][t];
                        r += (kt < kc) | ((kt == kc) & (jt < jc));
                    }
                    sel = r < k;
                }
                const uint64_t m = __ballot(sel) & gmask;
                if (sel) {
                    const int64_t o = out0 + outc + __popcll(m & below);
                    if (o < a.E_cap) a.blk_gid[o] = a.indices[start + jc];
                }
                outc += __popcll(m);
            }
            wave_lds_sync();
        }
    }
}

// ---- BLOCK: one workgroup per node --------------------------------------------------------------

__global__ __launch_bounds__(kBlockThreads) void k_sample_block(HopArgs a) {
    constexpr int NT = kBlockThreads;
    constexpr int CAP = kBlockCap;
    __shared__ uint64_t s_key[CAP];
    __shared__ int32_t s_pos[CAP];
    __shared__ uint8_t s_sel[CAP];
    __shared__ uint32_t s_cnt;
    __shared__ uint32_t s_item;
    const int lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;
    const int64_t n = a.class_count[kBlock];
    const int32_t *list = a.lists + static_cast<int64_t>(kBlock) * a.F_cap;
    const int k = a.k;
    for (;;) {
        if (threadIdx.x == 0) s_item = atomicAdd(&a.work[kBlock], 1u);
        __syncthreads();
        const int64_t item = s_item;
        if (item >= n) break;
        const int32_t i = list[item];
        const int32_t v = a.front[i];
        const int64_t start = row_ptr(a.indptr, a.ib, v);
        const int64_t deg = row_ptr(a.indptr, a.ib, v + 1) - start;
        const int64_t out0 = a.blk_indptr[i];
        const uint64_t ns = mix64(a.hop_seed ^ static_cast<uint64_t>(static_cast<uint32_t>(v)));
        uint64_t tau = initial_tau(deg, k), lo = 0, hi = 0;
        bool has_lo = false, has_hi = false, fail = false;
        int cnt = 0;
        for (int it = 0; it < 128; ++it) {
            if (threadIdx.x == 0) s_cnt = 0;
            __syncthreads();
            uint64_t z = ns + kGamma * static_cast<uint64_t>(threadIdx.x + 1);
            const uint64_t step = kGamma * static_cast<uint64_t>(NT);
            for (int64_t j0 = 0; j0 < deg; j0 += NT) {
                const int64_t j = j0 + threadIdx.x;
                const uint64_t key = mix64(z);
                z += step;
                const bool p = j < deg && key <= tau;
                const uint64_t m = __ballot(p);
                if (m) {
                    uint32_t wbase = 0;
                    if (lane == 0) wbase = atomicAdd(&s_cnt, static_cast<uint32_t>(__popcll(m)));
                    wbase = __shfl(wbase, 0, 64);
                    if (p) {
                        const uint32_t pos = wbase + __popcll(m & below);
                        if (pos < CAP) {
                            s_key[pos] = key;
                            s_pos[pos] = static_cast<int32_t>(j);
                        }
                    }
                }
            }
            __syncthreads();
            cnt = static_cast<int>(s_cnt);
            __syncthreads();
            if (!next_tau(cnt, k, CAP, tau, lo, hi, has_lo, has_hi, fail)) break;
        }
        if (fail || cnt < k || cnt > CAP) {
            if (threadIdx.x == 0) set_status(a.status, GNN_ERR_INTERNAL);
            cnt = 0;
        }
        for (int c = threadIdx.x; c < cnt; c += NT) {
            const uint64_t kc = s_key[c];
            const int32_t jc = s_pos[c];
            int r = 0;
            for (int t = 0; t < cnt; ++t) {
                const uint64_t kt = s_key[t];
                r += (kt < kc) | ((kt == kc) & (s_pos[t] < jc));
            }
            s_sel[c] = r < k ? 1 : 0;
        }
        __syncthreads();
        for (int c = threadIdx.x; c < cnt; c += NT) {
            if (!s_sel[c]) continue;
            const int32_t jc = s_pos[c];
            int r = 0;
            for (int t = 0; t < cnt; ++t) r += s_sel[t] & (s_pos[t] < jc);
            const int64_t o = out0 + r;
            if (o < a.E_cap) a.blk_gid[o] = a.indices[start + jc];
        }
        __syncthreads();
    }
}

// ---- launchers ---------------------------------------------------------------------------------

hipError_t launch_classify(const HopArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_classify_count, dim3(a.nb), dim3(kClassifyThreads), 0, s, a);
    hipLaunchKernelGGL(k_classify_scan, dim3(1), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(k_classify_scatter, dim3(a.nb), dim3(kClassifyThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sample(const HopArgs &a, hipStream_t s) {
    const int64_t F = a.F_cap;
    hipLaunchKernelGGL(k_sample_full, dim3(grid_for(F, 256, 1024)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_sample_lanes<kGroupLanes, kGroupCap>),
                       dim3(grid_for(F, 4 * (64 / kGroupLanes), 2048)), dim3(256), 0, s, a,
                       static_cast<int32_t>(kGroup));
    hipLaunchKernelGGL((k_sample_lanes<64, kWaveCap>), dim3(grid_for(F, 4, 2048)), dim3(256), 0,
                       s, a, static_cast<int32_t>(kWave));
    hipLaunchKernelGGL(k_sample_block, dim3(grid_for(F, 1, 512)), dim3(kBlockThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gnnmb
