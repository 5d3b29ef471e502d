// R-MAT draw kernel of the synthetic input generator (not part of the mini-batch library).
//
// Draw i: for level l = 0..L-1 a 16-bit uniform u is the (l % 2)-th half of
// word u32(gseed, i * W + l / 2), W = ceil(L / 2); u32 is MurmurHash3's 32-bit finalizer applied
// twice over the counter's halves (identical, bit for bit, to the torch version in synth/__init__.py).
// Quadrant a|b|c|d by thresholds ta < tb < tc on the 65536 scale; source bit = [u >= tb],
// destination bit = [ta <= u < tb or u >= tc], most significant first.  Draws with an endpoint >= N
// or a self-loop are rejected; kept draws are mapped through the id scramble new_id[] and appended
// (key = new_dst * N + new_src, draw index) when new_dst lies in [d_lo, d_hi).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

__device__ __forceinline__ uint32_t u32(uint64_t seed, uint64_t ctr) {
    const uint32_t s0 = static_cast<uint32_t>(seed), s1 = static_cast<uint32_t>(seed >> 32);
    const uint32_t a = static_cast<uint32_t>(ctr), b = static_cast<uint32_t>(ctr >> 32);
    uint32_t h = fmix32(a ^ s0);
    h = fmix32((h + b * 0x9E3779B1u) ^ s1);
    return h;
}

struct DrawArgs {
    uint64_t gseed;
    int64_t d0, d1;          // draw index range of this launch
    int32_t L, W;
    uint32_t ta, tb, tc;
    int64_t n;
    const int64_t *new_id;   // [n]
    int64_t dst_lo, dst_hi;  // partition of new destination ids
    int64_t *keys;           // out [cap]
    int64_t *idx;            // out [cap]
    unsigned long long *count;
    int64_t cap;
};

constexpr int kDrawsPerThread = 16;

__global__ __launch_bounds__(256) void k_rmat_draw(DrawArgs a) {
    __shared__ uint32_t s_n, s_base;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    int64_t key[kDrawsPerThread];
    int64_t id[kDrawsPerThread];
    uint32_t slot[kDrawsPerThread];
    int kept = 0;
    const int64_t first = a.d0 + (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * kDrawsPerThread;
    for (int q = 0; q < kDrawsPerThread; ++q) {
        const int64_t i = first + q;
        if (i >= a.d1) break;
        uint64_t src = 0, dst = 0;
        uint32_t word = 0;
        for (int l = 0; l < a.L; ++l) {
            if ((l & 1) == 0) word = u32(a.gseed, static_cast<uint64_t>(i) * a.W + (l >> 1));
            const uint32_t u = (word >> (16 * (l & 1))) & 0xFFFFu;
            const uint64_t sb = u >= a.tb;
            const uint64_t db = (u >= a.ta && u < a.tb) || u >= a.tc;
            src = src * 2 + sb;
            dst = dst * 2 + db;
        }
        if (src >= static_cast<uint64_t>(a.n) || dst >= static_cast<uint64_t>(a.n) || src == dst) continue;
        const int64_t nd = a.new_id[dst];
        if (nd < a.dst_lo || nd >= a.dst_hi) continue;
        key[kept] = nd * a.n + a.new_id[src];
        id[kept] = i;
        slot[kept] = atomicAdd(&s_n, 1u);
        ++kept;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_base = static_cast<uint32_t>(atomicAdd(a.count, static_cast<unsigned long long>(s_n)));
    __syncthreads();
    for (int q = 0; q < kept; ++q) {
        const int64_t p = static_cast<int64_t>(s_base) + slot[q];
        if (p < a.cap) {
            a.keys[p] = key[q];
            a.idx[p] = id[q];
        }
    }
}

}  // namespace

extern "C" int synth_rmat_draw(uint64_t gseed, int64_t d0, int64_t d1, int32_t L, uint32_t ta,
                               uint32_t tb, uint32_t tc, int64_t n, const int64_t *new_id,
                               int64_t dst_lo, int64_t dst_hi, int64_t *keys, int64_t *idx,
                               unsigned long long *count, int64_t cap, void *stream) {
    if (d1 <= d0) return 0;
    DrawArgs a{gseed, d0, d1, L, (L + 1) / 2, ta, tb, tc, n, new_id, dst_lo, dst_hi, keys, idx, count, cap};
    const int64_t threads = (d1 - d0 + kDrawsPerThread - 1) / kDrawsPerThread;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return -1;
    hipLaunchKernelGGL(k_rmat_draw, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
