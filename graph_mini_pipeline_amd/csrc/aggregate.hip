// Mean aggregation of one sampled block (gfx950).
//
// GARDEN: Efficient GPU-Accelerated Billion-Scale GNN Training via Caching-Sampling-Batching
// Co-Design, Sec. II.A eq. (1): a destination aggregates the states of its (sampled) in-neighbours
// with a permutation-invariant AGGREGATE, here the mean:
//   out[i] = (1/c_i) * sum_{e in [indptr[i], indptr[i+1])} src[lid[e]],  0 when c_i = 0.
// FastGL: A GPU-Efficient Framework for Accelerating Sampling-Based GNN Training at Large Scale
// (Memory-Aware computation) keeps each destination's running sum on chip; here it lives in
// registers: every lane owns one 16-byte chunk of one destination row and walks that
// destination's edges, so the partial sum never leaves the register file and each source chunk
// is read once per edge.  The (destination, chunk) pairs are flattened over all lanes, so
// consecutive lanes read consecutive chunks of the same source row.  fp32 accumulation in
// ascending edge order, one division by c_i.  Arithmetic intensity ~0.25 flop/byte: HBM-bound,
// no matrix cores.
#include "common.hpp"

namespace gnnmb {

// One block to aggregate (a segment of a batched launch).
struct MeanSeg {
    const int32_t *indptr;
    const int32_t *lid;
    int64_t e_cap;   // entries of lid: edge offsets are clamped to it
    const int64_t *d_n;
    int64_t n_cap;
    const float *src;
    int64_t n_src;   // rows of src: a local id outside [0, n_src) is an error
    float *out;
    uint32_t item0;  // first work item of this segment in the launch
};

struct MeanArgs {
    MeanSeg seg[kMaxMeanSegs];
    int32_t nseg;
    uint32_t items;  // total work items (segments' caps times slabs)
    int64_t ld_src;
    int64_t ld_out;
    int32_t *status;
    int32_t d;
    FastDiv cpr;
    // scatter (one segment): destination r's row goes to row scat[r * scat_g + g] - 1 of
    // scat_out[g] for every g whose bit is set in scat_mask[r], instead of to the segment's out
    const int32_t *scat;
    const uint32_t *scat_mask;
    int32_t scat_g;
    float *scat_out[kMaxGroup];
};

// A local id outside the source rows (only after an earlier device error) reads row 0 instead.
__device__ __forceinline__ int32_t valid_lid(const MeanArgs &m, const MeanSeg &S, int32_t u) {
    if (u >= 0 && u < S.n_src) return u;
    set_status(m.status, GNN_ERR_INTERNAL);
    return 0;
}

// The segment of item `it`.  Each segment's first item is a multiple of the items one wavefront
// takes at a time (the launcher pads the segments), so the segment is the same for every active
// lane and is found from the first one: its fields are then scalar loads, which leave the vector
// memory counter, and with it the row loads in flight, alone.
__device__ __forceinline__ int find_seg(const MeanArgs &m, uint32_t it) {
    const uint32_t it0 = __builtin_amdgcn_readfirstlane(it);
    int sgi = 0;
    while (sgi + 1 < m.nseg && m.seg[sgi + 1].item0 <= it0) ++sgi;
    return __builtin_amdgcn_readfirstlane(sgi);
}

// A segment by an index that is the same on every active lane (kept in scalar registers).
__device__ __forceinline__ const MeanSeg &seg_of(const MeanArgs &m, int sgi) {
    return m.seg[__builtin_amdgcn_readfirstlane(sgi)];
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// One group of G lanes per (destination, slab): lane gl owns the 16-byte chunks gl, gl + G, ...,
// up to CH of them (a slab; wide rows take several slabs), so one item covers a whole row of up to
// 4 G chunks.  The group reads the destination's local ids once (lane t holds edge e0 + t) and
// passes them round with cross-lane reads.  Row loads are software-pipelined over a ring of R
// edges: the sum of the oldest edge's chunks is taken and that slot is refilled with the load of
// the edge R places later, so R edges' loads stay in flight from the first edge to the last and
// no load waits on an id load or on the previous edge's sum.
template <int G, int CH, int R>
__global__ __launch_bounds__(256) void k_mean_v5(MeanArgs m) {
    const int lane = lane_id();
    const int grp = lane / G;
    const int gl = lane % G;
    const uint32_t cpr = m.cpr.d;
    const uint32_t slabs = (cpr + CH * G - 1) / (CH * G);
    __shared__ uint32_t s_n[kMaxMeanSegs];  // destination count of each segment
    if (threadIdx.x < static_cast<unsigned>(m.nseg))
        s_n[threadIdx.x] = static_cast<uint32_t>(load_count(m.seg[threadIdx.x].d_n, m.seg[threadIdx.x].n_cap));
    __syncthreads();
    const uint32_t g0 = (blockIdx.x * 4u + (threadIdx.x >> 6)) * (64 / G) + grp;
    const uint32_t gstride = gridDim.x * 4u * (64 / G);
    for (uint32_t it = g0; it < m.items; it += gstride) {
        const int sgi = find_seg(m, it);
        const MeanSeg &S = seg_of(m, sgi);
        const uint32_t li = it - S.item0;
        const uint32_t i = li / slabs;
        const uint32_t p = li - i * slabs;
        if (i >= s_n[sgi]) continue;
        int64_t e0 = S.indptr[i], e1 = S.indptr[i + 1];
        // lane g of the group: the destination's row in sub-batch g (+1; 0: absent), loaded here so
        // that it arrives with the local ids instead of after the rows
        int32_t mypos = 0;
        if (m.scat != nullptr && gl < m.scat_g) {
            // both loads in flight together: an entry without its mask bit is stale and unused
            const uint32_t mk = m.scat_mask[i];
            const int32_t pv = m.scat[static_cast<int64_t>(i) * m.scat_g + gl];
            mypos = (mk >> gl) & 1u ? pv : 0;
        }
        e0 = e0 < 0 ? 0 : (e0 > S.e_cap ? S.e_cap : e0);
        e1 = e1 < e0 ? e0 : (e1 > S.e_cap ? S.e_cap : e1);
        const uint32_t ch0 = p * CH * G + gl;  // this lane's first chunk
        bool act[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) act[q] = ch0 + q * G < cpr;
        // Chunks are read whole: rows are 16-byte aligned with ld_src a multiple of 4, so the last
        // chunk's padding columns are in the row; only the store honours d.
        const float *base = S.src + static_cast<int64_t>(ch0) * 4;
        float4 acc[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int64_t eb = e0; eb < e1; eb += G) {
            const int nb = static_cast<int>(e1 - eb < G ? e1 - eb : G);
            const int32_t mine = gl < nb ? valid_lid(m, S, S.lid[eb + gl]) : 0;
            float4 v[R][CH];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                int32_t u;
                if constexpr (G == 64) u = __builtin_amdgcn_readlane(mine, r < nb ? r : 0);
                else u = __shfl(mine, grp * G + (r < nb ? r : 0), 64);
                const float *row = base + static_cast<int64_t>(u) * m.ld_src;
#pragma unroll
                for (int q = 0; q < CH; ++q)
                    v[r][q] = (r < nb && act[q]) ? *reinterpret_cast<const float4 *>(row + q * G * 4)
                                                 : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            for (int e = 0; e < nb; e += R) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int q = 0; q < CH; ++q) acc[q] = f4add(acc[q], v[r][q]);
                    const int en = e + r + R;
                    int32_t u;
                    if constexpr (G == 64) u = __builtin_amdgcn_readlane(mine, en < nb ? en : 0);
                    else u = __shfl(mine, grp * G + (en < nb ? en : 0), 64);
                    const float *row = base + static_cast<int64_t>(u) * m.ld_src;
#pragma unroll
                    for (int q = 0; q < CH; ++q)
                        v[r][q] = (en < nb && act[q]) ? *reinterpret_cast<const float4 *>(row + q * G * 4)
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
        const int32_t c = static_cast<int32_t>(e1 - e0);
        float4 res[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            res[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c > 0) {
                const float fc = static_cast<float>(c);
                res[q] = make_float4(acc[q].x / fc, acc[q].y / fc, acc[q].z / fc, acc[q].w / fc);
            }
        }
        auto store_row = [&](float *orow) {
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                if (!act[q]) continue;
                const int col = static_cast<int>(ch0 + q * G) * 4;
                const int rem = m.d - col;
                if (rem >= 4) {
                    *reinterpret_cast<float4 *>(orow + col) = res[q];
                } else {
                    const float t[4] = {res[q].x, res[q].y, res[q].z, res[q].w};
                    for (int w = 0; w < rem; ++w) orow[col + w] = t[w];
                }
            }
        };
        if (m.scat == nullptr) {
            store_row(S.out + static_cast<int64_t>(i) * m.ld_out);
        } else {
            for (int g = 0; g < m.scat_g; ++g) {
                int32_t pos;
                if constexpr (G == 64) pos = __builtin_amdgcn_readlane(mypos, g);
                else pos = __shfl(mypos, grp * G + g, 64);
                if (pos > 0) store_row(m.scat_out[g] + static_cast<int64_t>(pos - 1) * m.ld_out);
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_mean_v1(MeanArgs m) {
    __shared__ uint32_t s_n[kMaxMeanSegs];  // destination count of each segment
    if (threadIdx.x < static_cast<unsigned>(m.nseg))
        s_n[threadIdx.x] = static_cast<uint32_t>(load_count(m.seg[threadIdx.x].d_n, m.seg[threadIdx.x].n_cap));
    __syncthreads();
    const uint32_t cpr = m.cpr.d;
    for (uint32_t it = blockIdx.x * 256u + threadIdx.x; it < m.items; it += gridDim.x * 256u) {
        const int sgi = find_seg(m, it);
        const MeanSeg &S = seg_of(m, sgi);
        const uint32_t li = it - S.item0;
        const uint32_t row = fast_div(li, m.cpr);
        const int col = static_cast<int>(li - row * cpr);
        if (row >= s_n[sgi]) continue;
        int64_t e0 = S.indptr[row], e1 = S.indptr[row + 1];
        e0 = e0 < 0 ? 0 : (e0 > S.e_cap ? S.e_cap : e0);
        e1 = e1 < e0 ? e0 : (e1 > S.e_cap ? S.e_cap : e1);
        float acc = 0.f;
        for (int64_t e = e0; e < e1; ++e)
            acc += S.src[static_cast<int64_t>(valid_lid(m, S, S.lid[e])) * m.ld_src + col];
        const int32_t c = static_cast<int32_t>(e1 - e0);
        const float val = c > 0 ? acc / static_cast<float>(c) : 0.f;
        if (m.scat == nullptr) {
            S.out[static_cast<int64_t>(row) * m.ld_out + col] = val;
        } else {
            const uint32_t mk = m.scat_mask[row];
            for (int g = 0; g < m.scat_g; ++g) {
                if (!((mk >> g) & 1u)) continue;
                const int32_t pos = m.scat[static_cast<int64_t>(row) * m.scat_g + g];
                if (pos > 0) m.scat_out[g][static_cast<int64_t>(pos - 1) * m.ld_out + col] = val;
            }
        }
    }
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static hipError_t launch_mean_impl(const MeanJob *jobs, int njobs, int64_t ld_src, int64_t ld_out,
                                   int64_t d, int32_t *status, const int32_t *scat,
                                   const uint32_t *scat_mask, int scat_g, float *const *scat_out,
                                   hipStream_t s) {
    if (njobs <= 0 || d <= 0) return hipSuccess;
    bool v4 = ld_src % 4 == 0 && ld_out % 4 == 0;
    for (int j = 0; j < njobs; ++j) v4 = v4 && aligned16(jobs[j].src) && aligned16(jobs[j].out);
    const int vec = v4 ? 4 : 1;
    const int64_t cpr = (d + vec - 1) / vec;
    const int G = !v4 ? 1 : (cpr <= 16 ? 16 : (cpr <= 32 ? 32 : 64));
    // chunk groups per lane in one item: G = 64 rows of up to 4 * 64 chunks take one item each
    const int CH = !v4 || G < 64 ? 1 : static_cast<int>((cpr + 63) / 64 < 4 ? (cpr + 63) / 64 : 4);
    const int64_t slabs = v4 ? (cpr + CH * G - 1) / (CH * G) : cpr;   // items per destination
    // items a wavefront takes at a time (64 / G groups of G lanes; one lane per item when G = 1):
    // every segment starts at a multiple of it, so that no wavefront spans two segments
    const int64_t per_wave = 64 / G;
    for (int j0 = 0; j0 < njobs; j0 += kMaxMeanSegs) {
        MeanArgs m{};
        m.scat = scat;
        m.scat_mask = scat_mask;
        m.scat_g = scat_g;
        for (int g = 0; g < scat_g; ++g) m.scat_out[g] = scat_out[g];
        m.ld_src = ld_src;
        m.ld_out = ld_out;
        m.status = status;
        m.d = static_cast<int32_t>(d);
        m.cpr = make_fastdiv(static_cast<uint32_t>(cpr));
        int64_t items = 0;
        for (int j = j0; j < njobs && j < j0 + kMaxMeanSegs; ++j) {
            const MeanJob &J = jobs[j];
            m.seg[m.nseg++] = MeanSeg{J.indptr, J.lid, J.e_cap, J.d_n, J.n_cap, J.src, J.n_src,
                                      J.out, static_cast<uint32_t>(items)};
            items += (J.n_cap * slabs + per_wave - 1) / per_wave * per_wave;
        }
        if (items == 0) continue;
        if (items > 0x7FFFFFFFLL) return hipErrorInvalidValue;
        m.items = static_cast<uint32_t>(items);
        if (!v4) {
            hipLaunchKernelGGL(k_mean_v1, dim3(grid_for(items, 256, 8192)), dim3(256), 0, s, m);
            continue;
        }
        const dim3 grid(grid_for(items, 4 * (64 / G), 8192));
        // edges in flight per group: 4 for one-chunk rows (a deeper ring costs occupancy and
        // measured slower); 2 for wider rows, whose 2-4 chunks per lane already keep several KB
        // in flight per wavefront (dense 602-float rows: 88 instead of 136 VGPRs, 5 instead of
        // 3 wavefronts per SIMD, outermost means of a super-batch of 16 0.262 -> 0.249 ms)
        constexpr int R = 4;
        constexpr int RW = 2;
        if (G == 16) hipLaunchKernelGGL((k_mean_v5<16, 1, R>), grid, dim3(256), 0, s, m);
        else if (G == 32) hipLaunchKernelGGL((k_mean_v5<32, 1, R>), grid, dim3(256), 0, s, m);
        else if (CH == 1) hipLaunchKernelGGL((k_mean_v5<64, 1, R>), grid, dim3(256), 0, s, m);
        else if (CH == 2) hipLaunchKernelGGL((k_mean_v5<64, 2, RW>), grid, dim3(256), 0, s, m);
        else if (CH == 3) hipLaunchKernelGGL((k_mean_v5<64, 3, RW>), grid, dim3(256), 0, s, m);
        else hipLaunchKernelGGL((k_mean_v5<64, 4, RW>), grid, dim3(256), 0, s, m);
    }
    return hipGetLastError();
}

hipError_t launch_mean(const MeanJob *jobs, int njobs, int64_t ld_src, int64_t ld_out, int64_t d,
                       int32_t max_c, int32_t *status, hipStream_t s) {
    (void)max_c;
    return launch_mean_impl(jobs, njobs, ld_src, ld_out, d, status, nullptr, nullptr, 0, nullptr, s);
}

hipError_t launch_mean_scatter(const MeanJob &job, const int32_t *inv, const uint32_t *inv_mask,
                               int G, float *const *outs, int64_t ld_src, int64_t ld_out, int64_t d,
                               int32_t *status, hipStream_t s) {
    if (G < 1 || G > kMaxGroup || inv == nullptr || inv_mask == nullptr) return hipErrorInvalidValue;
    return launch_mean_impl(&job, 1, ld_src, ld_out, d, status, inv, inv_mask, G, outs, s);
}

}  // namespace gnnmb
