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

struct MeanArgs {
    const int32_t *indptr;
    const int32_t *lid;
    const int64_t *d_n;
    int64_t n_cap;
    const float *src;
    int64_t ld_src;
    int64_t n_src;   // rows of src: a local id outside [0, n_src) is an error
    int64_t e_cap;   // entries of lid: edge offsets are clamped to it
    int32_t *status;
    int32_t d;
    float *out;
    int64_t ld_out;
    FastDiv cpr;
};

// A local id outside the source rows (only after an earlier device error) reads row 0 instead.
__device__ __forceinline__ int32_t valid_lid(const MeanArgs &m, int32_t u) {
    if (u >= 0 && u < m.n_src) return u;
    set_status(m.status, GNN_ERR_INTERNAL);
    return 0;
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float4 load_chunk4(const float *row, int col, int rem) {
    if (rem >= 4) return *reinterpret_cast<const float4 *>(row + col);
    float t[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < rem; ++q) t[q] = row[col + q];
    return make_float4(t[0], t[1], t[2], t[3]);
}

__global__ __launch_bounds__(256) void k_mean_v4(MeanArgs m) {
    const int64_t n = load_count(m.d_n, m.n_cap);
    const uint32_t total = static_cast<uint32_t>(n) * m.cpr.d;
    for (uint32_t idx = blockIdx.x * 256u + threadIdx.x; idx < total; idx += gridDim.x * 256u) {
        const uint32_t row = fast_div(idx, m.cpr);
        const int col = static_cast<int>(idx - row * m.cpr.d) * 4;
        const int rem = m.d - col;
        int64_t e0 = m.indptr[row], e1 = m.indptr[row + 1];
        e0 = e0 < 0 ? 0 : (e0 > m.e_cap ? m.e_cap : e0);
        e1 = e1 < e0 ? e0 : (e1 > m.e_cap ? m.e_cap : e1);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        int64_t e = e0;
        for (; e + 4 <= e1; e += 4) {
            const int32_t u0 = valid_lid(m, m.lid[e]), u1 = valid_lid(m, m.lid[e + 1]);
            const int32_t u2 = valid_lid(m, m.lid[e + 2]), u3 = valid_lid(m, m.lid[e + 3]);
            const float4 a0 = load_chunk4(m.src + static_cast<int64_t>(u0) * m.ld_src, col, rem);
            const float4 a1 = load_chunk4(m.src + static_cast<int64_t>(u1) * m.ld_src, col, rem);
            const float4 a2 = load_chunk4(m.src + static_cast<int64_t>(u2) * m.ld_src, col, rem);
            const float4 a3 = load_chunk4(m.src + static_cast<int64_t>(u3) * m.ld_src, col, rem);
            acc = f4add(acc, a0);
            acc = f4add(acc, a1);
            acc = f4add(acc, a2);
            acc = f4add(acc, a3);
        }
        for (; e < e1; ++e)
            acc = f4add(acc, load_chunk4(m.src + static_cast<int64_t>(valid_lid(m, m.lid[e])) * m.ld_src,
                                         col, rem));
        const int32_t c = static_cast<int32_t>(e1 - e0);
        float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c > 0) {
            const float fc = static_cast<float>(c);
            r = make_float4(acc.x / fc, acc.y / fc, acc.z / fc, acc.w / fc);
        }
        float *o = m.out + static_cast<int64_t>(row) * m.ld_out + col;
        if (rem >= 4) {
            *reinterpret_cast<float4 *>(o) = r;
        } else {
            const float t[4] = {r.x, r.y, r.z, r.w};
            for (int q = 0; q < rem; ++q) o[q] = t[q];
        }
    }
}

__global__ __launch_bounds__(256) void k_mean_v1(MeanArgs m) {
    const int64_t n = load_count(m.d_n, m.n_cap);
    const uint32_t total = static_cast<uint32_t>(n) * m.cpr.d;
    for (uint32_t idx = blockIdx.x * 256u + threadIdx.x; idx < total; idx += gridDim.x * 256u) {
        const uint32_t row = fast_div(idx, m.cpr);
        const int col = static_cast<int>(idx - row * m.cpr.d);
        int64_t e0 = m.indptr[row], e1 = m.indptr[row + 1];
        e0 = e0 < 0 ? 0 : (e0 > m.e_cap ? m.e_cap : e0);
        e1 = e1 < e0 ? e0 : (e1 > m.e_cap ? m.e_cap : e1);
        float acc = 0.f;
        for (int64_t e = e0; e < e1; ++e)
            acc += m.src[static_cast<int64_t>(valid_lid(m, m.lid[e])) * m.ld_src + col];
        const int32_t c = static_cast<int32_t>(e1 - e0);
        m.out[static_cast<int64_t>(row) * m.ld_out + col] = c > 0 ? acc / static_cast<float>(c) : 0.f;
    }
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipError_t launch_mean(const int32_t *indptr, const int32_t *lid, int64_t e_cap,
                       const int64_t *d_n, int64_t n_cap, const float *src, int64_t ld_src,
                       int64_t n_src, int64_t d, float *out, int64_t ld_out, int32_t *status,
                       hipStream_t s) {
    if (n_cap <= 0 || d <= 0) return hipSuccess;
    const bool v4 = ld_src % 4 == 0 && ld_out % 4 == 0 && aligned16(src) && aligned16(out);
    const int vec = v4 ? 4 : 1;
    const int64_t cpr = (d + vec - 1) / vec;
    MeanArgs m{indptr, lid, d_n, n_cap, src, ld_src, n_src, e_cap, status,
               static_cast<int32_t>(d), out, ld_out, make_fastdiv(static_cast<uint32_t>(cpr))};
    const unsigned grid = grid_for(n_cap * cpr, 256, 8192);
    if (v4) hipLaunchKernelGGL(k_mean_v4, dim3(grid), dim3(256), 0, s, m);
    else hipLaunchKernelGGL(k_mean_v1, dim3(grid), dim3(256), 0, s, m);
    return hipGetLastError();
}

}  // namespace gnnmb
