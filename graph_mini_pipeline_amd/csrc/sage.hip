// The dense UPDATE of a GraphSAGE-mean layer on the matrix cores.
//
// GARDEN (Sec. II.A, eq. (1)-(2)) writes a GNN layer as AGGREGATE over the sampled neighbours
// followed by a learnable UPDATE of the node's previous state and that message; its Sec. VI.A
// trains GraphSAGE, whose mean layer concatenates the two and applies one dense layer.  The mean
// comes from the aggregation kernel; this kernel computes
//   out[i, n] = act( sum_{k<d} src[dst_lid[i], k] W[k, n] + sum_{k<d} agg[i, k] W[d+k, n] + b[n] )
// as a [n_dst x 2d] x [2d x d_out] product whose A rows are gathered on the fly: the first d
// columns of row i are the destination's own row of src (its position dst_lid[i]), the last d the
// mean.  fp32 in, fp32 matrix-core products (v_mfma_f32_16x16x4_f32), fp32 accumulation.
//
// Tiling: a 256-thread workgroup owns a 64 x 64 output tile; its four wavefronts own 32 x 32
// quarters, each four 16 x 16 MFMA accumulators.  K advances in chunks of 32 through two LDS
// buffers: the next chunk's global loads are issued before the current chunk's MFMAs and stored
// to the other buffer after them, so one barrier per chunk suffices.  Workgroups b and b + 8 (the
// same XCD under round-robin dispatch) take the N tiles of one M tile, so the A rows they share
// are fetched into one L2.
#include "common.hpp"

namespace gnnmb {

namespace {

constexpr int kSageThreads = 256;
constexpr int kBM = 64, kBN = 64, kBK = 32;
constexpr int kAStride = kBK + 4;    // LDS row strides chosen so that one MFMA operand read
constexpr int kBStride = kBN + 16;   // touches 64 distinct banks
constexpr int kXcds = 8;

typedef float f4 __attribute__((ext_vector_type(4)));

struct SageArgs {
    const int32_t *dst_lid;
    const int64_t *d_n;
    int64_t n_cap;
    const float *src;
    int64_t ld_src;
    int64_t n_src;
    const float *agg;
    int64_t ld_agg;
    int64_t d;
    const float *W;
    const float *bias;
    int64_t d_out;
    int32_t relu;
    float *out;
    int64_t ld_out;
    int32_t m_tiles;
    int32_t n_tiles;
    int32_t *status;
};

__global__ __launch_bounds__(kSageThreads) void k_sage_update(SageArgs a) {
    __shared__ float As[2][kBM * kAStride];
    __shared__ float Bs[2][kBK * kBStride];
    // XCD-aware tile order: 8 consecutive M tiles, then the next N tile of the same 8.
    const int b = static_cast<int>(blockIdx.x);
    const int grp = b / (kXcds * a.n_tiles);
    const int in_grp = b - grp * (kXcds * a.n_tiles);
    const int mt = grp * kXcds + in_grp % kXcds;
    const int nt = in_grp / kXcds;
    if (mt >= a.m_tiles) return;   // whole workgroup
    const int64_t n_act = load_count(a.d_n, a.n_cap);
    const int64_t m0 = static_cast<int64_t>(mt) * kBM;
    if (m0 >= n_act) return;       // whole workgroup
    const int64_t n0 = static_cast<int64_t>(nt) * kBN;
    const int t = static_cast<int>(threadIdx.x);
    const int lane = lane_id();
    const int wv = t >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    const int64_t K = 2 * a.d;

    // This thread's A row (r) and column octet (ac) and B row (bk) and column octet (bc).
    const int r = t >> 2, ac = (t & 3) * 8;
    const int bk = t >> 3, bc = (t & 7) * 8;
    const int64_t m = m0 + r;
    const bool row_ok = m < n_act;
    const float *self_row = a.src;
    const float *agg_row = a.agg;
    if (row_ok) {
        int32_t dl = a.dst_lid[m];
        if (dl < 0 || dl >= a.n_src) {
            set_status(a.status, GNN_ERR_INTERNAL);
            dl = 0;
        }
        self_row = a.src + static_cast<int64_t>(dl) * a.ld_src;
        agg_row = a.agg + m * a.ld_agg;
    }
    float ra[8], rb[8];
    auto load_chunk = [&](int64_t k0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t kk = k0 + ac + u;
            float v = 0.f;
            if (row_ok && kk < K) v = kk < a.d ? self_row[kk] : agg_row[kk - a.d];
            ra[u] = v;
        }
        const int64_t k = k0 + bk;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t n = n0 + bc + u;
            rb[u] = (k < K && n < a.d_out) ? a.W[k * a.d_out + n] : 0.f;
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 8; ++u) As[buf][r * kAStride + ac + u] = ra[u];
#pragma unroll
        for (int u = 0; u < 8; ++u) Bs[buf][bk * kBStride + bc + u] = rb[u];
    };

    f4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = static_cast<int>((K + kBK - 1) / kBK);
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    const int arow = wm * 32 + (lane & 15);
    const int bcol = wn * 32 + (lane & 15);
    const int kq = lane >> 4;
    for (int c = 0; c < nchunks; ++c) {
        const int cur = c & 1;
        const bool more = c + 1 < nchunks;
        if (more) load_chunk(static_cast<int64_t>(c + 1) * kBK);
        const float *A = As[cur];
        const float *B = Bs[cur];
#pragma unroll
        for (int ks = 0; ks < kBK / 4; ++ks) {
            const int kr = ks * 4 + kq;
            float av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) av[i] = A[(arow + i * 16) * kAStride + kr];
#pragma unroll
            for (int j = 0; j < 2; ++j) bv[j] = B[kr * kBStride + bcol + j * 16];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (more) store_chunk(cur ^ 1);
        __syncthreads();
    }

    // Lane holds rows 4 * (lane / 16) + q, column lane % 16 of each 16 x 16 accumulator.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (col >= a.d_out) continue;
        const float bj = a.bias ? a.bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = m0 + wm * 32 + i * 16 + 4 * kq + q;
                if (row >= n_act) continue;
                float v = acc[i][j][q] + bj;
                if (a.relu && v < 0.f) v = 0.f;
                a.out[row * a.ld_out + col] = v;
            }
    }
}

}  // namespace

hipError_t launch_sage_update(const int32_t *dst_lid, const int64_t *d_n, int64_t n_cap,
                              const float *src, int64_t ld_src, int64_t n_src, const float *agg,
                              int64_t ld_agg, int64_t d, const float *W, const float *bias,
                              int64_t d_out, int32_t relu, float *out, int64_t ld_out,
                              int32_t *status, hipStream_t s) {
    if (n_cap <= 0 || d_out <= 0) return hipSuccess;
    SageArgs a{};
    a.dst_lid = dst_lid;
    a.d_n = d_n;
    a.n_cap = n_cap;
    a.src = src;
    a.ld_src = ld_src;
    a.n_src = n_src;
    a.agg = agg;
    a.ld_agg = ld_agg;
    a.d = d;
    a.W = W;
    a.bias = bias;
    a.d_out = d_out;
    a.relu = relu;
    a.out = out;
    a.ld_out = ld_out;
    a.m_tiles = static_cast<int32_t>((n_cap + kBM - 1) / kBM);
    a.n_tiles = static_cast<int32_t>((d_out + kBN - 1) / kBN);
    a.status = status;
    const int64_t groups = (a.m_tiles + kXcds - 1) / kXcds;
    const int64_t grid = groups * kXcds * a.n_tiles;
    hipLaunchKernelGGL(k_sage_update, dim3(static_cast<unsigned>(grid)), dim3(kSageThreads), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace gnnmb
