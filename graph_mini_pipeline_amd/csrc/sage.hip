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
// quarters, each four 16 x 16 MFMA accumulators (32-row tiles, which double the workgroups of a
// small block, measured slower: each still loads whole W chunks for half the rows).  K advances
// in chunks of 32 through two LDS buffers, with the global loads kDepth chunks ahead of the MFMAs
// (kDepth register sets): chunk c + 1 is stored to the other buffer after chunk c's MFMAs, so one
// barrier per chunk suffices.
// Workgroups b and b + 8 (the same XCD under round-robin dispatch) take the N tiles of one M
// tile, so the A rows they share are fetched into one L2.
#include "common.hpp"

namespace gnnmb {

namespace {

constexpr int kSageThreads = 256;
constexpr int kBM = 64, kBN = 64, kBK = 32;
constexpr int kDepth = 4;          // chunks of global loads in flight (measured best of 2..5)
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
    constexpr int BM = kBM;
    constexpr int EA = BM * kBK / kSageThreads;   // A values per thread per chunk
    constexpr int TPR = kBK / EA;                 // threads per A row
    constexpr int EB = kBK * kBN / kSageThreads;  // B values per thread per chunk
    constexpr int TPB = kBN / EB;                 // threads per B row
    constexpr int MI = BM / 32;                   // 16 x 16 accumulators per wavefront along M
    __shared__ float As[2][BM * kAStride];
    __shared__ float Bs[2][kBK * kBStride];
    // XCD-aware tile order: 8 consecutive M tiles, then the next N tile of the same 8.
    const int b = static_cast<int>(blockIdx.x);
    const int grp = b / (kXcds * a.n_tiles);
    const int in_grp = b - grp * (kXcds * a.n_tiles);
    const int mt = grp * kXcds + in_grp % kXcds;
    const int nt = in_grp / kXcds;
    if (mt >= a.m_tiles) return;   // whole workgroup
    const int64_t n_act = load_count(a.d_n, a.n_cap);
    const int64_t m0 = static_cast<int64_t>(mt) * BM;
    if (m0 >= n_act) return;       // whole workgroup
    const int64_t n0 = static_cast<int64_t>(nt) * kBN;
    const int t = static_cast<int>(threadIdx.x);
    const int lane = lane_id();
    const int wv = t >> 6;
    const int wm = wv & 1, wn = wv >> 1;

    // This thread's A row (r) and its EA columns (from ac), B row (bk) and column octet (bc).
    const int r = t / TPR, ac = (t % TPR) * EA;
    const int bk = t / TPB, bc = (t % TPB) * EB;
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
    // K runs over two segments, each padded to whole chunks: the node's own row (W rows 0..d)
    // then the mean (W rows d..2d), so a chunk's columns start at a multiple of 32 inside one
    // source row.  Octets that lie inside the row use 16-byte loads when rows are 16-byte aligned.
    const int seg_chunks = static_cast<int>((a.d + kBK - 1) / kBK);
    const bool a_vec = (a.ld_src % 4 == 0) && (a.ld_agg % 4 == 0) &&
                       ((reinterpret_cast<uintptr_t>(a.src) | reinterpret_cast<uintptr_t>(a.agg)) % 16 == 0);
    const bool b_vec = (a.d_out % 4 == 0) && (reinterpret_cast<uintptr_t>(a.W) % 16 == 0);
    auto load_chunk = [&](int c, f4 (&ra)[EA / 4], f4 (&rb)[EB / 4]) {
        const bool own = c < seg_chunks;
        const int64_t k0 = static_cast<int64_t>(own ? c : c - seg_chunks) * kBK;
        const float *row = own ? self_row : agg_row;
        const int64_t kk = k0 + ac;
        if (!row_ok || kk >= a.d) {
#pragma unroll
            for (int v = 0; v < EA / 4; ++v) ra[v] = f4{0.f, 0.f, 0.f, 0.f};
        } else if (a_vec && kk + EA <= a.d) {
            const f4 *p = reinterpret_cast<const f4 *>(row + kk);
#pragma unroll
            for (int v = 0; v < EA / 4; ++v) ra[v] = p[v];
        } else {
#pragma unroll
            for (int u = 0; u < EA; ++u) ra[u >> 2][u & 3] = kk + u < a.d ? row[kk + u] : 0.f;
        }
        const int64_t k = k0 + bk;
        const int64_t n = n0 + bc;
        const float *wrow = a.W + ((own ? 0 : a.d) + k) * a.d_out;
        if (k >= a.d || n >= a.d_out) {
#pragma unroll
            for (int v = 0; v < EB / 4; ++v) rb[v] = f4{0.f, 0.f, 0.f, 0.f};
        } else if (b_vec && n + EB <= a.d_out) {
            const f4 *p = reinterpret_cast<const f4 *>(wrow + n);
#pragma unroll
            for (int v = 0; v < EB / 4; ++v) rb[v] = p[v];
        } else {
#pragma unroll
            for (int u = 0; u < EB; ++u) rb[u >> 2][u & 3] = n + u < a.d_out ? wrow[n + u] : 0.f;
        }
    };
    auto store_chunk = [&](int buf, const f4 (&ra)[EA / 4], const f4 (&rb)[EB / 4]) {
#pragma unroll
        for (int u = 0; u < EA; ++u) As[buf][r * kAStride + ac + u] = ra[u >> 2][u & 3];
#pragma unroll
        for (int u = 0; u < EB; ++u) Bs[buf][bk * kBStride + bc + u] = rb[u >> 2][u & 3];
    };

    f4 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // kDepth chunks of loads in flight: at chunk c, chunks c + 1 .. c + kDepth - 1 sit in register
    // sets (c + 1) % kDepth ..., while chunk c + kDepth is fetched into set c % kDepth, whose chunk
    // c went to LDS one step earlier.  The loop is unrolled by kDepth so that the sets are
    // registers.
    const int nchunks = 2 * seg_chunks;
    f4 ra[kDepth][EA / 4], rb[kDepth][EB / 4];
#pragma unroll
    for (int q = 0; q < kDepth; ++q)
        if (q < nchunks) load_chunk(q, ra[q], rb[q]);
    store_chunk(0, ra[0], rb[0]);
    __syncthreads();
    const int arow = wm * (BM / 2) + (lane & 15);
    const int bcol = wn * 32 + (lane & 15);
    const int kq = lane >> 4;
    auto step = [&](int c, f4 (&la)[EA / 4], f4 (&lb)[EB / 4], const f4 (&sa)[EA / 4],
                    const f4 (&sb)[EB / 4]) {
        if (c + kDepth < nchunks) load_chunk(c + kDepth, la, lb);
        const float *A = As[c & 1];
        const float *B = Bs[c & 1];
#pragma unroll
        for (int ks = 0; ks < kBK / 4; ++ks) {
            const int kr = ks * 4 + kq;
            float av[MI], bv[2];
#pragma unroll
            for (int i = 0; i < MI; ++i) av[i] = A[(arow + i * 16) * kAStride + kr];
#pragma unroll
            for (int j = 0; j < 2; ++j) bv[j] = B[kr * kBStride + bcol + j * 16];
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (c + 1 < nchunks) store_chunk((c + 1) & 1, sa, sb);
        __syncthreads();
    };
    for (int c = 0; c < nchunks; c += kDepth) {
#pragma unroll
        for (int q = 0; q < kDepth; ++q)
            if (c + q < nchunks)
                step(c + q, ra[q], rb[q], ra[(q + 1) % kDepth], rb[(q + 1) % kDepth]);
    }

    // Lane holds rows 4 * (lane / 16) + q, column lane % 16 of each 16 x 16 accumulator.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (col >= a.d_out) continue;
        const float bj = a.bias ? a.bias[col] : 0.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = m0 + wm * (BM / 2) + i * 16 + 4 * kq + q;
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
    a.n_tiles = static_cast<int32_t>((d_out + kBN - 1) / kBN);
    a.status = status;
    a.m_tiles = static_cast<int32_t>((n_cap + kBM - 1) / kBM);
    const int64_t groups = (a.m_tiles + kXcds - 1) / kXcds;
    const int64_t grid = groups * kXcds * a.n_tiles;
    hipLaunchKernelGGL(k_sage_update, dim3(static_cast<unsigned>(grid)), dim3(kSageThreads), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace gnnmb
