// Split-K reductions: the K-split partials of the GEMV and GEMM routes summed in split order,
// so a result never depends on the launch.
//
//   * reduce_splits_kernel: row-major partials [splits][M][ld] (the streaming GEMVs and the
//     16x16x32 input gradient), up to three column segments;
//   * reduce_frags_kernel: partials in the 32x32 MFMA fragment order of the forward, input
//     gradient and dq8ca GEMMs (see internal.h), optionally adding the adapter's low-rank term.
#include "device.h"
#include "internal.h"

namespace q4gsw {

// Split-partial reduction: y_seg[m][c] = sum_s ws[s][m][off_seg + c] for c < cols_seg, over up to
// three column segments that share the workspace rows (the fused QKV's three outputs).  A block
// covers 4 rows x 256 columns, each thread 4 consecutive columns with 16-byte loads; segment
// starts and the row pitch are multiples of 4 columns.
struct ReduceSegs {
    float* y[3];
    int64_t y_ld[3];
    int64_t off[3];              // first workspace column of the segment
    int64_t cols[3];             // valid columns of the segment
    int nseg;
};

__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ ws, int splits, int64_t M,
                                                            int64_t ld, ReduceSegs seg, int vec_ok) {
    const int64_t c = ((int64_t)blockIdx.x * 64 + (threadIdx.x & 63)) * 4;
    if (c >= ld) return;
    int sg = 0;
    while (sg + 1 < seg.nseg && c >= seg.off[sg + 1]) ++sg;
    const int64_t cs = c - seg.off[sg];
    if (cs >= seg.cols[sg]) return;
    const int64_t plane = M * ld;
    for (int64_t m = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6); m < M; m += (int64_t)gridDim.y * 4) {
        const float* src = ws + m * ld + c;
        f4 acc = *reinterpret_cast<const f4*>(src);
        for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const f4*>(src + s * plane);
        float* dst = seg.y[sg] + m * seg.y_ld[sg] + cs;
        if (vec_ok && cs + 4 <= seg.cols[sg]) {
            *reinterpret_cast<f4*>(dst) = acc;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (cs + e < seg.cols[sg]) dst[e] = acc[e];
        }
    }
}

hipError_t launch_reduce_segments(const float* ws, int splits, int64_t M, int64_t ld, const float* const* y,
                                  const int64_t* y_ld, const int64_t* off, const int64_t* cols, int nseg,
                                  hipStream_t s) {
    ReduceSegs seg{};
    seg.nseg = nseg;
    int vec_ok = (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(ws) & 15u) == 0);
    for (int i = 0; i < nseg; ++i) {
        seg.y[i] = const_cast<float*>(y[i]);
        seg.y_ld[i] = y_ld[i];
        seg.off[i] = off[i];
        seg.cols[i] = cols[i];
        if (off[i] % 4 != 0) return hipErrorInvalidValue;
        vec_ok = vec_ok && (y_ld[i] % 4 == 0) && ((reinterpret_cast<uintptr_t>(y[i]) & 15u) == 0);
    }
    if (ld % 4 != 0 || (reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return hipErrorInvalidValue;
    const int64_t row_blocks = (M + 3) / 4;
    const dim3 grid((unsigned)((ld / 4 + 63) / 64), (unsigned)(row_blocks < 65535 ? row_blocks : 65535));
    hipLaunchKernelGGL(reduce_splits_kernel, grid, dim3(256), 0, s, ws, splits, M, ld, seg, vec_ok);
    return hipGetLastError();
}

// Split-partial reduction over the 32x32 MFMA fragment layout (see internal.h): one block per
// 32x32 tile, thread t sums the 4 rows q of fragment slot t (register group r4 = t / 64, lane
// L = t % 64: rows 8 r4 + 4 (L / 32) + q, column j = L % 32, or its octet permutation when perm
// is set) with one streaming 16-byte load per split, in split order, so the result does not
// depend on the launch.  The tile is transposed through LDS so that each thread stores 4 consecutive columns
// of one row.  R > 0 (rank bucket): the low-rank term of LowRankEpi is added to each sum, from the
// tile's rows of T and columns of G staged in the same LDS array (one segment only).  BATCH: the
// split loads are issued eight at a time instead of one round trip each (same sums in the same
// order): faster for launches of under two blocks per CU, slower for larger ones (the partial
// planes are 4 MB apart), so the launcher picks it by tile count.
template <int R, bool BATCH>
__global__ __launch_bounds__(256) void reduce_frags_kernel(const float* __restrict__ ws, int splits, int64_t M,
                                                           int64_t ntn, int64_t plane, ReduceSegs seg, int perm,
                                                           int vec_ok, LowRankEpi lr) {
    constexpr int kLR = R > 0 ? 32 * R + R * 33 : 0;
    __shared__ float sm[32 * 33 + kLR];
    float (*tile_s)[33] = reinterpret_cast<float (*)[33]>(sm);
    const int64_t tile = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t tm = tile / ntn, tn = tile - tm * ntn;
    const float* src = ws + tile * 1024 + 4 * t;
    f4 acc = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src));
    // R > 0: this thread's values of the tile's rows of T (their first NB chunk partials) and
    // columns of G are loaded next, in flight with the split partials
    constexpr int TPT = R > 0 ? (32 * R + 255) / 256 : 1;     // values of T (and of G) per thread
    constexpr int NB = TPT <= 2 ? 16 : 32 / TPT;
    float tp[TPT][NB];
    float gv[TPT];
    if constexpr (R > 0) {
        const int64_t C = seg.cols[0];
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = t + 256 * k, r = i / R, j = i % R;
            const int64_t m = 32 * tm + r;
            const bool ok = i < 32 * R && m < M && j < lr.rank;
#pragma unroll
            for (int c = 0; c < NB; ++c)
                tp[k][c] = load_sel(lr.P, (c * M + m) * lr.rank + j, ok && c < lr.chunks);
            const int jg = i / 32, cc = i % 32;
            const int64_t col = 32 * tn + cc;
            gv[k] = load_sel(lr.G, lr.gt == 0 ? (int64_t)jg * C + col : col * lr.rank + jg,
                             i < 32 * R && jg < lr.rank && col < C);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (BATCH) {
        for (int s0 = 1; s0 < splits; s0 += 8) {
            f4 p[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int sk = s0 + k < splits ? s0 + k : 0;     // plane 0 stands in past the last split
                p[k] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + sk * plane));
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (s0 + k < splits) acc += p[k];
        }
    } else {
        for (int s = 1; s < splits; ++s)
            acc += __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + s * plane));
    }
    {
        const int L = t & 63, j = L & 31;
        const int jc = perm ? ((j & ~7) | ((j & 3) << 1) | ((j >> 2) & 1)) : j;
        const int r0 = 8 * (t >> 6) + 4 * (L >> 5);
#pragma unroll
        for (int q = 0; q < 4; ++q) tile_s[r0 + q][jc] = acc[q];
    }
    if constexpr (R > 0) {
        // T: chunk sums in chunk order (the first NB from the registers); G as loaded
        float* t_s = sm + 32 * 33;       // [32][R]
        float* g_s = t_s + 32 * R;       // [R][33]
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = t + 256 * k, r = i / R, j = i % R;
            const int64_t m = 32 * tm + r;
            if (i < 32 * R) {
                float v = 0.0f;
#pragma unroll
                for (int c = 0; c < NB; ++c) v += tp[k][c];          // past the last partial: + 0, exact
                const bool ok = m < M && j < lr.rank;
                for (int64_t c0 = NB; c0 < lr.chunks; c0 += 16) {        // the rest, continuing the order
                    float p[16];
#pragma unroll
                    for (int c = 0; c < 16; ++c)
                        p[c] = load_sel(lr.P, ((c0 + c) * M + m) * lr.rank + j, ok && c0 + c < lr.chunks);
#pragma unroll
                    for (int c = 0; c < 16; ++c) v += p[c];
                }
                if (lr.Tout && tn == 0 && m < M && j < lr.rank) lr.Tout[m * lr.rank + j] = v;
                t_s[i] = v;
                g_s[(i / 32) * 33 + i % 32] = gv[k];
            }
        }
    }
    __syncthreads();
    const int row = t >> 3, c4 = 4 * (t & 7);
    const int64_t m = 32 * tm + row;
    if (m >= M) return;
    const int64_t col = 32 * tn + c4;
    int sg = 0;
    while (sg + 1 < seg.nseg && col >= seg.off[sg + 1]) ++sg;
    const int64_t cs = col - seg.off[sg];
    if (cs >= seg.cols[sg]) return;
    float* dst = seg.y[sg] + m * seg.y_ld[sg] + cs;
    f4 v = {tile_s[row][c4], tile_s[row][c4 + 1], tile_s[row][c4 + 2], tile_s[row][c4 + 3]};
    if constexpr (R > 0) {
        const float* t_s = sm + 32 * 33;
        const float* g_s = t_s + 32 * R;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < R; ++j) sum = fmaf(t_s[row * R + j], g_s[j * 33 + c4 + q], sum);
            v[q] = fmaf(lr.alpha, sum, v[q]);
        }
    }
    if (vec_ok && cs + 4 <= seg.cols[sg]) {
        *reinterpret_cast<f4*>(dst) = v;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (cs + e < seg.cols[sg]) dst[e] = v[e];
    }
}

hipError_t launch_reduce_frags(const float* ws, int splits, int64_t M, int64_t width, const float* const* y,
                               const int64_t* y_ld, const int64_t* off, const int64_t* cols, int nseg, int perm,
                               hipStream_t s, const LowRankEpi* lr) {
    if (width % 32 != 0 || (reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return hipErrorInvalidValue;
    if (lr && (nseg != 1 || lr->rank < 1 || lr->rank > 64)) return hipErrorInvalidValue;
    ReduceSegs seg{};
    seg.nseg = nseg;
    int vec_ok = 1;
    for (int i = 0; i < nseg; ++i) {
        seg.y[i] = const_cast<float*>(y[i]);
        seg.y_ld[i] = y_ld[i];
        seg.off[i] = off[i];
        seg.cols[i] = cols[i];
        if (off[i] % 32 != 0) return hipErrorInvalidValue;
        vec_ok = vec_ok && (y_ld[i] % 4 == 0) && ((reinterpret_cast<uintptr_t>(y[i]) & 15u) == 0);
    }
    const int64_t mt = (M + 31) / 32, ntn = width / 32;
    const int64_t tiles = mt * ntn;
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles);
    const int64_t plane = mt * 32 * width;
    const LowRankEpi none{};
    if (!lr && tiles < 512) {
        hipLaunchKernelGGL((reduce_frags_kernel<0, true>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm,
                           vec_ok, none);
    } else if (!lr) {
        hipLaunchKernelGGL((reduce_frags_kernel<0, false>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm,
                           vec_ok, none);
    } else if (lr->rank <= 4) {
        hipLaunchKernelGGL((reduce_frags_kernel<4, false>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm, vec_ok,
                           *lr);
    } else if (lr->rank <= 8) {
        hipLaunchKernelGGL((reduce_frags_kernel<8, false>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm, vec_ok,
                           *lr);
    } else if (lr->rank <= 16) {
        hipLaunchKernelGGL((reduce_frags_kernel<16, false>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm, vec_ok,
                           *lr);
    } else if (lr->rank <= 32) {
        hipLaunchKernelGGL((reduce_frags_kernel<32, false>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm, vec_ok,
                           *lr);
    } else {
        hipLaunchKernelGGL((reduce_frags_kernel<64, false>), grid, dim3(256), 0, s, ws, splits, M, ntn, plane, seg, perm, vec_ok,
                           *lr);
    }
    return hipGetLastError();
}

hipError_t launch_reduce_splits(const float* ws, int splits, int64_t M, int64_t cols, int64_t ld, float* y,
                                int64_t y_ld, hipStream_t s) {
    const float* yy[1] = {y};
    const int64_t yl[1] = {y_ld}, of[1] = {0}, cl[1] = {cols};
    return launch_reduce_segments(ws, splits, M, ld, yy, yl, of, cl, 1, s);
}

}  // namespace q4gsw
