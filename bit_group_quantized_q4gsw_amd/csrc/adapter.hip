// The adapter step around the frozen q4gsw base: a rank-r low-rank adapter beside the packed
// weight and the AdamW update of its factors.
//
// The input-gradient page (the Vulkan linear_q4gsw_backward pull request) says its op serves
// on-device adapter training around the frozen base, and its stack lists an on-GPU AdamW step;
// the pages give no adapter mathematics.  Reading: LoRA factors A [r, K] and B [N, r] in fp32,
//   t = x A^T [M, r],  y = x W^T + alpha t B^T,
//   u = d_out B [M, r],  d_x = d_out W + alpha u A,  d_A = alpha u^T x,  d_B = alpha d_out^T t,
// and AdamW (decoupled weight decay, bias-corrected moments).  The W terms are the library's
// forward and input gradient; this file holds the low-rank terms and the optimizer:
//
//   * rank_contract_kernel: out[m, j] = sum_c X[m, c] F(j, c) over one row of X per block (t, u);
//   * rank_expand_kernel:   Y[m, c] += alpha sum_j T[m, j] G(j, c) (the y and d_x updates);
//   * column_contract_kernel: O(j, c) = alpha sum_m T[m, j] X[m, c] (d_A, d_B);
//   * adamw_kernel: the elementwise update.
//
// F and G are A (row j at A + j K, columns c) or B^T (row j at B + j, stride r); O is written
// [r, C] (d_A) or [C, r] (d_B).  Every output is summed by one thread (or one block, in a fixed
// tree), in an order fixed by the shape alone.  Rounding: the row contraction sums C / 256 terms
// per thread and then a 256-way tree; the column contraction sums runs of kRun rows, the runs of a
// slab in order and then the slabs in order; the expansion sums the r terms in order and adds once.
#include "device.h"
#include "internal.h"

#include <cmath>
#include <type_traits>

namespace q4gsw {
namespace {

constexpr int kRankMax = 64;
constexpr int kRun = 32;               // rows per partial sum in the column contraction

// Rows of X per block in the row contraction: the factor is read once per block, so more rows
// cut its re-reads; the accumulators (rows x rank bucket) stay within 64 registers.
template <int R>
constexpr int contract_rows() { return R >= 64 ? 1 : R >= 32 ? 2 : R >= 16 ? 4 : 8; }

// out[m * r + j] = sum_c X[m, c] F(j, c) for X [M, C] (dtype XT); a block (256 threads) takes
// contract_rows<R>() consecutive rows.  FT = 0: F(j, c) = A[j * C + c]; FT = 1: F(j, c) = B[c * r + j].
template <int XT, int R, int FT>
__global__ __launch_bounds__(256) void rank_contract_kernel(const void* __restrict__ X, int64_t M, int64_t C,
                                                            const float* __restrict__ F, int rank,
                                                            float* __restrict__ out) {
    constexpr int RB = contract_rows<R>();
    __shared__ float red[4][RB * R];
    const int64_t m0 = (int64_t)blockIdx.x * RB;
    const int tid = threadIdx.x;
    const int rows = (int)min((int64_t)RB, M - m0);
    float acc[RB][R];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[i][j] = 0.0f;
    for (int64_t c = tid; c < C; c += 256) {
        float f[R];
#pragma unroll
        for (int j = 0; j < R; ++j) f[j] = j < rank ? (FT == 0 ? F[(int64_t)j * C + c] : F[c * rank + j]) : 0.0f;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (i < rows) {
                const float xv = load_elem<XT>(X, (m0 + i) * C + c);
#pragma unroll
                for (int j = 0; j < R; ++j) acc[i][j] = fmaf(xv, f[j], acc[i][j]);
            }
        }
    }
    // fixed tree: the wave's 64 lanes by xor steps, then the 4 waves in order
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
            float v = acc[i][j];
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
            acc[i][j] = v;
        }
    if ((tid & 63) == 0) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < R; ++j) red[tid >> 6][i * R + j] = acc[i][j];
    }
    __syncthreads();
    for (int e = tid; e < RB * R; e += 256) {
        const int i = e / R, j = e % R;
        if (i < rows && j < rank)
            out[(m0 + i) * rank + j] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
    }
}

// Y [M, C] (row-major, fp32) += alpha * T [M, r] . G, G(j, c) = A[j * C + c] (GT = 0) or
// B[c * r + j] (GT = 1).  Block: 8 rows x 256 columns; thread = one column, 8 rows.
template <int R, int GT>
__global__ __launch_bounds__(256) void rank_expand_kernel(float* __restrict__ Y, int64_t M, int64_t C,
                                                          const float* __restrict__ T, const float* __restrict__ G,
                                                          int rank, float alpha) {
    __shared__ float ts[8][R];
    const int tid = threadIdx.x;
    const int64_t c = (int64_t)blockIdx.x * 256 + tid;
    const bool live = c < C;
    float g[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
        g[j] = (live && j < rank) ? (GT == 0 ? G[(int64_t)j * C + c] : G[c * rank + j]) : 0.0f;
    for (int64_t m0 = (int64_t)blockIdx.y * 8; m0 < M; m0 += (int64_t)gridDim.y * 8) {
        __syncthreads();
        for (int i = tid; i < 8 * R; i += 256) {
            const int r = i / R, j = i % R;
            ts[r][j] = (m0 + r < M && j < rank) ? T[(m0 + r) * rank + j] : 0.0f;
        }
        __syncthreads();
        if (!live) continue;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t m = m0 + r;
            if (m >= M) break;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < R; ++j) s = fmaf(ts[r][j], g[j], s);
            Y[m * C + c] = fmaf(alpha, s, Y[m * C + c]);
        }
    }
}

// O(j, c) = alpha * sum_m T[m, j] X[m, c] for X [M, C] (dtype XT) and T [M, r] (fp32); thread = one
// column c of a 256-column block, all j.  Rows are cut into slabs of `slab` rows (a multiple of
// kRun), one slab per blockIdx.y; within a slab, runs of kRun rows are summed apart and then in
// order.  One slab: O is written directly, OT = 0: O[j * C + c] (d_A, [r, C]), OT = 1:
// O[c * r + j] (d_B, [C, r]).  Several: the slab sums go to P [slabs, r, C] unscaled, and
// column_reduce_kernel adds them in slab order.
template <int XT, int R, int OT>
__global__ __launch_bounds__(256) void column_contract_kernel(const void* __restrict__ X, int64_t M, int64_t C,
                                                              const float* __restrict__ T, int rank, float alpha,
                                                              int64_t slab, float* __restrict__ O,
                                                              float* __restrict__ P) {
    __shared__ float ts[kRun][R];
    const int tid = threadIdx.x;
    const int64_t c = (int64_t)blockIdx.x * 256 + tid;
    const bool live = c < C;
    const int64_t lo = (int64_t)blockIdx.y * slab, hi = min(M, lo + slab);
    float tot[R];
#pragma unroll
    for (int j = 0; j < R; ++j) tot[j] = 0.0f;
    for (int64_t r0 = lo; r0 < hi; r0 += kRun) {
        __syncthreads();
        for (int i = tid; i < kRun * R; i += 256) {
            const int r = i / R, j = i % R;
            ts[r][j] = (r0 + r < hi && j < rank) ? T[(r0 + r) * rank + j] : 0.0f;
        }
        __syncthreads();
        float run[R];
#pragma unroll
        for (int j = 0; j < R; ++j) run[j] = 0.0f;
        const int rows = (int)min((int64_t)kRun, hi - r0);
        if (live) {
            for (int r = 0; r < rows; ++r) {
                const float xv = load_elem<XT>(X, (r0 + r) * C + c);
#pragma unroll
                for (int j = 0; j < R; ++j) run[j] = fmaf(ts[r][j], xv, run[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < R; ++j) tot[j] += run[j];
    }
    if (!live) return;
    if (P) {
        float* ps = P + (int64_t)blockIdx.y * rank * C;
#pragma unroll
        for (int j = 0; j < R; ++j)
            if (j < rank) ps[(int64_t)j * C + c] = tot[j];
        return;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < rank) {
            if (OT == 0) O[(int64_t)j * C + c] = alpha * tot[j];
            else O[c * rank + j] = alpha * tot[j];
        }
    }
}

// O(j, c) = alpha * (P[0, j, c] + P[1, j, c] + ... ) in slab order; one thread per (j, c) of
// r x C, c fastest; O laid out as in column_contract_kernel.
template <int OT>
__global__ __launch_bounds__(256) void column_reduce_kernel(const float* __restrict__ P, int slabs, int64_t C,
                                                            int rank, float alpha, float* __restrict__ O) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)rank * C) return;
    const int64_t stride = (int64_t)rank * C;
    float s = 0.0f;
    for (int i = 0; i < slabs; ++i) s += P[i * stride + e];
    const int64_t j = e / C, c = e % C;
    if (OT == 0) O[e] = alpha * s;
    else O[c * rank + j] = alpha * s;
}

// AdamW on n fp32 values: p *= decay; m = b1 m + (1 - b1) g; v = b2 v + (1 - b2) g^2;
// p -= step_size * m / (sqrt(v) * inv_sqrt_bias2 + eps), with decay = 1 - lr wd,
// step_size = lr / (1 - b1^s) and inv_sqrt_bias2 = 1 / sqrt(1 - b2^s) from the host.
struct AdamwArgs {
    float decay, beta1, one_m_beta1, beta2, one_m_beta2, step_size, inv_sqrt_bias2, eps;
};

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const AdamwArgs& a) {
    p *= a.decay;
    m = fmaf(a.beta1, m, a.one_m_beta1 * g);
    v = fmaf(a.beta2, v, a.one_m_beta2 * (g * g));
    const float denom = fmaf(__builtin_sqrtf(v), a.inv_sqrt_bias2, a.eps);
    p = fmaf(-a.step_size, m / denom, p);
}

template <bool VEC>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                    AdamwArgs a) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    if constexpr (VEC) {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; 4 * i < n; i += stride) {
            f4 pp = reinterpret_cast<f4*>(p)[i];
            const f4 gg = reinterpret_cast<const f4*>(g)[i];
            f4 mm = reinterpret_cast<f4*>(m)[i];
            f4 vv = reinterpret_cast<f4*>(v)[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float pe = pp[e], me = mm[e], ve = vv[e];
                adamw_one(pe, gg[e], me, ve, a);
                pp[e] = pe;
                mm[e] = me;
                vv[e] = ve;
            }
            reinterpret_cast<f4*>(p)[i] = pp;
            reinterpret_cast<f4*>(m)[i] = mm;
            reinterpret_cast<f4*>(v)[i] = vv;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
            float pe = p[i], me = m[i], ve = v[i];
            adamw_one(pe, g[i], me, ve, a);
            p[i] = pe;
            m[i] = me;
            v[i] = ve;
        }
    }
}

template <typename F>
void with_xt(int xt, F&& f) {
    if (xt == kF32) f(std::integral_constant<int, kF32>{});
    else if (xt == kF16) f(std::integral_constant<int, kF16>{});
    else f(std::integral_constant<int, kBF16>{});
}

template <typename F>
void with_rank(int rank, F&& f) {
    if (rank <= 4) f(std::integral_constant<int, 4>{});
    else if (rank <= 8) f(std::integral_constant<int, 8>{});
    else if (rank <= 16) f(std::integral_constant<int, 16>{});
    else if (rank <= 32) f(std::integral_constant<int, 32>{});
    else f(std::integral_constant<int, 64>{});
}

template <int FT>
hipError_t launch_rank_contract(const void* X, int xt, int64_t M, int64_t C, const float* F, int rank, float* out,
                                hipStream_t s) {
    with_rank(rank, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        constexpr int RB = contract_rows<R>();
        with_xt(xt, [&](auto xc) {
            constexpr int XT = decltype(xc)::value;
            hipLaunchKernelGGL((rank_contract_kernel<XT, R, FT>), dim3((unsigned)((M + RB - 1) / RB)), dim3(256), 0, s,
                               X, M, C, F, rank, out);
        });
    });
    return hipGetLastError();
}

template <int GT>
hipError_t launch_rank_expand(float* Y, int64_t M, int64_t C, const float* T, const float* G, int rank, float alpha,
                              hipStream_t s) {
    const int64_t gx = (C + 255) / 256, gy = min((M + 7) / 8, (int64_t)4096);
    if (gx > 0x7fffffff) return hipErrorInvalidConfiguration;
    with_rank(rank, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        hipLaunchKernelGGL((rank_expand_kernel<R, GT>), dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, Y, M, C,
                           T, G, rank, alpha);
    });
    return hipGetLastError();
}

// Row slabs of the column contraction: enough blocks (columns / 256 x slabs) to reach about 512,
// at most kMaxSlabs, each slab a whole number of kRun-row runs.  A function of (M, C) alone.
constexpr int64_t kMaxSlabs = 64;

struct Slabs {
    int64_t count, rows;
};

Slabs column_slabs(int64_t M, int64_t C) {
    const int64_t runs = (M + kRun - 1) / kRun, gx = (C + 255) / 256;
    const int64_t want = max((int64_t)1, min(kMaxSlabs, 512 / gx));
    const int64_t per = (runs + min(runs, want) - 1) / min(runs, want);   // runs per slab
    return Slabs{(runs + per - 1) / per, per * kRun};
}

template <int OT>
hipError_t launch_column_contract(const void* X, int xt, int64_t M, int64_t C, const float* T, int rank, float alpha,
                                  float* O, float* P, hipStream_t s) {
    const int64_t gx = (C + 255) / 256;
    if (gx > 0x7fffffff) return hipErrorInvalidConfiguration;
    const Slabs sl = column_slabs(M, C);
    float* part = sl.count > 1 ? P : nullptr;
    with_rank(rank, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        with_xt(xt, [&](auto xc) {
            constexpr int XT = decltype(xc)::value;
            hipLaunchKernelGGL((column_contract_kernel<XT, R, OT>), dim3((unsigned)gx, (unsigned)sl.count), dim3(256),
                               0, s, X, M, C, T, rank, alpha, sl.rows, O, part);
        });
    });
    if (part) {
        const int64_t blocks = ((int64_t)rank * C + 255) / 256;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((column_reduce_kernel<OT>), dim3((unsigned)blocks), dim3(256), 0, s, part, (int)sl.count,
                           C, rank, alpha, O);
    }
    return hipGetLastError();
}

}  // namespace

int adapter_rank_max() { return kRankMax; }

uint64_t adapter_bwd_terms_ws_bytes(int64_t M, int64_t N, int64_t K, int rank) {
    // u [M, r], then the slab partials of d_A and of d_B (one region, used one after the other)
    auto up = [](uint64_t b) { return (b + 255) / 256 * 256; };
    const Slabs a = column_slabs(M, K), b = column_slabs(M, N);
    const uint64_t pa = a.count > 1 ? (uint64_t)a.count * rank * K * 4 : 0;
    const uint64_t pb = b.count > 1 ? (uint64_t)b.count * rank * N * 4 : 0;
    return up((uint64_t)M * rank * 4) + up(max(pa, pb));
}

hipError_t launch_adapter_fwd_terms(const void* x, int x_dtype, int64_t M, int64_t N, int64_t K, const float* A,
                                    const float* B, int rank, float alpha, float* y, float* t, hipStream_t s) {
    hipError_t e = launch_rank_contract<0>(x, x_dtype, M, K, A, rank, t, s);
    if (e != hipSuccess) return e;
    return launch_rank_expand<1>(y, M, N, t, B, rank, alpha, s);
}

hipError_t launch_adapter_bwd_terms(const void* x, const void* d_out, int dtype, int64_t M, int64_t N, int64_t K,
                                    const float* A, const float* B, int rank, float alpha, const float* t,
                                    float* d_x, float* d_A, float* d_B, void* ws, hipStream_t s) {
    float* u = static_cast<float*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + ((uint64_t)M * rank * 4 + 255) / 256 * 256);
    hipError_t e = launch_rank_contract<1>(d_out, dtype, M, N, B, rank, u, s);
    if (e == hipSuccess) e = launch_rank_expand<0>(d_x, M, K, u, A, rank, alpha, s);
    if (e == hipSuccess) e = launch_column_contract<0>(x, dtype, M, K, u, rank, alpha, d_A, part, s);
    if (e == hipSuccess) e = launch_column_contract<1>(d_out, dtype, M, N, t, rank, alpha, d_B, part, s);
    return e;
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, double lr, double beta1,
                        double beta2, double eps, double weight_decay, int64_t step, hipStream_t s) {
    if (n == 0) return hipSuccess;
    AdamwArgs a;
    a.decay = (float)(1.0 - lr * weight_decay);
    a.beta1 = (float)beta1;
    a.one_m_beta1 = (float)(1.0 - beta1);
    a.beta2 = (float)beta2;
    a.one_m_beta2 = (float)(1.0 - beta2);
    a.step_size = (float)(lr / (1.0 - pow(beta1, (double)step)));
    a.inv_sqrt_bias2 = (float)(1.0 / sqrt(1.0 - pow(beta2, (double)step)));
    a.eps = (float)eps;
    const bool vec = n % 4 == 0 && ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g) |
                                     reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) & 15u) == 0;
    const int64_t units = vec ? n / 4 : n;
    const int64_t blocks = min((units + 255) / 256, (int64_t)2048);
    if (vec) hipLaunchKernelGGL((adamw_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, p, g, m, v, n, a);
    else hipLaunchKernelGGL((adamw_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, p, g, m, v, n, a);
    return hipGetLastError();
}

}  // namespace q4gsw
