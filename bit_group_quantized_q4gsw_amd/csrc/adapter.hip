// The adapter step around the frozen q4gsw base: a rank-r low-rank adapter beside the packed
// weight and the AdamW update of its factors.
//
// The input-gradient page (the Vulkan linear_q4gsw_backward pull request) says its op serves
// on-device adapter training around the frozen base, and its stack lists an on-GPU AdamW step;
// the pages give no adapter mathematics.  Reading: LoRA factors A [r, K] and B [N, r] in fp32,
//   t = x A^T [M, r],  y = x W^T + alpha t B^T,
//   u = d_out B [M, r],  d_x = d_out W + alpha u A,  d_A = alpha u^T x,  d_B = alpha d_out^T t,
// and AdamW (decoupled weight decay, bias-corrected moments).  The W terms are the library's
// forward and input gradient; this file holds the low-rank terms and the optimizer.  With
// r <= 64 they are bound by memory and latency, not arithmetic, so they run on the vector ALUs
// in fp32, laid out for many loads in flight per lane:
//
//   * row_partial_kernel: P[s, m, j] = sum over column chunk s of X[m, c] F(j, c) (t, u); the
//     chunk of F is staged in LDS, each lane sums its column quads, and a butterfly over the
//     64 lanes leaves output (row, j) in one lane;
//   * expand_kernel: T[m, j] = sum_s P[s, m, j] (chunks in order; written once as t or u), then
//     Y[m, c] += alpha sum_j T[m, j] G(j, c) (the y and d_x updates);
//   * column_partial_kernel, column_reduce_kernel: O(j, c) = alpha sum_m T[m, j] X[m, c]
//     (d_A, d_B) by row slabs, the slabs added in order;
//   * adamw_kernel: the elementwise update.
//
// F and G are A (F(j, c) = A[j C + c]) or B^T (F(j, c) = B[c r + j]).  Every output is summed in
// an order fixed by the shape alone, so results do not depend on timing.  Rounding chains (fp32):
// the row contraction adds at most 32 products per lane, 6 tree levels and C / 256 chunks; the
// expansion r products and one fma; the column contraction a quarter of a slab's rows per wave,
// 3 wave combines, at most 64 slabs and the scale.
#include "device.h"
#include "internal.h"

#include <cmath>
#include <type_traits>

namespace q4gsw {
namespace {

constexpr int kRankMax = 64;
constexpr int kExpRows = 32;          // rows per block of the expansion (8 per wave)
constexpr int kSlabRows = 32;         // rows of a slab piece in the column contraction
constexpr int64_t kMaxSlabs = 64;

// Row contraction tiling for rank bucket R: RW rows per wave (4 waves), chunks of CC columns
// (the F chunk, R x CC fp32, about 33 KB of LDS up to R = 32), NG column quads per lane.
// NARROW: 256-column chunks at every rank, for launches that the wide chunks would leave under
// 256 blocks (t = x A^T at M = 512, K = 2048, r = 16: 128 blocks and 7.7 us wide; narrow, 256
// blocks, the adapter forward is 2.3 us faster).  Launches of 256 blocks or more keep the wide
// chunks: narrowing u = d_out B at N = 8192 (512 -> 1024 blocks, twice the partials to sum) made
// the adapter backward 1.5 us slower.
template <int R, bool NARROW = false>
struct RowTile {
    static constexpr int RW = R >= 64 ? 1 : R >= 32 ? 2 : 4;
    static constexpr int ROWS = 4 * RW;
    static constexpr int CC = (NARROW || R >= 32) ? 256 : 8192 / R;
    static constexpr int NG = CC / 256;
    static constexpr int LD = CC + 4;     // LDS row stride: quads stay 16-B aligned, staging spreads banks
};

// Columns per lane of the expansion and the column contraction: CQ x R accumulators <= 64.
template <int R>
constexpr int cols_per_lane() { return R >= 64 ? 1 : R >= 32 ? 2 : 4; }

// Four consecutive elements of X (dtype XT) widened to fp32; i % 4 == 0 and the address aligned.
template <int XT>
__device__ __forceinline__ f4 load_quad(const void* X, int64_t i) {
    if constexpr (XT == kF32) {
        return *reinterpret_cast<const f4*>(static_cast<const float*>(X) + i);
    } else {
        const u2 w = *reinterpret_cast<const u2*>(static_cast<const uint16_t*>(X) + i);
        f4 r;
        if constexpr (XT == kF16) {
            r[0] = f16_bits_to_f32((uint16_t)(w[0] & 0xffffu));
            r[1] = f16_bits_to_f32((uint16_t)(w[0] >> 16));
            r[2] = f16_bits_to_f32((uint16_t)(w[1] & 0xffffu));
            r[3] = f16_bits_to_f32((uint16_t)(w[1] >> 16));
        } else {
            r[0] = bitcast<float>(w[0] << 16);
            r[1] = bitcast<float>(w[0] & 0xffff0000u);
            r[2] = bitcast<float>(w[1] << 16);
            r[3] = bitcast<float>(w[1] & 0xffff0000u);
        }
        return r;
    }
}

// X[row_base + c .. + 4) with zeros past C or when !row_ok; VEC: rows hold whole aligned quads
// (C % 4 == 0).  Every load is issued unconditionally (from element 0 when out of range) and
// the zeros are selected afterwards, so no branch forces a wait between a lane's loads.
template <int XT, bool VEC>
__device__ __forceinline__ f4 load_quad_sel(const void* X, int64_t row_base, int64_t c, int64_t C, bool row_ok) {
    if constexpr (VEC) {
        const bool ok = row_ok && c < C;
        const f4 v = load_quad<XT>(X, ok ? row_base + c : 0);
        return ok ? v : f4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
        f4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = row_ok && c + q < C;
            const float e = load_elem<XT>(X, ok ? row_base + c + q : 0);
            r[q] = ok ? e : 0.0f;
        }
        return r;
    }
}


// Sum over the 64 lanes of each of the N values v[i] (N a power of two, <= 64); lane l returns
// the total of value l % N.  Offsets 32 .. N add whole vectors; below N each level keeps the
// half of the values named by the lane's bit and adds the partner's copy of that half.
template <int N>
__device__ __forceinline__ float lanes_spread(const float* v, int lane) {
    if constexpr (N == 1) {
        return v[0];
    } else {
        constexpr int H = N / 2;
        const bool hi = (lane & H) != 0;
        float w[H];
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float keep = hi ? v[H + i] : v[i];
            const float send = hi ? v[i] : v[H + i];
            w[i] = keep + __shfl_xor(send, H);
        }
        return lanes_spread<H>(w, lane);
    }
}

template <int N>
__device__ __forceinline__ float wave_sum_spread(float (&v)[N], int lane) {
#pragma unroll
    for (int off = 32; off >= N; off >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] += __shfl_xor(v[i], off);
    return lanes_spread<N>(v, lane);
}

// P[s, m, j] = sum_{c in chunk s} X[m, c] F(j, c) for X [M, C] (dtype XT); FT = 0: F(j, c) =
// A[j C + c], FT = 1: F(j, c) = B[c r + j].  Block b: rows (b / chunks) ROWS .. (wave w: RW of
// them), chunk b % chunks (lane l: column quads 4 l + 256 g).
template <int XT, int R, int FT, bool VEC, bool NARROW>
__global__ __launch_bounds__(256) void row_partial_kernel(const void* __restrict__ X, int64_t M, int64_t C,
                                                          const float* __restrict__ F, int rank, int64_t chunks,
                                                          float* __restrict__ P) {
    using T = RowTile<R, NARROW>;
    __shared__ __align__(16) float Fl[R * T::LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rb = blockIdx.x / chunks, s = blockIdx.x % chunks;
    const int64_t c0 = s * T::CC;
    const int64_t m0 = rb * T::ROWS + wave * T::RW;
    // every load is issued before the first wait: this lane's X quads, then its share of F
    f4 xv[T::NG][T::RW];
#pragma unroll
    for (int g = 0; g < T::NG; ++g)
#pragma unroll
        for (int r = 0; r < T::RW; ++r)
            xv[g][r] = load_quad_sel<XT, VEC>(X, (m0 + r) * C, c0 + 256 * g + 4 * lane, C, m0 + r < M);
    constexpr int PER = R * T::CC / 256;
    float fv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid + 256 * k;
        const int j = FT == 0 ? i / T::CC : i % R;
        const int64_t c = c0 + (FT == 0 ? i % T::CC : i / R);
        fv[k] = load_sel(F, FT == 0 ? (int64_t)j * C + c : c * rank + j, j < rank && c < C);
    }
    __builtin_amdgcn_sched_barrier(0);      // keep every load above ahead of the first wait
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = tid + 256 * k;
        const int j = FT == 0 ? i / T::CC : i % R;
        const int cc = FT == 0 ? i % T::CC : i / R;
        Fl[j * T::LD + cc] = fv[k];
    }
    __syncthreads();
    float acc[T::RW * R];
#pragma unroll
    for (int i = 0; i < T::RW * R; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int g = 0; g < T::NG; ++g) {
        const int cc = 256 * g + 4 * lane;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const f4 f = *reinterpret_cast<const f4*>(&Fl[j * T::LD + cc]);
#pragma unroll
            for (int r = 0; r < T::RW; ++r) {
                float a = acc[r * R + j];
                a = fmaf(xv[g][r][0], f[0], a);
                a = fmaf(xv[g][r][1], f[1], a);
                a = fmaf(xv[g][r][2], f[2], a);
                a = fmaf(xv[g][r][3], f[3], a);
                acc[r * R + j] = a;
            }
        }
    }
    const float mine = wave_sum_spread<T::RW * R>(acc, lane);
    const int r = lane / R, j = lane % R;
    const int64_t m = m0 + r;
    if (lane < T::RW * R && j < rank && m < M) P[(s * M + m) * rank + j] = mine;
}


// T[m, j] = sum_s P[s, m, j] (s ascending; written to Tout by the blocks of column block 0),
// then Y [M, C] (fp32) += alpha T G with G(j, c) = A[j C + c] (GT = 0) or B[c r + j] (GT = 1).
// Block: 64 CQ columns (lane l: columns CQ l ..) x 32 rows (wave w: rows 8w .. 8w + 7), over row
// blocks blockIdx.y, blockIdx.y + gridDim.y, ...  Every global load of a row block (its rows of
// Y, the chunk partials of its rows of T and, for B, the block's chunk of B, which is contiguous)
// is issued before the first wait; B then goes to LDS j-major, A is read by the lanes directly.
// VEC: rows of Y (and of A) hold whole aligned groups of CQ values.
template <int R, int GT, bool VEC>
__global__ __launch_bounds__(256) void expand_kernel(float* __restrict__ Y, int64_t M, int64_t C,
                                                     const float* __restrict__ P, int64_t chunks,
                                                     const float* __restrict__ G, int rank, float alpha,
                                                     float* __restrict__ Tout) {
    constexpr int CQ = cols_per_lane<R>();
    constexpr int SPAN = 64 * CQ;                  // columns per block
    constexpr int LDG = SPAN + 4;
    constexpr int kG = GT == 1 ? R * LDG : 0;
    constexpr int RPW = kExpRows / 4;              // rows per wave
    constexpr int TPT = (kExpRows * R + 255) / 256;  // values of T per thread
    __shared__ __align__(16) float smem[kExpRows * R + kG];
    float* Tl = smem;
    float* Gl = smem + kExpRows * R;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t cb = (int64_t)blockIdx.x * SPAN;
    const int64_t c = cb + (int64_t)lane * CQ;
    const bool live = c < C;
    const int64_t nrb = (M + kExpRows - 1) / kExpRows;
    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        const int64_t m0 = rb * kExpRows;
        // ---- issue: rows of Y, the factor, the chunk partials of T
        float yv[RPW][CQ];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t m = m0 + RPW * wave + i;
            const bool ok = live && m < M;
            const float* yp = Y + (ok ? m * C + c : 0);      // element 0 stands in for rows past M
            if constexpr (VEC && CQ == 4) {
                const f4 v = *reinterpret_cast<const f4*>(yp);
#pragma unroll
                for (int q = 0; q < 4; ++q) yv[i][q] = v[q];
            } else if constexpr (VEC && CQ == 2) {
                const float2 v = *reinterpret_cast<const float2*>(yp);
                yv[i][0] = v.x;
                yv[i][1] = v.y;
            } else {
#pragma unroll
                for (int q = 0; q < CQ; ++q) yv[i][q] = load_sel(Y, m * C + c + q, ok && c + q < C);
            }
        }
        float g[CQ][R];
        constexpr int PER = GT == 1 ? SPAN * R / 256 : 1;
        float gv[PER];
        const int64_t avail = min((int64_t)SPAN, C - cb) * rank;   // B[cb r ..) holds the block's columns
        if constexpr (GT == 1) {
#pragma unroll
            for (int k = 0; k < PER; ++k) gv[k] = load_sel(G, cb * rank + tid + 256 * k, tid + 256 * k < avail);
        } else {
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const bool okj = j < rank && live;
                if constexpr (VEC && CQ == 4) {
                    const f4 v = *reinterpret_cast<const f4*>(G + (okj ? (int64_t)j * C + c : 0));
#pragma unroll
                    for (int q = 0; q < 4; ++q) g[q][j] = okj ? v[q] : 0.0f;
                } else {
#pragma unroll
                    for (int q = 0; q < CQ; ++q) g[q][j] = load_sel(G, (int64_t)j * C + c + q, okj && c + q < C);
                }
            }
        }
        float tv[TPT];
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + 256 * k, r = i / R, j = i % R;
            const int64_t m = m0 + r;
            tv[k] = (i < kExpRows * R && m < M && j < rank) ? chunk_sum<8>(P, chunks, M * rank, m * rank + j) : 0.0f;
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- stage: T (and B) into LDS
        __syncthreads();                                   // the previous row block's readers are done
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + 256 * k, r = i / R, j = i % R;
            if (i < kExpRows * R) {
                Tl[i] = tv[k];
                if (Tout && blockIdx.x == 0 && m0 + r < M && j < rank) Tout[(m0 + r) * rank + j] = tv[k];
            }
        }
        if constexpr (GT == 1) {
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int i = tid + 256 * k;
                if (i < avail) {
                    const int cc = i / rank, j = i - cc * rank;
                    Gl[j * LDG + cc] = gv[k];
                }
            }
            for (int i = tid; i < R * LDG; i += 256) {   // the rank bucket's padding and columns past C
                if (i / LDG >= rank || i % LDG >= SPAN || cb + i % LDG >= C) Gl[i] = 0.0f;
            }
        }
        __syncthreads();
        if (!live) continue;
        if constexpr (GT == 1) {
#pragma unroll
            for (int q = 0; q < CQ; ++q)
#pragma unroll
                for (int j = 0; j < R; ++j) g[q][j] = Gl[j * LDG + lane * CQ + q];
        }
        // ---- the rows
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rr = RPW * wave + i;
            const int64_t m = m0 + rr;
            if (m >= M) break;
#pragma unroll
            for (int q = 0; q < CQ; ++q) {
                float sum = 0.0f;
#pragma unroll
                for (int j = 0; j < R; ++j) sum = fmaf(Tl[rr * R + j], g[q][j], sum);
                yv[i][q] = fmaf(alpha, sum, yv[i][q]);
            }
            float* yp = Y + m * C + c;
            if constexpr (VEC && CQ == 4) {
                *reinterpret_cast<f4*>(yp) = f4{yv[i][0], yv[i][1], yv[i][2], yv[i][3]};
            } else if constexpr (VEC && CQ == 2) {
                *reinterpret_cast<float2*>(yp) = make_float2(yv[i][0], yv[i][1]);
            } else {
#pragma unroll
                for (int q = 0; q < CQ; ++q)
                    if (c + q < C) yp[q] = yv[i][q];
            }
        }
    }
}

// One output of the column contraction: O(j, c) = alpha sum_m T[m, j] X[m, c] for X [M, C],
// T [M, r] fp32, cut into gx column blocks x `slabs` row slabs of `slab` rows; ot = 0: O[j C + c]
// ([r, C], d_A), ot = 1: O[c r + j] ([C, r], d_B); Pc [slabs, r, C] holds unscaled slab sums when
// slabs > 1.
struct ColSeg {
    const void* X;
    const float* T;
    float* O;
    float* Pc;
    int64_t C, gx, slabs, slab;
    int ot;
};

// Slab sums of both column contractions of the backward in one launch: blocks [0, a.gx a.slabs)
// take a (d_A), the rest b (d_B).  Block: 64 CQ columns (lane l: columns CQ l ..) x one slab,
// taken in pieces of 32 rows staged in LDS; wave w adds rows w, w + 4, ... of each piece in
// order, then the four waves' sums are added in wave order.  One slab: O is written with alpha
// applied; several: the unscaled slab sums go to Pc.
template <int XT, int R, bool VEC>
__global__ __launch_bounds__(256) void column_partial_kernel(ColSeg a, ColSeg b, int64_t M, int rank, float alpha) {
    constexpr int CQ = cols_per_lane<R>();
    constexpr int kT = kSlabRows * R;
    // one LDS array: the T piece [32][R], then the wave-combine buffer [CQ R][64]
    __shared__ __align__(16) float smem[kT + CQ * R * 64];
    float* Ts = smem;
    float* red = smem + kT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t na = a.gx * a.slabs;
    const bool second = (int64_t)blockIdx.x >= na;
    const ColSeg sg = second ? b : a;
    const int64_t bi = second ? (int64_t)blockIdx.x - na : (int64_t)blockIdx.x;
    const int64_t bx = bi % sg.gx, by = bi / sg.gx;
    const int64_t C = sg.C;
    const void* X = sg.X;
    const float* T = sg.T;
    const int64_t c = (bx * 64 + lane) * CQ;
    const int64_t lo = by * sg.slab, hi = min(M, lo + sg.slab);
    float acc[CQ][R];
#pragma unroll
    for (int q = 0; q < CQ; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[q][j] = 0.0f;
    for (int64_t p0 = lo; p0 < hi; p0 += kSlabRows) {
        const int rows = (int)min((int64_t)kSlabRows, hi - p0);
        // this wave's 8 rows of the piece (rows wave + 4 i), loaded before the T piece is waited for
        constexpr int RPW = kSlabRows / 4;
        float xv[RPW][CQ];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = wave + 4 * i;
            const int64_t rbase = (p0 + r) * C;
            if constexpr (CQ == 4) {
                const f4 v = load_quad_sel<XT, VEC>(X, rbase, c, C, r < rows);
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[i][q] = v[q];
            } else {
#pragma unroll
                for (int q = 0; q < CQ; ++q) {
                    const bool ok = r < rows && c + q < C;
                    const float e = load_elem<XT>(X, ok ? rbase + c + q : 0);
                    xv[i][q] = ok ? e : 0.0f;
                }
            }
        }
        // the T piece goes into registers in the same round trip as the X rows; the barrier then
        // frees Ts of the previous piece before it is overwritten
        constexpr int TPT = (kT + 255) / 256;
        float tv_pre[TPT];
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + 256 * k, r = i / R, j = i % R;
            tv_pre[k] = load_sel(T, (p0 + r) * rank + j, i < kT && p0 + r < hi && j < rank);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TPT; ++k)
            if (tid + 256 * k < kT) Ts[tid + 256 * k] = tv_pre[k];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = wave + 4 * i;
            if (r >= rows) break;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float tv = Ts[r * R + j];
#pragma unroll
                for (int q = 0; q < CQ; ++q) acc[q][j] = fmaf(tv, xv[i][q], acc[q][j]);
            }
        }
    }
    // the four waves' sums, in wave order
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        __syncthreads();
        if (wave == w) {
#pragma unroll
            for (int q = 0; q < CQ; ++q)
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    float& d = red[(q * R + j) * 64 + lane];
                    d = w == 0 ? acc[q][j] : d + acc[q][j];
                }
        }
    }
    __syncthreads();
    // thread i takes column (i % (64 CQ)) of the block and rank i / (64 CQ): consecutive threads
    // store consecutive columns of the slab sums (d_A's rows likewise)
    for (int i = tid; i < CQ * R * 64; i += 256) {
        const int cl = i % (64 * CQ), j = i / (64 * CQ), l = cl / CQ, q = cl % CQ;
        const int64_t cc = (bx * 64 + l) * CQ + q;
        if (j >= rank || cc >= C) continue;
        const float v = red[(q * R + j) * 64 + l];
        if (sg.slabs > 1) sg.Pc[(by * rank + j) * C + cc] = v;
        else if (sg.ot == 0) sg.O[(int64_t)j * C + cc] = alpha * v;
        else sg.O[cc * rank + j] = alpha * v;
    }
}

// O(j, c) = alpha * (Pc[0, j, c] + Pc[1, j, c] + ...) in slab order for the outputs of a and b
// that have several slabs; one thread per (j, c), a's first.
__global__ __launch_bounds__(256) void column_reduce_kernel(ColSeg a, ColSeg b, int rank, float alpha) {
    const int64_t ea = a.slabs > 1 ? (int64_t)rank * a.C : 0, eb = b.slabs > 1 ? (int64_t)rank * b.C : 0;
    int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= ea + eb) return;
    const bool second = e >= ea;
    const ColSeg sg = second ? b : a;
    if (second) e -= ea;
    const float s = chunk_sum<16>(sg.Pc, sg.slabs, (int64_t)rank * sg.C, e);
    const int64_t j = e / sg.C, c = e % sg.C;
    if (sg.ot == 0) sg.O[e] = alpha * s;
    else sg.O[c * rank + j] = alpha * s;
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

template <typename F>
void with_bool(bool b, F&& f) {
    if (b) f(std::true_type{});
    else f(std::false_type{});
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int es_of(int xt) { return xt == kF32 ? 4 : 2; }

// rows of X (element size es) hold whole quads that start aligned
bool quads_ok(const void* X, int64_t C, int es) { return C % 4 == 0 && aligned(X, 4 * (uintptr_t)es); }

// the narrow chunks when the wide ones leave the row contraction under 256 blocks
bool row_narrow(int64_t M, int64_t C, int rank) {
    int64_t rows = 0, cc = 0;
    with_rank(rank, [&](auto rc) {
        rows = RowTile<decltype(rc)::value>::ROWS;
        cc = RowTile<decltype(rc)::value>::CC;
    });
    return cc > 256 && (M + rows - 1) / rows * ((C + cc - 1) / cc) < 256;
}

int64_t row_chunks(int64_t M, int64_t C, int rank) {
    int64_t cc = 0;
    with_rank(rank, [&](auto rc) { cc = RowTile<decltype(rc)::value>::CC; });
    if (row_narrow(M, C, rank)) cc = 256;
    return (C + cc - 1) / cc;
}

int64_t row_blocks(int64_t M, int64_t C, int rank) {
    int64_t rows = 0;
    with_rank(rank, [&](auto rc) { rows = RowTile<decltype(rc)::value>::ROWS; });
    return (M + rows - 1) / rows * row_chunks(M, C, rank);
}

int64_t lane_cols(int rank) {
    int64_t cq = 0;
    with_rank(rank, [&](auto rc) { cq = cols_per_lane<decltype(rc)::value>(); });
    return cq;
}

// Row slabs of the column contraction: about 512 blocks (column blocks x slabs), at most
// kMaxSlabs, each a whole number of 32-row pieces.  A function of (M, C, rank) alone.
struct Slabs {
    int64_t count, rows;
};

Slabs column_slabs(int64_t M, int64_t C, int rank) {
    const int64_t span = 64 * lane_cols(rank);
    const int64_t pieces = (M + kSlabRows - 1) / kSlabRows, gx = (C + span - 1) / span;
    const int64_t want = min(pieces, max((int64_t)1, min(kMaxSlabs, 512 / gx)));
    const int64_t per = (pieces + want - 1) / want;
    return Slabs{(pieces + per - 1) / per, per * kSlabRows};
}

uint64_t up256(uint64_t b) { return (b + 255) / 256 * 256; }

uint64_t row_partial_bytes(int64_t M, int64_t C, int rank) {
    return up256((uint64_t)row_chunks(M, C, rank) * M * rank * 4);
}

uint64_t column_partial_bytes(int64_t M, int64_t C, int rank) {
    const Slabs sl = column_slabs(M, C, rank);
    return sl.count > 1 ? up256((uint64_t)sl.count * rank * C * 4) : 0;
}

template <int FT>
hipError_t launch_row_partial(const void* X, int xt, int64_t M, int64_t C, const float* F, int rank, float* P,
                              hipStream_t s) {
    const int64_t chunks = row_chunks(M, C, rank), blocks = row_blocks(M, C, rank);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    with_rank(rank, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        with_xt(xt, [&](auto xc) {
            constexpr int XT = decltype(xc)::value;
            with_bool(quads_ok(X, C, es_of(XT)), [&](auto vc) {
                with_bool(row_narrow(M, C, rank), [&](auto nc) {
                    hipLaunchKernelGGL((row_partial_kernel<XT, R, FT, decltype(vc)::value, decltype(nc)::value>),
                                       dim3((unsigned)blocks), dim3(256), 0, s, X, M, C, F, rank, chunks, P);
                });
            });
        });
    });
    return hipGetLastError();
}

template <int GT>
hipError_t launch_expand(float* Y, int64_t M, int64_t C, const float* P, int64_t chunks, const float* G, int rank,
                         float alpha, float* Tout, hipStream_t s) {
    const int64_t cq = lane_cols(rank);
    const int64_t gx = (C + 64 * cq - 1) / (64 * cq), gy = min((M + kExpRows - 1) / kExpRows, (int64_t)8192);
    if (gx > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = C % cq == 0 && aligned(Y, 4 * (uintptr_t)cq) && (GT == 1 || aligned(G, 4 * (uintptr_t)cq));
    with_rank(rank, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        with_bool(vec, [&](auto vc) {
            hipLaunchKernelGGL((expand_kernel<R, GT, decltype(vc)::value>), dim3((unsigned)gx, (unsigned)gy),
                               dim3(256), 0, s, Y, M, C, P, chunks, G, rank, alpha, Tout);
        });
    });
    return hipGetLastError();
}

ColSeg column_seg(const void* X, int64_t M, int64_t C, const float* T, int rank, float* O, float* Pc, int ot) {
    const Slabs sl = column_slabs(M, C, rank);
    const int64_t cq = lane_cols(rank);
    return ColSeg{X, T, O, Pc, C, (C + 64 * cq - 1) / (64 * cq), sl.count, sl.rows, ot};
}

// d_A (a) and d_B (b) in one launch of column_partial_kernel and, for the outputs with several
// slabs, one of column_reduce_kernel.
hipError_t launch_columns(const ColSeg& a, const ColSeg& b, int xt, int64_t M, int rank, float alpha, bool vec,
                          hipStream_t s) {
    const int64_t blocks = a.gx * a.slabs + b.gx * b.slabs;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    with_rank(rank, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        with_xt(xt, [&](auto xc) {
            constexpr int XT = decltype(xc)::value;
            with_bool(vec, [&](auto vc) {
                hipLaunchKernelGGL((column_partial_kernel<XT, R, decltype(vc)::value>), dim3((unsigned)blocks),
                                   dim3(256), 0, s, a, b, M, rank, alpha);
            });
        });
    });
    const int64_t elems = (a.slabs > 1 ? (int64_t)rank * a.C : 0) + (b.slabs > 1 ? (int64_t)rank * b.C : 0);
    if (elems > 0) {
        const int64_t rblocks = (elems + 255) / 256;
        if (rblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(column_reduce_kernel, dim3((unsigned)rblocks), dim3(256), 0, s, a, b, rank, alpha);
    }
    return hipGetLastError();
}

// Backward workspace: the chunk sums of u, u [M, r], then the slab sums of d_A and of d_B.
struct BwdWs {
    float *P, *u, *PcA, *PcB;
    uint64_t bytes;
};

BwdWs bwd_ws(void* ws, int64_t M, int64_t N, int64_t K, int rank) {
    uint8_t* w = static_cast<uint8_t*>(ws);
    const uint64_t pb = row_partial_bytes(M, N, rank), ub = up256((uint64_t)M * rank * 4);
    const uint64_t ab = column_partial_bytes(M, K, rank), bb = column_partial_bytes(M, N, rank);
    return BwdWs{reinterpret_cast<float*>(w), reinterpret_cast<float*>(w + pb), reinterpret_cast<float*>(w + pb + ub),
                 reinterpret_cast<float*>(w + pb + ub + ab), pb + ub + ab + bb};
}

}  // namespace

int adapter_rank_max() { return kRankMax; }

bool adapter_shape_ok(int64_t M, int64_t N, int64_t K, int rank) {
    const int64_t lim = 0x7fffffff;
    if (row_blocks(M, K, rank) > lim || row_blocks(M, N, rank) > lim) return false;
    if (((int64_t)rank * N + 255) / 256 > lim || ((int64_t)rank * K + 255) / 256 > lim) return false;
    return (N + 63) / 64 <= lim && (K + 63) / 64 <= lim;
}

uint64_t adapter_fwd_terms_ws_bytes(int64_t M, int64_t N, int64_t K, int rank) {
    (void)N;
    return row_partial_bytes(M, K, rank);     // the chunk sums of t
}

uint64_t adapter_bwd_terms_ws_bytes(int64_t M, int64_t N, int64_t K, int rank) {
    return bwd_ws(nullptr, M, N, K, rank).bytes;
}

hipError_t launch_adapter_fwd_t(const void* x, int x_dtype, int64_t M, int64_t K, const float* A, int rank, void* ws,
                                hipStream_t s) {
    return launch_row_partial<0>(x, x_dtype, M, K, A, rank, static_cast<float*>(ws), s);
}

LowRankEpi adapter_fwd_epi(int64_t M, int64_t K, const float* B, int rank, float alpha, float* t, void* ws) {
    return LowRankEpi{static_cast<const float*>(ws), row_chunks(M, K, rank), B, t, alpha, rank, 1};
}

hipError_t launch_adapter_fwd_expand(float* y, int64_t M, int64_t N, int64_t K, const float* B, int rank, float alpha,
                                     float* t, void* ws, hipStream_t s) {
    return launch_expand<1>(y, M, N, static_cast<const float*>(ws), row_chunks(M, K, rank), B, rank, alpha, t, s);
}

hipError_t launch_adapter_bwd_u(const void* d_out, int dtype, int64_t M, int64_t N, int64_t K, const float* B,
                                int rank, void* ws, hipStream_t s) {
    return launch_row_partial<1>(d_out, dtype, M, N, B, rank, bwd_ws(ws, M, N, K, rank).P, s);
}

LowRankEpi adapter_bwd_epi(int64_t M, int64_t N, int64_t K, const float* A, int rank, float alpha, void* ws) {
    const BwdWs w = bwd_ws(ws, M, N, K, rank);
    return LowRankEpi{w.P, row_chunks(M, N, rank), A, w.u, alpha, rank, 0};
}

hipError_t launch_adapter_bwd_rest(const void* x, const void* d_out, int dtype, int64_t M, int64_t N, int64_t K,
                                   const float* A, int rank, float alpha, const float* t, float* d_x, bool dx_done,
                                   float* d_A, float* d_B, void* ws, hipStream_t s) {
    const BwdWs w = bwd_ws(ws, M, N, K, rank);
    hipError_t e = hipSuccess;
    if (!dx_done) e = launch_expand<0>(d_x, M, K, w.P, row_chunks(M, N, rank), A, rank, alpha, w.u, s);
    if (e != hipSuccess) return e;
    const int es = es_of(dtype);
    const ColSeg a = column_seg(x, M, K, w.u, rank, d_A, w.PcA, 0);
    const ColSeg b = column_seg(d_out, M, N, t, rank, d_B, w.PcB, 1);
    return launch_columns(a, b, dtype, M, rank, alpha, quads_ok(x, K, es) && quads_ok(d_out, N, es), s);
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
