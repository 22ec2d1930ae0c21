// Internal interface between the C-ABI front end (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace q4gsw {

// Device view of one packed weight.
struct WView {
    const uint8_t* nib;      // nibble plane
    const void* scales;      // scale plane, indexed by scale_index(g_pad, n, g)
    int scale_f16;           // 1: fp16 scales, 0: fp32
    int64_t N, K, gs, n_pad, k_pad, g_pad;
};

// embedding.hip: out [T, K] fp32, row t = row ids[t] of dequant(W) (zeros for ids outside [0, N)).
// embedding_blocks is the launch's block count (it must stay below 2^31).
uint64_t embedding_blocks(int64_t T, int64_t K);
hipError_t launch_embedding(const WView& w, const int64_t* ids, int64_t T, float* out, hipStream_t s);

// pack.hip
hipError_t launch_pack(const uint8_t* codes, const void* scales, int scale_f16, int64_t N, int64_t K,
                       int64_t gs, const Layout& L, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack(const WView& w, uint8_t* codes, void* scales, hipStream_t s);

// gemv.hip: M <= 8 routes.  `out` is y [M, N] when splits == 1, else ws [splits][M][n_pad].
hipError_t launch_gemv_fwd(const WView& w, const void* x, int x_dtype, int64_t M, float* out,
                           int splits, hipStream_t s);
int gemv_fwd_splits(const WView& w, int64_t M);
// The one-row decode path (M = 1, fp16 or bf16 x 16-byte aligned, K = k_pad = 512 U with U in
// 1..4, 8 or 16, no K split), and one launch of it over up to three weights sharing K, group size
// and scale dtype.
bool gemv_row_eligible(const WView& w, const void* x, int x_dtype, int64_t M);
hipError_t launch_gemv_fwd_row(const WView* w, float* const* out, int nseg, const void* x, int x_dtype,
                               hipStream_t s);
// One launch of the small-M GEMV over up to three weights sharing K, group size and scale dtype,
// none of which splits K (the row-octet decode path when it is eligible): out[i] is y_i [M, N_i].
hipError_t launch_gemv_fwd_multi(const WView* w, float* const* out, int nseg, const void* x, int x_dtype,
                                 int64_t M, hipStream_t s);
// `out` is d_x [M, K] when splits == 1, else ws [splits][M][k_pad].
hipError_t launch_gemv_bwd(const WView& w, const void* d_out, int g_dtype, int64_t M, float* out,
                           int splits, hipStream_t s);
int gemv_bwd_splits(const WView& w, int64_t M);
// y[m][c] = sum_s ws[s][m][c] for c < cols (ws row pitch ld, a multiple of 4; ws 16-byte aligned).
hipError_t launch_reduce_splits(const float* ws, int splits, int64_t M, int64_t cols, int64_t ld,
                                float* y, int64_t y_ld, hipStream_t s);
// The same over up to three column segments in one launch: y[i][m][c] = sum_s ws[s][m][off[i] + c]
// for c < cols[i] (off[i] multiples of 4).
hipError_t launch_reduce_segments(const float* ws, int splits, int64_t M, int64_t ld, const float* const* y,
                                  const int64_t* y_ld, const int64_t* off, const int64_t* cols, int nseg,
                                  hipStream_t s);

// Split partials of the 32x32 MFMA GEMMs, fragment layout: plane s (of (M rounded up to 32) x
// width floats, width a multiple of 32) holds the 32x32 output tiles (tm, tn) in order
// tm * (width / 32) + tn, 4 KB each; inside a tile, lane L's accumulators r = 4 r4 + q (rows
// 8 r4 + 4 (L / 32) + q, tile column L % 32, octet-permuted when perm is set) sit at float
// 4 (64 r4 + L) + q, so a wave stores a tile with four 16-byte-per-lane writes.  The reduction
// writes y[i][m][c] = sum_s for the tile columns of segment i (off[i] multiples of 32).
inline int64_t frag_plane_floats(int64_t M, int64_t width) { return (M + 31) / 32 * 32 * width; }
// Optional low-rank term of a one-segment reduction (the adapter's forward and input gradient):
// y[m, c] = (sum of the splits) then += alpha sum_j T[m, j] G(j, c), with T[m, j] = sum_s
// P[(s M + m) r + j] over `chunks` partials in order (written to Tout once when Tout is set) and
// G(j, c) = G[j C + c] (gt 0) or G[c r + j] (gt 1), C the segment's columns; the same fp32
// operations, in the same order, as the separate expansion kernel, so the results match it bit
// for bit.
struct LowRankEpi {
    const float* P;
    int64_t chunks;
    const float* G;
    float* Tout;
    float alpha;
    int rank;
    int gt;
};
hipError_t launch_reduce_frags(const float* ws, int splits, int64_t M, int64_t width, const float* const* y,
                               const int64_t* y_ld, const int64_t* off, const int64_t* cols, int nseg, int perm,
                               hipStream_t s, const LowRankEpi* lr = nullptr);

// generic.hip: any shape, any group size.
hipError_t launch_generic_fwd(const WView& w, const void* x, int x_dtype, int64_t M, float* y,
                              hipStream_t s);
hipError_t launch_generic_bwd(const WView& w, const void* d_out, int g_dtype, int64_t M, float* d_x,
                              hipStream_t s);

// gemm_fwd.hip: MFMA forward over up to three weights sharing K (fused QKV uses three).
enum GemmMode : int { kModeFold = 0, kModeGroup = 1, kModeSplit = 2, kModeBSplit = 3 };
struct FwdSeg {
    WView w;
    float* out;              // [M, N] final output of this segment
};
struct FwdPlan {
    int mode;
    int mi;                  // 32-row MFMA tiles per wave: 4 (128-row blocks) or 2 (64-row blocks)
    int splits;              // K splits (1: write outputs directly)
    int64_t ws_bytes;        // workspace needed
};
// force_rows (64 or 128) and force_splits (> 0) pin the block rows and the K splits of this plan;
// 0 leaves each to the shape.
FwdPlan plan_gemm_fwd(const FwdSeg* segs, int nseg, int x_dtype, int fold_ok, int64_t M, int force_rows = 0,
                      int force_splits = 0);
// Contraction splits for an MFMA GEMM of `blocks` output blocks, `slots` of which run at once,
// n_chunks contraction chunks of ~chunk_us each (plus `fill` chunks of pipeline fill and
// epilogue per block) and an M x width fp32 output; the modelled time (microseconds) goes to
// *cost when cost is not null; force_splits > 0 pins the split count (clamped to the chunks and
// rounded to one without empty splits).
int pick_gemm_splits(int64_t blocks, int64_t n_chunks, int64_t M, int64_t width, int64_t slots = 256,
                     double chunk_us = 2.0, double* cost = nullptr, int force_splits = 0, double fill = 2.0);
bool gemm_fwd_supported(const WView& w, int x_dtype, int fold_ok);
// lr (one segment only): the low-rank term of LowRankEpi, added in the split reduction (the same
// operations in the same order as the separate expansion) or, with one split, by the exact-code
// group instances with 128-column chunks and fp16 scales in their epilogue (fp32 MFMAs into the
// accumulators); *lr_done tells whether this launch applied it.
hipError_t launch_gemm_fwd(const FwdSeg* segs, int nseg, const void* x, int x_dtype, int64_t M,
                           const FwdPlan& plan, float* ws, hipStream_t s, const LowRankEpi* lr = nullptr,
                           bool* lr_done = nullptr);

// MFMA input gradient: gemm_bwd2.hip (32x32x16) dispatches, gemm_bwd.hip (16x16x32) covers
// the group sizes the former does not take.
struct BwdPlan {
    int mode;                // kModeFold, kModeSplit or kModeBSplit
    int splits;              // N (contraction) splits
    int64_t ws_bytes;
    int v1;                  // 1: the 16x16x32 kernel serves this call
};
bool gemm_bwd_supported(const WView& w, int g_dtype, int fold_ok);
// force_splits > 0 pins the contraction splits of the 32x32 routes (0: chosen per shape).
BwdPlan plan_gemm_bwd(const WView& w, int g_dtype, int fold_ok, int64_t M, int force_splits = 0);
// lr (the adapter's low-rank term) is applied by the split reduction: only with !plan.v1 and
// plan.splits > 1 (the caller checks).
hipError_t launch_gemm_bwd(const WView& w, const void* d_out, int g_dtype, int64_t M, float* d_x,
                           const BwdPlan& plan, float* ws, hipStream_t s, const LowRankEpi* lr = nullptr);
bool gemm_bwd_v1_supported(const WView& w, int g_dtype, int fold_ok);
BwdPlan plan_gemm_bwd_v1(const WView& w, int g_dtype, int fold_ok, int64_t M);
hipError_t launch_gemm_bwd_v1(const WView& w, const void* d_out, int g_dtype, int64_t M, float* d_x,
                              const BwdPlan& plan, float* ws, hipStream_t s);

// dq8ca.hip: the linear on per-row int8 activations (gs % 64 == 0 or gs == 32).  The workspace
// holds the GEMM-layout codes [M][k_pad], the row scales and -zero points, then the split partials.
struct Dq8caPlan {
    int splits;
    int64_t ws_bytes;
};
bool dq8ca_supported(const WView& w);
Dq8caPlan plan_dq8ca(const WView& w, int64_t M, int force_splits = 0);
hipError_t launch_dq8ca_quantize(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* scale,
                                 int32_t* zp, hipStream_t s);
hipError_t launch_dq8ca(const WView& w, const void* x, int x_dtype, int64_t M, float* y, const Dq8caPlan& plan,
                        void* ws, hipStream_t s);

// adapter.hip: the low-rank adapter terms beside the frozen weight (rank 1..adapter_rank_max())
// and the AdamW update.  The forward writes t = x A^T [M, r], then y += alpha t B^T; its
// workspace (the column-chunk sums of t) is adapter_fwd_terms_ws_bytes.  The backward, in order:
// launch_adapter_bwd_u (the chunk sums of u = d_out B, before the input gradient), the input
// gradient, which takes adapter_bwd_epi (d_x += alpha u A, u written) into its split reduction
// when it has one, then launch_adapter_bwd_rest (d_x += alpha u A unless done, d_A = alpha u^T x,
// d_B = alpha d_out^T t).  Its workspace (chunk sums of u, u, slab sums of d_A and d_B) is
// adapter_bwd_terms_ws_bytes.  adapter_shape_ok: every launch of both fits the grid limits.
int adapter_rank_max();
bool adapter_shape_ok(int64_t M, int64_t N, int64_t K, int rank);
uint64_t adapter_fwd_terms_ws_bytes(int64_t M, int64_t N, int64_t K, int rank);
uint64_t adapter_bwd_terms_ws_bytes(int64_t M, int64_t N, int64_t K, int rank);
// Forward: launch_adapter_fwd_t (the column-chunk partials of t = x A^T, before the GEMM), the
// GEMM, which takes adapter_fwd_epi (y += alpha t B^T, t written) when it runs on the MFMA route,
// else launch_adapter_fwd_expand after it.
hipError_t launch_adapter_fwd_t(const void* x, int x_dtype, int64_t M, int64_t K, const float* A, int rank, void* ws,
                                hipStream_t s);
LowRankEpi adapter_fwd_epi(int64_t M, int64_t K, const float* B, int rank, float alpha, float* t, void* ws);
hipError_t launch_adapter_fwd_expand(float* y, int64_t M, int64_t N, int64_t K, const float* B, int rank, float alpha,
                                     float* t, void* ws, hipStream_t s);
hipError_t launch_adapter_bwd_u(const void* d_out, int dtype, int64_t M, int64_t N, int64_t K, const float* B,
                                int rank, void* ws, hipStream_t s);
LowRankEpi adapter_bwd_epi(int64_t M, int64_t N, int64_t K, const float* A, int rank, float alpha, void* ws);
hipError_t launch_adapter_bwd_rest(const void* x, const void* d_out, int dtype, int64_t M, int64_t N, int64_t K,
                                   const float* A, int rank, float alpha, const float* t, float* d_x, bool dx_done,
                                   float* d_A, float* d_B, void* ws, hipStream_t s);
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, double lr, double beta1,
                        double beta2, double eps, double weight_decay, int64_t step, hipStream_t s);

}  // namespace q4gsw
