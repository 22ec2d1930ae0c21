// MFMA forward for M > 8:  y[m, n] = sum_k x[m, k] * (code[n, k] - 8) * scale[k / gs, n].
//
// The forward GEMM of the pages (the linear_q4gsw op; the WebGPU BK64 QKV PR body
// mirrors the Vulkan q4gsw forward GEMM per projection) re-designed for gfx950:
//
//   * block = 4 waves, block tile 128 (M) x 256 (N); wave tile 128 x 64 as
//     8 x 4 tiles of v_mfma_f32_16x16x32 with fp32 accumulators;
//   * activations are staged through LDS (double-buffered chunks of CK columns);
//   * codes are never staged: each wave streams its own 16-byte code quads
//     (4 rows x 8 columns) straight from HBM into registers and unpacks them
//     there, so the LDS carries only the activation tile;
//   * K is split across blocks when the output tiles alone cannot fill the GPU;
//     split partials go to a workspace and a reduction kernel sums them.
//
// Precision routes (all with fp32 accumulation):
//   kModeFold  (fp16 x, fp16 scales checked foldable at pack time):
//       B = fp16((code - 8) * scale), one rounding, |err| <= 2^-11 |w|.
//   kModeGroup (fp16 or bf16 x): B = code - 8 held exactly (fp16 or bf16) and the scale
//       multiplies the fp32 partial sum of each CK-column chunk (the chunk lies inside
//       one group).
//   kModeSplit (fp32 x): x = hi + lo in bf16 (|err| <= 2^-18 |x|), two MFMA passes
//       against B = code - 8 (exact bf16), scale per chunk as in kModeGroup.
#include "device.h"
#include "internal.h"

namespace q4gsw {

constexpr int kBM = 128;          // block rows (M)
constexpr int kWN = 64;           // wave columns (N)
constexpr int kBN = 4 * kWN;      // block columns (N)

struct FwdSegArgs {
    const uint8_t* nib[3];
    const void* scales[3];
    float* out[3];                // final output (splits == 1) or workspace base of the segment
    int64_t N[3];
    int64_t n_pad[3];
    int64_t out_ld[3];            // row pitch of out
    int64_t tile_start[4];        // first N tile of each segment (prefix sums), tile_start[nseg] = total
    int64_t g_pad;                // scale groups stored (shared: the segments share K and group size)
    int nseg;
};

template <int XT, int MODE, int CK>
struct FwdCfg {
    static constexpr int kSteps = CK / 32;                       // MFMA K-steps per chunk
    static constexpr int kPitch = CK + 8;                        // LDS row pitch, 16-bit elements
    static constexpr int kPlanes = (MODE == kModeSplit) ? 2 : 1; // hi (+ lo) planes
    static constexpr int kStageElems = kPlanes * kBM * kPitch;
    static constexpr int kUnitsPerRow = (XT == kF32) ? CK / 4 : CK / 8;   // 16-byte global loads per row
    static constexpr int kUnits = kBM * kUnitsPerRow / 256;               // per thread per chunk
};

template <int XT, int MODE, int CK>
__global__ __launch_bounds__(256) void gemm_fwd_kernel(FwdSegArgs seg, const void* __restrict__ x, int64_t M,
                                                       int64_t K, int64_t k_pad, int64_t gs, int scale_f16,
                                                       int x_vec, int chunks_per_split, int64_t split_stride) {
    using C = FwdCfg<XT, MODE, CK>;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][C::kStageElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lrow = lane & 15;       // MFMA row/column index inside a 16x16 tile
    const int lq = lane >> 4;         // MFMA k-group (8 elements each)

    // ---- which segment / N tile / M tile / K split this block owns ----
    const int64_t tile = blockIdx.x;
    int sg = 0;
    while (sg + 1 < seg.nseg && tile >= seg.tile_start[sg + 1]) ++sg;
    const int64_t n_block0 = (tile - seg.tile_start[sg]) * kBN;
    const int64_t n0 = n_block0 + (int64_t)wave * kWN;           // first row of W for this wave
    const bool wave_active = n0 < seg.n_pad[sg];
    const uint8_t* nib = seg.nib[sg];
    const void* scales = seg.scales[sg];
    const int64_t n_pad = seg.n_pad[sg];
    const int64_t g_pad = seg.g_pad;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t kocts = k_pad >> 3;
    const int64_t n_chunks = (K + CK - 1) / CK;
    const int64_t c_begin = (int64_t)blockIdx.z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    // Code quads: lane (lrow, lq) reads rows n0 + 4*lrow .. +3, k-octet 4*step + lq of the chunk.
    const uint8_t* qbase = nib + 32 * (((n0 >> 3) + (lrow >> 1)) * kocts) + 16 * (lrow & 1);

    f4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[i][u] = f4{0.f, 0.f, 0.f, 0.f};

    // ---------------- activation staging ----------------
    u4 areg[C::kUnits];
    auto load_a = [&](int64_t kc) {
#pragma unroll
        for (int c = 0; c < C::kUnits; ++c) {
            const int unit = tid + 256 * c;
            const int row = unit / C::kUnitsPerRow;
            const int64_t m = m0 + row;
            if constexpr (XT == kF32) {
                const int64_t k = kc + 4 * (unit % C::kUnitsPerRow);
                f4 v = {0.f, 0.f, 0.f, 0.f};
                if (m < M) {
                    const float* src = static_cast<const float*>(x) + m * K + k;
                    if (x_vec && k + 4 <= K) {
                        v = *reinterpret_cast<const f4*>(src);
                    } else {
                        v.x = (k + 0 < K) ? src[0] : 0.f;
                        v.y = (k + 1 < K) ? src[1] : 0.f;
                        v.z = (k + 2 < K) ? src[2] : 0.f;
                        v.w = (k + 3 < K) ? src[3] : 0.f;
                    }
                }
                areg[c] = bitcast<u4>(v);
            } else {
                const int64_t k = kc + 8 * (unit % C::kUnitsPerRow);
                u4 v = {0u, 0u, 0u, 0u};
                if (m < M) {
                    const uint16_t* src = static_cast<const uint16_t*>(x) + m * K + k;
                    if (x_vec && k + 8 <= K) {
                        v = ldg16(src);
                    } else {
                        uint32_t e[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) e[j] = (k + j < K) ? src[j] : 0u;
                        v = u4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                    }
                }
                areg[c] = v;
            }
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int c = 0; c < C::kUnits; ++c) {
            const int unit = tid + 256 * c;
            const int row = unit / C::kUnitsPerRow;
            const int col = unit % C::kUnitsPerRow;
            if constexpr (XT == kF32) {
                const f4 v = bitcast<f4>(areg[c]);
                uint32_t h0, l0, h1, l1;
                split_bf16(v.x, v.y, h0, l0);
                split_bf16(v.z, v.w, h1, l1);
                uint16_t* hi = &As[buf][row * C::kPitch + 4 * col];
                uint16_t* lo = hi + kBM * C::kPitch;
                *reinterpret_cast<u2*>(hi) = u2{h0, h1};
                *reinterpret_cast<u2*>(lo) = u2{l0, l1};
            } else {
                *reinterpret_cast<u4*>(&As[buf][row * C::kPitch + 8 * col]) = areg[c];
            }
        }
    };

    // ---------------- code quads ----------------
    u4 breg[C::kSteps];
    auto load_b = [&](int64_t kc, u4 (&dst)[C::kSteps]) {
        if (!wave_active) return;
#pragma unroll
        for (int t = 0; t < C::kSteps; ++t) dst[t] = ldg16_stream(qbase + 32 * ((kc >> 3) + 4 * t + lq));
    };

    if (c_begin < c_end) {
        load_a(c_begin * CK);
        load_b(c_begin * CK, breg);
        store_a(0);
    }
    __syncthreads();

    for (int64_t ci = c_begin; ci < c_end; ++ci) {
        const int buf = (int)((ci - c_begin) & 1);
        const int64_t kc = ci * CK;
        const bool has_next = ci + 1 < c_end;
        u4 bnext[C::kSteps];
        if (has_next) {
            load_a(kc + CK);
            load_b(kc + CK, bnext);
        }
        if (wave_active) {
            // ---- unpack this wave's code fragments for the chunk ----
            u4 bfr[C::kSteps][4];
            float gscale[4];
            if constexpr (MODE == kModeFold) {
#pragma unroll
                for (int t = 0; t < C::kSteps; ++t) {
                    const int64_t g = (kc + 32 * t + 8 * lq) / gs;
                    const u2 sv = *reinterpret_cast<const u2*>(static_cast<const uint16_t*>(scales) +
                                                               scale_index(g_pad, n0 + 4 * lrow, g));
                    const uint32_t s01 = sv.x, s23 = sv.y;
                    const uint32_t sw[4] = {s01 & 0xFFFFu, s01 >> 16, s23 & 0xFFFFu, s23 >> 16};
                    const uint32_t wd[4] = {breg[t].x, breg[t].y, breg[t].z, breg[t].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const h2 s2 = bitcast<h2>(sw[u] | (sw[u] << 16));
                        uint32_t p[4];
#pragma unroll
                        for (int s = 0; s < 4; ++s) p[s] = bitcast<uint32_t>(codes_minus8_f16(wd[u], s) * s2);
                        bfr[t][u] = u4{p[0], p[1], p[2], p[3]};
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < C::kSteps; ++t) {
                    const uint32_t wd[4] = {breg[t].x, breg[t].y, breg[t].z, breg[t].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        uint32_t p[4];
                        const uint32_t wx = wd[u] ^ 0x88888888u;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            if constexpr (XT == kF16) p[s] = bitcast<uint32_t>(codes_minus8_f16(wd[u], s));
                            else p[s] = codes_minus8_bf16(wx, s);
                        }
                        bfr[t][u] = u4{p[0], p[1], p[2], p[3]};
                    }
                }
                const int64_t g = kc / gs;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    gscale[u] = load_scale(scales, scale_f16, scale_index(g_pad, n0 + 4 * lrow + u, g));
            }

            // ---- MFMA over the 8 row tiles ----
            const uint16_t* Ab = &As[buf][0];
#pragma unroll
            for (int mi = 0; mi < 8; ++mi) {
                u4 afr[C::kSteps];
                u4 alo[C::kSteps];
#pragma unroll
                for (int t = 0; t < C::kSteps; ++t) {
                    const uint16_t* p = Ab + (mi * 16 + lrow) * C::kPitch + 32 * t + 8 * lq;
                    afr[t] = *reinterpret_cast<const u4*>(p);
                    if constexpr (MODE == kModeSplit) alo[t] = *reinterpret_cast<const u4*>(p + kBM * C::kPitch);
                }
                if constexpr (MODE == kModeFold) {
#pragma unroll
                    for (int t = 0; t < C::kSteps; ++t)
#pragma unroll
                        for (int u = 0; u < 4; ++u) acc[mi][u] = mfma_f16(afr[t], bfr[t][u], acc[mi][u]);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        f4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int t = 0; t < C::kSteps; ++t) {
                            if constexpr (XT == kF16) {
                                tmp = mfma_f16(afr[t], bfr[t][u], tmp);
                            } else {
                                tmp = mfma_bf16(afr[t], bfr[t][u], tmp);
                                if constexpr (MODE == kModeSplit) tmp = mfma_bf16(alo[t], bfr[t][u], tmp);
                            }
                        }
                        acc[mi][u] = acc[mi][u] + tmp * gscale[u];
                    }
                }
            }
        }
        if (has_next) {
            store_a(buf ^ 1);
#pragma unroll
            for (int t = 0; t < C::kSteps; ++t) breg[t] = bnext[t];
        }
        __syncthreads();
    }

    // ---------------- epilogue ----------------
    if (!wave_active) return;
    float* out = seg.out[sg] + (int64_t)blockIdx.z * split_stride;
    const int64_t ld = seg.out_ld[sg];
    const int64_t ncols = split_stride ? n_pad : seg.N[sg];
    const int64_t ncol0 = n0 + 4 * lrow;
    const bool vec_ok = (ld % 4 == 0) && (ncol0 + 4 <= ncols);
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + mi * 16 + 4 * lq + r;
            if (m >= M) continue;
            const f4 v = {acc[mi][0][r], acc[mi][1][r], acc[mi][2][r], acc[mi][3][r]};
            float* dst = out + m * ld + ncol0;
            if (vec_ok) {
                *reinterpret_cast<f4*>(dst) = v;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (ncol0 + u < ncols) dst[u] = v[u];
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
static int fwd_chunk(int mode, int64_t gs) {
    if (mode == kModeFold) return 64;
    if (mode == kModeSplit) return 32;
    return (gs % 64 == 0) ? 64 : 32;
}

bool gemm_fwd_supported(const WView& w, int x_dtype, int fold_ok) {
    if (x_dtype == kF16 && w.scale_f16 && fold_ok) return w.gs % 8 == 0;
    return w.gs % 32 == 0;
}

FwdPlan plan_gemm_fwd(const FwdSeg* segs, int nseg, int x_dtype, int fold_ok, int64_t M) {
    FwdPlan p{};
    const WView& w0 = segs[0].w;
    if (x_dtype == kF32) p.mode = kModeSplit;
    else if (x_dtype == kF16 && w0.scale_f16 && fold_ok) p.mode = kModeFold;
    else p.mode = kModeGroup;
    int64_t tiles = 0, npad_total = 0;
    for (int i = 0; i < nseg; ++i) {
        tiles += (segs[i].w.n_pad + kBN - 1) / kBN;
        npad_total += segs[i].w.n_pad;
    }
    const int64_t blocks = tiles * ((M + kBM - 1) / kBM);
    const int64_t n_chunks = (w0.K + fwd_chunk(p.mode, w0.gs) - 1) / fwd_chunk(p.mode, w0.gs);
    int64_t splits = 1;
    while (blocks * splits < 256 && n_chunks / (splits * 2) >= 4) splits *= 2;
    p.splits = (int)splits;
    p.ws_bytes = splits > 1 ? (int64_t)splits * M * npad_total * 4 : 0;
    return p;
}

template <int XT, int MODE, int CK>
static void launch_fwd_t(dim3 grid, hipStream_t s, const FwdSegArgs& a, const void* x, int64_t M, int64_t K,
                         int64_t k_pad, int64_t gs, int scale_f16, int x_vec, int per, int64_t stride) {
    hipLaunchKernelGGL((gemm_fwd_kernel<XT, MODE, CK>), grid, dim3(256), 0, s, a, x, M, K, k_pad, gs, scale_f16,
                       x_vec, per, stride);
}

// One launch over every segment.  With K splits the partials go to ws laid out as
// [splits][M][sum of n_pad], segment i starting at column offset sum_{j<i} n_pad_j.
hipError_t launch_gemm_fwd(const FwdSeg* segs, int nseg, const void* x, int x_dtype, int64_t M,
                           const FwdPlan& plan, float* ws, hipStream_t s) {
    const WView& w0 = segs[0].w;
    FwdSegArgs a{};
    a.nseg = nseg;
    int64_t tiles = 0, npad_total = 0;
    for (int i = 0; i < nseg; ++i) npad_total += segs[i].w.n_pad;
    int64_t col = 0;
    for (int i = 0; i < nseg; ++i) {
        a.nib[i] = segs[i].w.nib;
        a.scales[i] = segs[i].w.scales;
        a.N[i] = segs[i].w.N;
        a.n_pad[i] = segs[i].w.n_pad;
        a.tile_start[i] = tiles;
        tiles += (segs[i].w.n_pad + kBN - 1) / kBN;
        if (plan.splits == 1) {
            a.out[i] = segs[i].out;
            a.out_ld[i] = segs[i].w.N;
        } else {
            a.out[i] = ws + col;
            a.out_ld[i] = npad_total;
        }
        col += segs[i].w.n_pad;
    }
    a.tile_start[nseg] = tiles;
    a.g_pad = w0.g_pad;
    const int mode = plan.mode;
    const int ck = fwd_chunk(mode, w0.gs);
    const int64_t n_chunks = (w0.K + ck - 1) / ck;
    const int per = (int)((n_chunks + plan.splits - 1) / plan.splits);
    const int esize = x_dtype == kF32 ? 4 : 2;
    const int x_vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0) && ((w0.K * esize) % 16 == 0);
    const dim3 g((unsigned)tiles, (unsigned)((M + kBM - 1) / kBM), (unsigned)plan.splits);
    const int64_t st = plan.splits == 1 ? 0 : M * npad_total;
    const int64_t K = w0.K, kp = w0.k_pad, gs = w0.gs;
    const int sf = w0.scale_f16;
    if (mode == kModeFold) {
        launch_fwd_t<kF16, kModeFold, 64>(g, s, a, x, M, K, kp, gs, sf, x_vec, per, st);
    } else if (mode == kModeSplit) {
        launch_fwd_t<kF32, kModeSplit, 32>(g, s, a, x, M, K, kp, gs, sf, x_vec, per, st);
    } else if (x_dtype == kF16) {
        if (ck == 64) launch_fwd_t<kF16, kModeGroup, 64>(g, s, a, x, M, K, kp, gs, sf, x_vec, per, st);
        else launch_fwd_t<kF16, kModeGroup, 32>(g, s, a, x, M, K, kp, gs, sf, x_vec, per, st);
    } else {
        if (ck == 64) launch_fwd_t<kBF16, kModeGroup, 64>(g, s, a, x, M, K, kp, gs, sf, x_vec, per, st);
        else launch_fwd_t<kBF16, kModeGroup, 32>(g, s, a, x, M, K, kp, gs, sf, x_vec, per, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    for (int i = 0; i < nseg; ++i) {
        e = launch_reduce_splits(a.out[i], plan.splits, M, segs[i].w.N, npad_total, segs[i].out, segs[i].w.N, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4gsw
