// MFMA input gradient for M > 8, 16x16x32 form with an LDS transpose of the codes; serves
// fp16 d_out with foldable fp16 scales at the group sizes the 32x32x16 kernels (gemm_bwd2.hip)
// do not take (gs % 8 == 0 other than 32 and multiples of 64):
//   d_x[m, k] = sum_n d_out[m, n] * (code[n, k] - 8) * scale[k / gs, n]     (contract over N)
// the frozen-base input gradient of the Vulkan q4gsw-backward PR body, reading the
// forward's packed buffer as it is (no re-pack).
//
// The contraction runs over n, but a packed word holds 8 consecutive k of one row.
// Each block therefore unpacks its code tile once into LDS *transposed*: thread t
// takes one 8x8 micro-block, builds (n, n+1) pairs for every k with one byte
// permute across the two rows' words, and writes, per k, the 8 n-values as one
// 16-byte row of Bt[k][n].  The MFMA then reads B fragments (8 consecutive n of
// one k) and A fragments (8 consecutive n of one d_out row) with 16-byte LDS loads.
//
// Precision (fp32 accumulation): fp16 d_out with fp16 scales checked foldable at pack time,
// B = fp16((code - 8) * scale), one MFMA pass, |err| <= 2^-11 |w|.
#include "device.h"
#include "internal.h"

namespace q4gsw {

constexpr int kBBM = 128;     // block rows (M)
constexpr int kBCN = 64;      // contraction chunk (n) per LDS stage
constexpr int kBPitch = kBCN + 8;

struct BwdCfg {
    static constexpr int kWK = 128;                              // wave output columns (k)
    static constexpr int kBK = 2 * kWK;                          // block output columns
    static constexpr int kUI = kWK / 16;                         // 16-column MFMA tiles per wave
    static constexpr int kAElems = kBBM * kBPitch;
    static constexpr int kBElems = kBK * kBPitch;
};

__device__ __forceinline__ uint32_t byte_pair(uint32_t w_lo_row, uint32_t w_hi_row, int b) {
    // byte b of the even row's word -> byte 0, byte b of the odd row's word -> byte 2
    const uint32_t sel = (uint32_t)b | ((uint32_t)(4 + b) << 16) | 0x0C000C00u;
    return __builtin_amdgcn_perm(w_hi_row, w_lo_row, sel);
}

__global__ __launch_bounds__(256) void gemm_bwd_kernel(WView w, const void* __restrict__ d_out, int64_t M,
                                                       float* __restrict__ out, int64_t out_ld, int64_t split_stride,
                                                       int64_t col_limit, int g_vec, int chunks_per_split) {
    using C = BwdCfg;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][C::kAElems];
    __shared__ __attribute__((aligned(16))) uint16_t Bt[2][C::kBElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lrow = lane & 15;
    const int lq = lane >> 4;
    const int wm = wave >> 1;           // wave row half (64 rows)
    const int wk = wave & 1;            // wave column half

    const int64_t kb0 = (int64_t)blockIdx.x * C::kBK;      // first output column of the block
    const int64_t m0 = (int64_t)blockIdx.y * kBBM;
    const int64_t kocts = w.k_pad >> 3;
    const int64_t n_chunks = (w.N + kBCN - 1) / kBCN;
    const int64_t c_begin = (int64_t)blockIdx.z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    f4 acc[4][C::kUI];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < C::kUI; ++u) acc[i][u] = f4{0.f, 0.f, 0.f, 0.f};

    // ---- code tile -> Bt[k][n] (one micro-block per thread) ----
    const int mb_ro = tid / (C::kBK / 8);        // row-octet within the chunk (0..7)
    const int mb_ko = tid % (C::kBK / 8);        // k-octet within the block
    const bool mb_active = tid < 8 * (C::kBK / 8);
    const int64_t mb_O = (kb0 >> 3) + mb_ko;
    const bool mb_in = mb_active && mb_O < kocts;
    uint32_t wreg[8];
    auto load_codes = [&](int64_t nc) {
        if (!mb_in) return;
        const int64_t R = (nc >> 3) + mb_ro;
        const uint8_t* p = w.nib + 32 * (R * kocts + mb_O);
        const u4 a = ldg16_stream(p);
        const u4 b = ldg16_stream(p + 16);
        wreg[0] = a.x; wreg[1] = a.y; wreg[2] = a.z; wreg[3] = a.w;
        wreg[4] = b.x; wreg[5] = b.y; wreg[6] = b.z; wreg[7] = b.w;
    };
    uint32_t sreg[4];     // fp16 scale pairs (n, n+1) for the micro-block's rows
    auto load_fold_scales = [&](int64_t nc) {
        if (!mb_in) return;
        const int64_t g = (mb_O * 8) / w.gs;
        const u4 v = ldg16(static_cast<const uint16_t*>(w.scales) + scale_index(w.g_pad, nc + 8 * mb_ro, g));
        sreg[0] = v.x; sreg[1] = v.y; sreg[2] = v.z; sreg[3] = v.w;
    };
    auto store_codes = [&](int buf) {
        if (!mb_active) return;
        uint32_t col[8][4];           // col[j][a]: pair (n = 2a, 2a+1) at k-offset j
        if (!mb_in) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int a = 0; a < 4; ++a) col[j][a] = 0u;
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t t = byte_pair(wreg[2 * a], wreg[2 * a + 1], b);
                    const uint32_t plo = t & 0x000F000Fu;           // k-offset nib_pos^-1(2b)
                    const uint32_t phi = (t >> 4) & 0x000F000Fu;    // k-offset nib_pos^-1(2b+1)
                    // nibble positions 0..3 hold k-offsets 0,2,4,6 and positions 4..7 hold 1,3,5,7
                    const int jlo = ((2 * b) < 4) ? 2 * (2 * b) : 2 * (2 * b - 4) + 1;
                    const int jhi = ((2 * b + 1) < 4) ? 2 * (2 * b + 1) : 2 * (2 * b + 1 - 4) + 1;
                    const h2 s2 = bitcast<h2>(sreg[a]);
                    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
                    col[jlo][a] = bitcast<uint32_t>((bitcast<h2>(plo | 0x64006400u) - off) * s2);
                    col[jhi][a] = bitcast<uint32_t>((bitcast<h2>(phi | 0x64006400u) - off) * s2);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<u4*>(&Bt[buf][(mb_ko * 8 + j) * kBPitch + 8 * mb_ro]) =
                u4{col[j][0], col[j][1], col[j][2], col[j][3]};
    };

    // ---- d_out tile -> As (fp16 copy) ----
    constexpr int kUnitsPerRow = kBCN / 8;
    constexpr int kUnits = kBBM * kUnitsPerRow / 256;
    u4 areg[kUnits];
    auto load_a = [&](int64_t nc) {
        const int colu = tid % kUnitsPerRow;           // same for every unit of this thread
        const int64_t n = nc + 8 * colu;
#pragma unroll
        for (int c = 0; c < kUnits; ++c) {
            const int unit = tid + 256 * c;
            const int64_t m = m0 + unit / kUnitsPerRow;
            u4 v = {0u, 0u, 0u, 0u};
            if (m < M) {
                const uint16_t* src = static_cast<const uint16_t*>(d_out) + m * w.N + n;
                if (g_vec && n + 8 <= w.N) {
                    v = ldg16(src);
                } else {
                    uint32_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (n + j < w.N) ? src[j] : 0u;
                    v = u4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                }
            }
            areg[c] = v;
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int c = 0; c < kUnits; ++c) {
            const int unit = tid + 256 * c;
            const int row = unit / kUnitsPerRow;
            const int colu = unit % kUnitsPerRow;
            *reinterpret_cast<u4*>(&As[buf][row * kBPitch + 8 * colu]) = areg[c];
        }
    };

    if (c_begin < c_end) {
        load_codes(c_begin * kBCN);
        load_fold_scales(c_begin * kBCN);
        load_a(c_begin * kBCN);
        store_codes(0);
        store_a(0);
    }
    __syncthreads();

    for (int64_t ci = c_begin; ci < c_end; ++ci) {
        const int buf = (int)((ci - c_begin) & 1);
        const bool has_next = ci + 1 < c_end;
        if (has_next) {
            const int64_t nn = (ci + 1) * kBCN;
            load_codes(nn);
            load_fold_scales(nn);
            load_a(nn);
        }
        const uint16_t* Ab = &As[buf][0];
        const uint16_t* Bb = &Bt[buf][0];
#pragma unroll
        for (int t = 0; t < kBCN / 32; ++t) {
            u4 bfr[C::kUI];
#pragma unroll
            for (int u = 0; u < C::kUI; ++u)
                bfr[u] = *reinterpret_cast<const u4*>(Bb + (wk * C::kWK + 16 * u + lrow) * kBPitch + 32 * t + 8 * lq);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const uint16_t* pa = Ab + (wm * 64 + 16 * mi + lrow) * kBPitch + 32 * t + 8 * lq;
                const u4 a = *reinterpret_cast<const u4*>(pa);
#pragma unroll
                for (int u = 0; u < C::kUI; ++u) acc[mi][u] = mfma_f16(a, bfr[u], acc[mi][u]);
            }
        }
        if (has_next) {
            store_codes(buf ^ 1);
            store_a(buf ^ 1);
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds D[4*lq + r][lrow] of each 16x16 tile ----
    float* o = out + (int64_t)blockIdx.z * split_stride;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wm * 64 + 16 * mi + 4 * lq + r;
            if (m >= M) continue;
#pragma unroll
            for (int u = 0; u < C::kUI; ++u) {
                const int64_t k = kb0 + wk * C::kWK + 16 * u + lrow;
                if (k < col_limit) o[m * out_ld + k] = acc[mi][u][r];
            }
        }
}

bool gemm_bwd_v1_supported(const WView& w, int g_dtype, int fold_ok) {
    return g_dtype == kF16 && w.scale_f16 && fold_ok && w.gs % 8 == 0;
}

BwdPlan plan_gemm_bwd_v1(const WView& w, int g_dtype, int fold_ok, int64_t M) {
    (void)g_dtype;
    (void)fold_ok;
    BwdPlan p{};
    p.mode = kModeFold;
    const int bk = BwdCfg::kBK;
    const int64_t blocks = ((w.k_pad + bk - 1) / bk) * ((M + kBBM - 1) / kBBM);
    const int64_t n_chunks = (w.N + kBCN - 1) / kBCN;
    int64_t splits = 1;
    while (blocks * splits < 256 && n_chunks / (splits * 2) >= 4) splits *= 2;
    p.splits = (int)splits;
    p.ws_bytes = splits > 1 ? (int64_t)splits * M * w.k_pad * 4 : 0;
    return p;
}

hipError_t launch_gemm_bwd_v1(const WView& w, const void* d_out, int g_dtype, int64_t M, float* d_x,
                              const BwdPlan& plan, float* ws, hipStream_t s) {
    if (plan.mode != kModeFold || g_dtype != kF16) return hipErrorInvalidValue;
    const int bk = BwdCfg::kBK;
    const int64_t n_chunks = (w.N + kBCN - 1) / kBCN;
    const int per = (int)((n_chunks + plan.splits - 1) / plan.splits);
    const dim3 grid((unsigned)((w.k_pad + bk - 1) / bk), (unsigned)((M + kBBM - 1) / kBBM), (unsigned)plan.splits);
    const int g_vec = ((reinterpret_cast<uintptr_t>(d_out) & 15u) == 0) && ((w.N * 2) % 16 == 0);
    float* out = plan.splits == 1 ? d_x : ws;
    const int64_t ld = plan.splits == 1 ? w.K : w.k_pad;
    const int64_t stride = plan.splits == 1 ? 0 : M * w.k_pad;
    const int64_t limit = plan.splits == 1 ? w.K : w.k_pad;
    hipLaunchKernelGGL(gemm_bwd_kernel, grid, dim3(256), 0, s, w, d_out, M, out, ld, stride, limit, g_vec, per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    return launch_reduce_splits(ws, plan.splits, M, w.K, w.k_pad, d_x, w.K, s);
}

}  // namespace q4gsw
