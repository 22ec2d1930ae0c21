// MFMA input gradient for M > 8, 32x32x16 form:
//   d_x[m, k] = sum_n d_out[m, n] * (code[n, k] - 8) * scale[k / gs, n]     (contract over N)
// the frozen-base input gradient of the Vulkan q4gsw-backward PR body, reading the forward's
// packed buffer as it is (no re-pack).
//
// A wave owns a 128 (M) x 64 (K) output tile = 4 x 2 MFMA tiles; a block holds four such tiles
// side by side in K (block tile 128 x 256).  The contraction runs over n in 64-row chunks.  Two
// kernels:
//
//   * gemm_bwd_fold_kernel (fp16 d_out, fp16 scales checked foldable at pack time), 4 waves:
//     d_out is LDS-DMA'd as it is and B = fp16((code - 8) * scale[g, n]), one rounding,
//     |err| <= 2^-11 |w|; one pass.  Each wave LDS-DMAs its 64 (n) x 64 (k) code tile per chunk
//     (8 row-octets x 256 contiguous bytes, the row-octet R run rotated by R 32-byte blocks).
//     The MFMA B fragment needs 8 consecutive n of one k: one nibble position of the 8 words of
//     a 32-byte micro-block, so each lane reads its micro-block and extracts its nibble from
//     every word (a register transpose).  Issue order per MFMA step: the next step's LDS reads,
//     then (MFMA, unpacking piece) pairs fenced with sched_barrier.
//   * the same kernel with an exact bf16 B (XB > 0; fp32 / bf16 d_out, and fp16 with scales that
//     cannot be folded, at the group sizes the split kernel does not take): for fp16 scales
//     (code - 8) * scale / 16 has at most 14 significant bits, so it is exactly the sum of two
//     bf16 values hi + lo; d_out is staged by a pre-pass as one bf16 plane (bf16 d_out as it is)
//     or two (fp32 / fp16 d_out split into bf16 hi + lo, |err| <= 2^-18 |d_out|, exact for fp16),
//     and two or four MFMA passes multiply them;
//   * gemm_bwd_split_kernel (fp32 / bf16 d_out, and fp16 with scales that cannot be folded),
//     4 consumer + 4 producer waves: the block's columns lie in at most two scale groups
//     (gs % 128 == 0; a change can only fall at column 128 of the block), so the scale moves to
//     the A side: A' = d_out * scale[g, n] in fp32, split into bf16 hi + lo (|err| <= 2^-18 |A'|)
//     by the producers while it is staged into LDS, one copy per group; B = code - 8 exactly in
//     bf16 from the transposing 4-bit LDS read; two MFMA passes.
#include "device.h"
#include "internal.h"

#include <type_traits>

namespace q4gsw {
namespace {

constexpr int kBM = 128;            // block rows (M)
constexpr int kWK = 64;             // wave output columns (K)
constexpr int kBK = 4 * kWK;        // block output columns
constexpr int kCN = 64;             // contraction rows (n) per chunk
constexpr int kRowBytes = 128;      // one 16-bit A row of a chunk in LDS
constexpr int kPlaneBytes = kBM * kRowBytes;
constexpr int kCodeBytes = 2048;    // one wave's codes per chunk: 64 n x 64 k x 4 bits

// A wave's 128 x 64 split partials (4 x 2 tiles of 32 x 32, times f) in the fragment layout of
// a plane with ntn 32-column tiles: four 16-byte stores per lane and tile, streamed past the
// caches (the reduction reads each byte once); tiles wholly past M are skipped.
__device__ __forceinline__ void store_frag_partials(float* plane, int64_t ntn, int64_t M, int64_t m0, int64_t kw0,
                                                    int lane, const f32x16 (&acc)[4][2], float f) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int64_t tm = m0 / 32 + mi;
        if (32 * tm >= M) break;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float* tp = plane + (tm * ntn + kw0 / 32 + u) * 1024 + 4 * lane;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                __builtin_nontemporal_store(f4{f * acc[mi][u][4 * r4], f * acc[mi][u][4 * r4 + 1],
                                               f * acc[mi][u][4 * r4 + 2], f * acc[mi][u][4 * r4 + 3]},
                                            reinterpret_cast<f4*>(tp + 256 * r4));
        }
    }
}

// x * s for an fp16 s held in the low / high half of sw, rounded once to fp32.  Written as an FMA
// with a zero addend so it maps to the mixed-precision FMA, which takes the fp16 operand directly.
__device__ __forceinline__ float mul_f16_lo(float x, uint32_t sw) {
    return __builtin_fmaf(x, f16_bits_to_f32((uint16_t)(sw & 0xFFFFu)), 0.0f);
}
__device__ __forceinline__ float mul_f16_hi(float x, uint32_t sw) {
    return __builtin_fmaf(x, f16_bits_to_f32((uint16_t)(sw >> 16)), 0.0f);
}
// bf16 hi / lo split of two fp32 values (both roundings to nearest even): a = hi + lo + e with
// |e| <= 2^-18 |a|.  a - hi is exact in fp32.  Both fp32 hi values come from the packed hi word
// (a byte permute and a mask), so the conversion is done once.
__device__ __forceinline__ void split_bf16_pair(float a0, float a1, uint32_t& hi, uint32_t& lo) {
    b2 h = {(__bf16)a0, (__bf16)a1};
    const uint32_t hb = bitcast<uint32_t>(h);
    const float r0 = a0 - bitcast<float>(__builtin_amdgcn_perm(hb, hb, 0x05040c0cu));   // hb << 16
    const float r1 = a1 - bitcast<float>(hb & 0xFFFF0000u);
    b2 l = {(__bf16)r0, (__bf16)r1};
    hi = hb;
    lo = bitcast<uint32_t>(l);
}

// NV = scale groups per wave (1: gs % 64 == 0, 2: gs == 32).
// XB = 0: fp16 d_out and B = fp16((code - 8) * scale), one pass.  XB = 1 or 2: exact bf16
// B = hi + lo of (code - 8) * scale / 16 against XB bf16 planes of d_out (a_plane elements apart),
// two or four passes; the output carries the factor 16 back exactly.
template <int NV, int XB>
__global__ __launch_bounds__(256, 1) void gemm_bwd_fold_kernel(WView w, const void* __restrict__ d_out, int64_t M,
                                                               float* __restrict__ out, int64_t out_ld,
                                                               int64_t split_stride, int64_t col_limit, int g_fast,
                                                               int chunks_per_split, int splits, int mtiles,
                                                               int64_t a_plane) {
    constexpr int kAPlanes = XB == 2 ? 2 : 1;
    constexpr int kARing = 3;                                   // A stages
    constexpr int kAStage = kAPlanes * kPlaneBytes;
    constexpr int kSBytes = 256;                                // per-wave scales per chunk
    constexpr int kCStage = 4 * (kCodeBytes + kSBytes);
    constexpr int kDmaPerChunk = 4 * kAPlanes + 2 + 1;
    constexpr float kOutScale = XB == 0 ? 1.0f : 16.0f;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kARing * kAStage + 3 * kCStage];
    uint8_t* const Aring = smem;
    uint8_t* const Cring = smem + kARing * kAStage;
    lds_u8* const sm_l = (lds_u8*)smem;
    const int kCOff = kARing * kAStage;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = lane & 31;          // MFMA row / column inside a 32x32 tile
    const int h = lane >> 5;          // MFMA contraction group: n-octet 2t + h of step t

    // ---- block -> (N split, M tile, K tile); the split index varies fastest ----
    const int64_t bid = blockIdx.x;
    const int z = (int)(bid % splits);
    const int64_t rest = bid / splits;
    const int64_t mb = rest % mtiles;
    const int64_t tile = rest / mtiles;
    const int64_t kb0 = tile * kBK;
    const int64_t m0 = mb * kBM;
    const int64_t kw0 = kb0 + (int64_t)wave * kWK;            // first output column of the wave
    const bool wave_active = kw0 < w.k_pad;
    const int64_t kwc = wave_active ? kw0 : 0;                // an idle wave streams valid columns
    const int64_t kocts = w.k_pad >> 3;
    const int64_t N = w.N;
    const int64_t n_chunks = (N + kCN - 1) / kCN;
    const int64_t c_begin = (int64_t)z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    // ---------------- code and scale DMA ----------------
    // DMA r covers row-octets 4r .. 4r+3 of the chunk; lane l fills bytes 16 l: row-octet
    // R = 4r + (l >> 4), rotated block slot p = (l & 15) >> 1, half l & 1, holding the wave's
    // k-octet (p - R) & 7.
    const uint8_t* csrc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int R = 4 * r + (lane >> 4);
        const int o = (((lane & 15) >> 1) - R) & 7;
        csrc[r] = w.nib + 32 * ((int64_t)R * kocts + (kwc >> 3) + o) + 16 * (lane & 1);
    }
    const int64_t chunk_code_stride = 32 * 8 * kocts;         // 8 row-octets
    // scales: lane l loads 4 bytes = the fp16 scales of rows 2 (l & 3), +1 of row-octet
    // (l & 31) >> 2 for group slot l >> 5 (two slots only when gs == 32).
    const int fgl = (NV == 2) ? (lane >> 5) : 0;
    const int64_t fgroup = (kwc + 32 * fgl) / w.gs;
    const int64_t fsrc = (int64_t)((lane & 31) >> 2) * (w.g_pad * 8) + fgroup * 8 + 2 * (lane & 3);
    auto issue_codes = [&](int64_t c, int st) {
        lds_u8* base = sm_l + kCOff + st * kCStage + wave * (kCodeBytes + kSBytes);
#pragma unroll
        for (int r = 0; r < 2; ++r) dma16(csrc[r] + chunk_code_stride * c, base + 1024 * r);
        dma4(static_cast<const uint16_t*>(w.scales) + fsrc + 8 * c * (w.g_pad * 8), base + kCodeBytes);
    };

    // ---------------- d_out (fp16) DMA, as the forward's activation staging ----------------
    const uint16_t* xa[4];
    int xoct[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = 32 * wave + 8 * q + (lane >> 3);
        xoct[q] = (lane & 7) ^ ((row >> 1) & 7);
        const int64_t m = min(m0 + row, M - 1);                // rows past M only feed discarded outputs
        xa[q] = static_cast<const uint16_t*>(d_out) + m * N + 8 * xoct[q];
    }
    auto issue_a16 = [&](int64_t c, int st) {
        const int64_t nc = c * kCN;
        if (g_fast && nc + kCN <= N) {
#pragma unroll
            for (int pl = 0; pl < kAPlanes; ++pl)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dma16(xa[q] + pl * a_plane + nc,
                          sm_l + st * kAStage + pl * kPlaneBytes + (32 * wave + 8 * q) * kRowBytes);
        } else {
            // ragged n tail or unaligned d_out: zero-filled register loads into the same slots
#pragma unroll
            for (int pl = 0; pl < kAPlanes; ++pl)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 32 * wave + 8 * q + (lane >> 3);
                    const int64_t m = m0 + row;
                    const int64_t n = nc + 8 * xoct[q];
                    const uint16_t* src = static_cast<const uint16_t*>(d_out) + pl * a_plane;
                    uint32_t e[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) e[i] = (m < M && n + i < N) ? src[m * N + n + i] : 0u;
                    *reinterpret_cast<u4*>(Aring + st * kAStage + pl * kPlaneBytes + row * kRowBytes + 16 * (lane & 7)) =
                        u4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                }
        }
    };

    // ---------------- accumulators and one chunk of MFMAs ----------------
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][u][r] = 0.f;

    const int swz = (j >> 1) & 7;                 // ((row >> 1) & 7) of every A row this lane reads
    const int npos = 4 * nib_pos(j & 7);          // bit offset of this lane's k in each code word
    // A fragments of step t (and of the lo plane when there is one)
    auto read_a = [&](const uint8_t* Ab, int t, u4 (&a)[4], u4 (&alo)[4]) {
        const int slot = 16 * ((2 * t + h) ^ swz);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            a[mi] = *reinterpret_cast<const u4*>(Ab + (32 * mi + j) * kRowBytes + slot);
            if constexpr (kAPlanes == 2) alo[mi] = *reinterpret_cast<const u4*>(Ab + kPlaneBytes + (32 * mi + j) * kRowBytes + slot);
        }
    };
    // the 8 code words of step t for column u (micro-block row-octet 2t + h, k-octet 4u + j/8)
    auto read_b = [&](const uint8_t* Cb, int t, u4 (&wd)[2][2]) {
        const int R = 2 * t + h;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int o = 4 * u + (j >> 3);
            const uint8_t* p = Cb + 256 * R + 32 * ((o + R) & 7);
            wd[u][0] = *reinterpret_cast<const u4*>(p);
            wd[u][1] = *reinterpret_cast<const u4*>(p + 16);
        }
    };
    auto read_fs = [&](const uint8_t* Sb, int t, u4 (&fs)[2]) {
        const int R = 2 * t + h;
#pragma unroll
        for (int u = 0; u < 2; ++u) fs[u] = *reinterpret_cast<const u4*>(Sb + 128 * (NV == 2 ? u : 0) + 16 * R);
    };
    // dword e of B fragment u: rows 2e, 2e+1 of the micro-block at this lane's k.  XB = 0: fp16
    // (code - 8) * scale, one rounding.  XB > 0: the exact fp32 value (code - 8) / 16 * scale (a
    // 4-bit signed convert of code ^ 8, times the fp16 scale in a mixed-precision FMA) split into
    // bf16 hi (b) + lo (blo) with no error.
    auto bpiece = [&](const u4 (&wd)[2][2], const u4 (&fs)[2], u4 (&b)[2], u4 (&blo)[2], int i) {
        const int u = i >> 2, e = i & 3;
        const uint32_t w0 = wd[u][e >> 1][2 * (e & 1)];
        const uint32_t w1 = wd[u][e >> 1][2 * (e & 1) + 1];
        if constexpr (XB == 0) {
            const uint32_t c0 = __builtin_amdgcn_ubfe(w0, npos, 4);
            const uint32_t c1 = __builtin_amdgcn_ubfe(w1, npos, 4);
            const h2 v = bitcast<h2>((c0 | (c1 << 16)) | 0x64006400u);
            const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
            b[u][e] = bitcast<uint32_t>((v - off) * bitcast<h2>(fs[u][e]));
        } else {
            const float v0 = __builtin_amdgcn_cvt_off_f32_i4((int)__builtin_amdgcn_ubfe(w0 ^ 0x88888888u, npos, 4));
            const float v1 = __builtin_amdgcn_cvt_off_f32_i4((int)__builtin_amdgcn_ubfe(w1 ^ 0x88888888u, npos, 4));
            uint32_t hi, lo;
            split_bf16_pair(mul_f16_lo(v0, fs[u][e]), mul_f16_hi(v1, fs[u][e]), hi, lo);
            b[u][e] = hi;
            blo[u][e] = lo;
        }
    };
    auto compute = [&](int st) {
        const uint8_t* Ab = Aring + st * kAStage;
        const uint8_t* Cb = Cring + st * kCStage + wave * (kCodeBytes + kSBytes);
        const uint8_t* Sb = Cb + kCodeBytes;
        u4 a[2][4], alo[2][4], wd[2][2][2], fs[2][2], b[2][2], blo[2][2];
        read_a(Ab, 0, a[0], alo[0]);
        read_b(Cb, 0, wd[0]);
        read_fs(Sb, 0, fs[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) bpiece(wd[0], fs[0], b[0], blo[0], i);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cur = t & 1, nxt = (t + 1) & 1;
            if (t < 3) {
                read_a(Ab, t + 1, a[nxt], alo[nxt]);
                read_b(Cb, t + 1, wd[nxt]);
                read_fs(Sb, t + 1, fs[nxt]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int mi = i >> 1, u = i & 1;
                if constexpr (XB == 0) {
                    acc[mi][u] = mfma32_f16(a[cur][mi], b[cur][u], acc[mi][u]);
                } else {
                    acc[mi][u] = mfma32_bf16(a[cur][mi], b[cur][u], acc[mi][u]);
                    acc[mi][u] = mfma32_bf16(a[cur][mi], blo[cur][u], acc[mi][u]);
                    if constexpr (XB == 2) {
                        acc[mi][u] = mfma32_bf16(alo[cur][mi], b[cur][u], acc[mi][u]);
                        acc[mi][u] = mfma32_bf16(alo[cur][mi], blo[cur][u], acc[mi][u]);
                    }
                }
                if (t < 3) bpiece(wd[nxt], fs[nxt], b[nxt], blo[nxt], (i & 1) * 4 + (i >> 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---------------- pipeline ----------------
    // d_out, codes and scales are DMA'd two chunks ahead into a 3-stage ring; before chunk c is
    // read only chunk c + 1's DMAs may be in flight (a chunk staged through the synchronous
    // fallback drained every older load already).
    if (c_begin < c_end) {
        issue_a16(c_begin, 0);
        issue_codes(c_begin, 0);
        if (c_begin + 1 < c_end) {
            issue_a16(c_begin + 1, 1);
            issue_codes(c_begin + 1, 1);
        }
    }
    int st = 0;
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int st_next = (st == 2) ? 0 : st + 1;
        const int st_prev = (st == 0) ? 2 : st - 1;
        if (c + 1 < c_end) wait_loads_barrier<kDmaPerChunk>();
        else wait_loads_barrier<0>();
        if (c + 2 < c_end) {
            issue_a16(c + 2, st_prev);
            issue_codes(c + 2, st_prev);
        }
        compute(st);
        st = st_next;
    }

    // ---------------- epilogue: lane holds D[8 (r/4) + 4 h + r%4][j] of each 32x32 tile ----------------
    if (!wave_active) return;
    if (split_stride) {
        store_frag_partials(out + (int64_t)z * split_stride, out_ld / 32, M, m0, kw0, lane, acc, kOutScale);
        return;
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t k = kw0 + 32 * u + j;
            if (k >= col_limit) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + 32 * mi + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) out[m * out_ld + k] = kOutScale * acc[mi][u][r];
            }
        }
    }
}

// Split route with specialised waves: 8 waves per block, two per SIMD.  Waves 0..3 are
// consumers (each owns 64 output columns: code DMA, per-lane transpose, MFMAs); waves 4..7 are
// producers that stage A' = d_out * scale as bf16 hi / lo for the next chunk while the
// consumers multiply, so the staging VALU runs beside the other wave's MFMAs.  One block
// barrier per chunk hands the A' stage over.
template <int GT, int NV, int SF>
__global__ __launch_bounds__(512, 1) void gemm_bwd_split_kernel(WView w, const void* __restrict__ d_out, int64_t M,
                                                                float* __restrict__ out, int64_t out_ld,
                                                                int64_t split_stride, int64_t col_limit, int g_fast,
                                                                int chunks_per_split, int splits, int mtiles) {
    constexpr int kAStage = NV * 2 * kPlaneBytes;
    constexpr int kCStage = 4 * kCodeBytes;
    constexpr int kSBuf = 1024;                  // one chunk's scales (one 64-lane 16-byte DMA)
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kAStage + 3 * kCStage + 2 * kSBuf];
    uint8_t* const Aring = smem;
    uint8_t* const Cring = smem + 2 * kAStage;
    uint8_t* const Sbuf = smem + 2 * kAStage + 3 * kCStage;
    lds_u8* const sm_l = (lds_u8*)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool consumer = wave < 4;

    const int64_t bid = blockIdx.x;
    const int z = (int)(bid % splits);
    const int64_t rest = bid / splits;
    const int64_t mb = rest % mtiles;
    const int64_t tile = rest / mtiles;
    const int64_t kb0 = tile * kBK;
    const int64_t m0 = mb * kBM;
    const int64_t N = w.N;
    const int64_t n_chunks = (N + kCN - 1) / kCN;
    const int64_t c_begin = (int64_t)z * chunks_per_split;
    const int64_t c_end = min(c_begin + (int64_t)chunks_per_split, n_chunks);

    if (!consumer) {
        // ---------------- producer: thread p stages row p >> 1, n-octets 4 (p & 1) .. +3 ----------------
        const int p = tid - 256;
        const int arow = p >> 1;
        const int ahalf = p & 1;
        const int64_t am = min(m0 + arow, M - 1);              // rows past M only feed discarded outputs
        constexpr int kXU = (GT == kF32) ? 8 : 4;
        constexpr int kSU = SF ? 4 : 8;
        u4 xreg[kXU];
        u4 sreg[NV][kSU];
        // Scales of chunk c, NV copies x 8 n-octets x 8 rows: one DMA by the first producer wave
        // into a 2-slot LDS buffer, lane l -> (copy v, octet o[, 16-byte half of an fp32 run]) at
        // byte 16 l; lanes past the data repeat it.  A copy for columns past k_pad only feeds
        // idle consumers; its group index stays in the plane.
        const uint8_t* ssrc;
        {
            int v, o, half;
            if constexpr (SF) {
                const int l = lane & (8 * NV - 1);
                v = l >> 3;
                o = l & 7;
                half = 0;
            } else {
                const int l = lane & (16 * NV - 1);
                v = l >> 4;
                o = (l >> 1) & 7;
                half = l & 1;
            }
            const int64_t g = min((kb0 + 128 * v) / w.gs, w.g_pad - 1);
            ssrc = static_cast<const uint8_t*>(w.scales) + ((int64_t)o * w.g_pad + g) * 8 * (SF ? 2 : 4) + 16 * half;
        }
        const int64_t s_chunk_stride = (int64_t)8 * w.g_pad * 8 * (SF ? 2 : 4);
        auto issue_scales = [&](int64_t c) {
            if (wave == 4) dma16(ssrc + s_chunk_stride * c, (lds_u8*)Sbuf + kSBuf * ((c - c_begin) & 1));
        };
        auto load_a = [&](int64_t c) {
            const int64_t n0 = c * kCN + 32 * ahalf;
            if (g_fast && n0 + 32 <= N) {
#pragma unroll
                for (int i = 0; i < kXU; ++i) {
                    if constexpr (GT == kF32) xreg[i] = ldg16(static_cast<const float*>(d_out) + am * N + n0 + 4 * i);
                    else xreg[i] = ldg16(static_cast<const uint16_t*>(d_out) + am * N + n0 + 8 * i);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kXU; ++i) {
                    uint32_t e[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (GT == kF32) {
                            const int64_t n = n0 + 4 * i + q;
                            e[q] = (n < N) ? static_cast<const uint32_t*>(d_out)[am * N + n] : 0u;
                        } else {
                            const int64_t n = n0 + 8 * i + 2 * q;
                            const uint32_t lo = (n < N) ? static_cast<const uint16_t*>(d_out)[am * N + n] : 0u;
                            const uint32_t hi = (n + 1 < N) ? static_cast<const uint16_t*>(d_out)[am * N + n + 1] : 0u;
                            e[q] = lo | (hi << 16);
                        }
                    }
                    xreg[i] = u4{e[0], e[1], e[2], e[3]};
                }
            }
        };
        // the thread's scales (octets 4 ahalf .. +3 of each copy) from the chunk's LDS slot
        auto read_scales = [&](int64_t c) {
            const uint8_t* Sb = Sbuf + kSBuf * ((c - c_begin) & 1);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int o = 8 * v + 4 * ahalf + q;
                    if constexpr (SF) {
                        sreg[v][q] = *reinterpret_cast<const u4*>(Sb + 16 * o);
                    } else {
                        sreg[v][2 * q] = *reinterpret_cast<const u4*>(Sb + 32 * o);
                        sreg[v][2 * q + 1] = *reinterpret_cast<const u4*>(Sb + 32 * o + 16);
                    }
                }
        };
        auto x_at = [&](int i) -> float {
            if constexpr (GT == kF32) return bitcast<float>(xreg[i >> 2][i & 3]);
            else {
                const uint32_t wd = xreg[i >> 3][(i >> 1) & 3];
                const uint16_t b = (i & 1) ? (uint16_t)(wd >> 16) : (uint16_t)(wd & 0xFFFFu);
                if constexpr (GT == kF16) return f16_bits_to_f32(b);
                else return bf16_bits_to_f32(b);
            }
        };
        auto s_at = [&](int v, int i) -> float {
            if constexpr (SF) {
                const uint32_t wd = sreg[v][i >> 3][(i >> 1) & 3];
                return f16_bits_to_f32((i & 1) ? (uint16_t)(wd >> 16) : (uint16_t)(wd & 0xFFFFu));
            } else {
                return bitcast<float>(sreg[v][i >> 2][i & 3]);
            }
        };
        auto store_a = [&](int st, int64_t c) {
            read_scales(c);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                uint8_t* hiP = Aring + st * kAStage + v * 2 * kPlaneBytes;
                uint8_t* loP = hiP + kPlaneBytes;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 8 * q + 2 * e;
                        float a0, a1;
                        if constexpr (SF) {
                            const uint32_t sw = sreg[v][i >> 3][(i >> 1) & 3];
                            a0 = mul_f16_lo(x_at(i), sw);
                            a1 = mul_f16_hi(x_at(i + 1), sw);
                        } else {
                            a0 = x_at(i) * s_at(v, i);
                            a1 = x_at(i + 1) * s_at(v, i + 1);
                        }
                        split_bf16_pair(a0, a1, hw[e], lw[e]);
                    }
                    const int off = arow * kRowBytes + 16 * ((4 * ahalf + q) ^ ((arow >> 1) & 7));
                    *reinterpret_cast<u4*>(hiP + off) = u4{hw[0], hw[1], hw[2], hw[3]};
                    *reinterpret_cast<u4*>(loP + off) = u4{lw[0], lw[1], lw[2], lw[3]};
                }
            }
        };
        // A' of chunk c + 1 is built during chunk c; its loads were issued one chunk earlier, each
        // chunk's scale DMA just before them, so allowing those kXU loads in flight completes it.
        if (c_begin < c_end) {
            issue_scales(c_begin);
            if (c_begin + 1 < c_end) issue_scales(c_begin + 1);
            load_a(c_begin);
        }
        wait_loads_barrier<kXU>();                     // the first two scale slots are in LDS
        if (c_begin < c_end) {
            store_a(0, c_begin);
            if (c_begin + 1 < c_end) load_a(c_begin + 1);
        }
        int sa = 0;
        for (int64_t c = c_begin; c < c_end; ++c) {
            wait_loads_barrier<kXU>();                 // the stores of chunk c and scales of c + 1 are done
            if (c + 1 < c_end) {
                store_a(sa ^ 1, c + 1);
                if (c + 2 < c_end) {
                    issue_scales(c + 2);               // the slot chunk c's scales used
                    load_a(c + 2);
                }
            }
            sa ^= 1;
        }
        return;
    }

    // ---------------- consumer ----------------
    const int j = lane & 31;
    const int h = lane >> 5;
    const int64_t kw0 = kb0 + (int64_t)wave * kWK;
    const bool wave_active = kw0 < w.k_pad;
    const int64_t kwc = wave_active ? kw0 : 0;
    const int64_t kocts = w.k_pad >> 3;
    // Codes in LDS: the wave's 64 n x 64 k codes of a chunk as 8-byte rows (n, P) = code words
    // (n, octet 2P), (n, octet 2P + 1) for octet pair P = 0..3, row (n, P) at byte
    // 8 (64 P + (n ^ 8 (P & 1))).  The xor keeps the rows that one transposing read takes for
    // two neighbouring pairs in different banks.  Word-granular DMA builds the rows: instruction i
    // moves LDS words 64 i .. 64 i + 63, i.e. pair P = i >> 1, n = 32 (i & 1) + (lane >> 1)
    // (xor 8 for odd P), octet 2P + (lane & 1).
    const uint8_t* cpt[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int n = (lane >> 1) ^ (8 * par);
        cpt[par] = w.nib + 32 * ((int64_t)(n >> 3) * kocts + (kwc >> 3) + (lane & 1)) + 4 * (n & 7);
    }
    const int64_t chunk_code_stride = 32 * 8 * kocts;
    auto issue_codes = [&](int64_t c, int st) {
        lds_u8* base = sm_l + 2 * kAStage + st * kCStage + wave * kCodeBytes;
        const int64_t cofs = chunk_code_stride * c;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dma4(cpt[(i >> 1) & 1] + cofs + 128 * kocts * (i & 1) + 64 * (i >> 1), base + 256 * i);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][u][r] = 0.f;

    const int swz = (j >> 1) & 7;
    const int aver = (NV == 2) ? (wave >> 1) : 0;
    // One transposing 4-bit read gives lane (G = lane >> 4, j = lane & 15) the nibbles of row q
    // (the row this read's lane q of group G addresses) at column j, for q = 0..15.  Lane q of
    // group G addresses row n = 16 (q >> 3) + 8 (G >> 1) + (q & 7) of pair 2u + (G & 1) in step
    // pair tp, so the low word holds n = 8 h + 0..7 of step 2 tp and the high word those of step
    // 2 tp + 1 (h = lane >> 5, as the MFMA B operand wants), at k column 32 u + 8 (j' >> 3) +
    // (k offset of nibble j' & 7) with j' = lane & 31.
    const int trG = lane >> 4, trq = lane & 15;
    const int trn = 16 * (trq >> 3) + 8 * (trG >> 1) + (trq & 7);
    const int trofs = 8 * (64 * (trG & 1) + (trn ^ (8 * (trG & 1))));
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i lds_v2i;
    auto read_bt = [&](const uint8_t* Cb, v2i (&bt)[2][2]) {
        const lds_u8* p = (const lds_u8*)Cb + trofs;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int tp = 0; tp < 2; ++tp)
                bt[u][tp] = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_v2i*)(p + 1024 * u + 256 * tp));
    };
    // Eight codes (n = 0..7 in nibbles 0..7) to the bf16 B operand: the 4-bit signed convert of
    // (c ^ 8) gives (c - 8) / 16 exactly (the output is scaled by 16 at the end); byte selects
    // pick the even nibbles from the word and the odd ones from the word rotated by 4 bits.
    auto bconv = [&](uint32_t wd, u4& b) {
        const uint32_t x = wd ^ 0x88888888u;
        const uint32_t x4 = __builtin_amdgcn_alignbit(x, x, 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = __builtin_amdgcn_cvt_off_f32_i4((int)((x >> (8 * e)) & 0xFFu));
            const float hi = __builtin_amdgcn_cvt_off_f32_i4((int)((x4 >> (8 * e)) & 0xFFu));
            b[e] = __builtin_amdgcn_perm(bitcast<uint32_t>(hi), bitcast<uint32_t>(lo), 0x07060302u);
        }
    };
    auto read_a = [&](const uint8_t* Ab, int t, u4 (&a)[4], u4 (&alo)[4]) {
        const int slot = 16 * ((2 * t + h) ^ swz);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int off = (32 * mi + j) * kRowBytes + slot;
            a[mi] = *reinterpret_cast<const u4*>(Ab + off);
            alo[mi] = *reinterpret_cast<const u4*>(Ab + kPlaneBytes + off);
        }
    };
    // A operands of step t + 1 are read, and its B operands converted, between the MFMAs of step t.
    auto compute = [&](int sa, int sc) {
        const uint8_t* Ab = Aring + sa * kAStage + aver * 2 * kPlaneBytes;
        const uint8_t* Cb = Cring + sc * kCStage + wave * kCodeBytes;
        u4 a[2][4], alo[2][4], b[2][2];
        v2i bt[2][2];
        read_bt(Cb, bt);
        read_a(Ab, 0, a[0], alo[0]);
#pragma unroll
        for (int u = 0; u < 2; ++u) bconv((uint32_t)bt[u][0].x, b[0][u]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < 3) read_a(Ab, t + 1, a[nxt], alo[nxt]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int mi = i >> 1, u = i & 1;
                acc[mi][u] = mfma32_bf16(alo[cur][mi], b[cur][u], mfma32_bf16(a[cur][mi], b[cur][u], acc[mi][u]));
                if (t < 3 && (i & 3) == 0) {
                    const int tn = t + 1, un = i >> 2;
                    const v2i wv = bt[un][tn >> 1];
                    bconv((uint32_t)((tn & 1) ? wv.y : wv.x), b[nxt][un]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (c_begin < c_end) {
        issue_codes(c_begin, 0);
        if (c_begin + 1 < c_end) issue_codes(c_begin + 1, 1);
    }
    wait_loads_barrier<63>();                          // the producers' first scale slots
    int sc = 0, sa = 0;
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int sc_next = (sc == 2) ? 0 : sc + 1;
        const int sc_prev = (sc == 0) ? 2 : sc - 1;
        // chunk c's code DMAs are done once only chunk c + 1's eight may be in flight
        if (c + 1 < c_end) wait_loads_barrier<8>();
        else wait_loads_barrier<0>();
        if (c + 2 < c_end) issue_codes(c + 2, sc_prev);
        compute(sa, sc);
        sa ^= 1;
        sc = sc_next;
    }

    if (!wave_active) return;
    if (split_stride) {
        // the fragment layout keeps the lane order; the reduction applies the column permutation
        store_frag_partials(out + (int64_t)z * split_stride, out_ld / 32, M, m0, kw0, lane, acc, 16.0f);
        return;
    }
    float* dst = out;
    // column of this lane in each 32-wide tile: k offset of nibble (j & 7) within octet j >> 3
    const int kcol = (j & ~7) | (((j & 3) << 1) | ((j >> 2) & 1));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t k = kw0 + 32 * u + kcol;
            if (k >= col_limit) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + 32 * mi + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) dst[m * out_ld + k] = 16.0f * acc[mi][u][r];
            }
        }
    }
}

// d_out -> bf16 planes hi and lo ([M][N] each): 8 values per thread, each split to nearest even
// twice (fp32: |err| <= 2^-18 |d_out|; fp16 values split exactly).  vec: 16-byte-aligned source.
template <int GT>
__global__ __launch_bounds__(256) void split_planes_kernel(const void* __restrict__ src, int64_t total, int vec,
                                                           uint32_t* __restrict__ hi, uint32_t* __restrict__ lo) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i0 >= total) return;
    float v[8];
    if (vec && i0 + 8 <= total) {
        if constexpr (GT == kF32) {
            const f4 a = bitcast<f4>(ldg16_stream(static_cast<const float*>(src) + i0 + 0));
            const f4 b = bitcast<f4>(ldg16_stream(static_cast<const float*>(src) + i0 + 4));
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            const u4 a = ldg16_stream(static_cast<const uint16_t*>(src) + i0);
            const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = f16_bits_to_f32((uint16_t)(u[e] & 0xFFFFu));
                v[2 * e + 1] = f16_bits_to_f32((uint16_t)(u[e] >> 16));
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (i0 + e < total) ? load_elem<GT>(src, i0 + e) : 0.f;
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16_pair(v[2 * e], v[2 * e + 1], h[e], l[e]);
    if (i0 + 8 <= total) {
        *reinterpret_cast<u4*>(hi + i0 / 2) = u4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<u4*>(lo + i0 / 2) = u4{l[0], l[1], l[2], l[3]};
    } else {
        uint16_t* h16 = reinterpret_cast<uint16_t*>(hi);
        uint16_t* l16 = reinterpret_cast<uint16_t*>(lo);
        for (int e = 0; e < 8 && i0 + e < total; ++e) {
            h16[i0 + e] = (uint16_t)(h[e >> 1] >> (16 * (e & 1)));
            l16[i0 + e] = (uint16_t)(l[e >> 1] >> (16 * (e & 1)));
        }
    }
}

bool v2_fold(const WView& w, int g_dtype, int fold_ok) { return g_dtype == kF16 && w.scale_f16 && fold_ok; }

// Which 32x32 route serves an input gradient: kModeFold, kModeSplit (gs % 128 == 0), kModeBSplit
// (the exact bf16 B, fp16 scales, gs % 64 == 0 or gs == 32), or -1.
int v2_mode(const WView& w, int g_dtype, int fold_ok) {
    if (v2_fold(w, g_dtype, fold_ok)) return (w.gs % 64 == 0 || w.gs == 32) ? kModeFold : -1;
    if (w.gs % 128 == 0) return kModeSplit;
    if (w.scale_f16 && (w.gs % 64 == 0 || w.gs == 32)) return kModeBSplit;
    return -1;
}

bool v2_supported(const WView& w, int g_dtype, int fold_ok) { return v2_mode(w, g_dtype, fold_ok) >= 0; }

// Elements from the hi plane to the lo plane of the bf16 d_out planes (a 256-byte multiple), and
// the bytes the exact-B route stages at the start of the workspace (none for bf16 d_out).
int64_t bsplit_plane_elems(int64_t M, int64_t N) { return round_up(M * N, 128); }
int64_t bsplit_plane_bytes(int g_dtype, int64_t M, int64_t N) {
    return g_dtype == kBF16 ? 0 : 2 * 2 * bsplit_plane_elems(M, N);
}

template <int NV, int XB>
void launch_fold(dim3 grid, hipStream_t s, const WView& w, const void* d_out, int64_t M, float* out, int64_t ld,
                 int64_t stride, int64_t limit, int g_fast, int per, int splits, int mtiles, int64_t a_plane) {
    hipLaunchKernelGGL((gemm_bwd_fold_kernel<NV, XB>), grid, dim3(256), 0, s, w, d_out, M, out, ld, stride, limit,
                       g_fast, per, splits, mtiles, a_plane);
}

template <int GT, int NV>
void launch_split(int sf, dim3 grid, hipStream_t s, const WView& w, const void* d_out, int64_t M, float* out,
                  int64_t ld, int64_t stride, int64_t limit, int g_fast, int per, int splits, int mtiles) {
    if (sf)
        hipLaunchKernelGGL((gemm_bwd_split_kernel<GT, NV, 1>), grid, dim3(512), 0, s, w, d_out, M, out, ld, stride,
                           limit, g_fast, per, splits, mtiles);
    else
        hipLaunchKernelGGL((gemm_bwd_split_kernel<GT, NV, 0>), grid, dim3(512), 0, s, w, d_out, M, out, ld, stride,
                           limit, g_fast, per, splits, mtiles);
}

}  // namespace

bool gemm_bwd_supported(const WView& w, int g_dtype, int fold_ok) {
    return v2_supported(w, g_dtype, fold_ok) || gemm_bwd_v1_supported(w, g_dtype, fold_ok);
}

BwdPlan plan_gemm_bwd(const WView& w, int g_dtype, int fold_ok, int64_t M, int force_splits) {
    if (!v2_supported(w, g_dtype, fold_ok)) {
        BwdPlan p = plan_gemm_bwd_v1(w, g_dtype, fold_ok, M);
        p.v1 = 1;
        return p;
    }
    BwdPlan p{};
    p.mode = v2_mode(w, g_dtype, fold_ok);
    const int64_t blocks = ((w.k_pad + kBK - 1) / kBK) * ((M + kBM - 1) / kBM);
    const int64_t n_chunks = (w.N + kCN - 1) / kCN;
    p.splits = pick_gemm_splits(blocks, n_chunks, M, w.k_pad, 256, 2.0, nullptr, force_splits);
    p.ws_bytes = p.splits > 1 ? (int64_t)p.splits * frag_plane_floats(M, w.k_pad) * 4 : 0;
    if (p.mode == kModeBSplit) p.ws_bytes += bsplit_plane_bytes(g_dtype, M, w.N);
    p.v1 = 0;
    return p;
}

hipError_t launch_gemm_bwd(const WView& w, const void* d_out, int g_dtype, int64_t M, float* d_x,
                           const BwdPlan& plan, float* ws, hipStream_t s, const LowRankEpi* lr) {
    if (plan.v1) return launch_gemm_bwd_v1(w, d_out, g_dtype, M, d_x, plan, ws, s);
    const int64_t n_chunks = (w.N + kCN - 1) / kCN;
    const int per = (int)((n_chunks + plan.splits - 1) / plan.splits);
    const int64_t mtiles = (M + kBM - 1) / kBM;
    const int64_t blocks = ((w.k_pad + kBK - 1) / kBK) * mtiles * plan.splits;
    if (blocks > (int64_t(1) << 24)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const int esize = g_dtype == kF32 ? 4 : 2;
    const int g_fast = ((reinterpret_cast<uintptr_t>(d_out) & 15u) == 0) && ((w.N * esize) % 16 == 0);
    float* out = plan.splits == 1 ? d_x : ws;
    const int64_t ld = plan.splits == 1 ? w.K : w.k_pad;
    const int64_t stride = plan.splits == 1 ? 0 : frag_plane_floats(M, w.k_pad);
    const int64_t limit = plan.splits == 1 ? w.K : w.k_pad;
    const int sp = plan.splits, mt = (int)mtiles;
    if (plan.mode == kModeFold) {
        if (w.gs == 32) launch_fold<2, 0>(grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt, 0);
        else launch_fold<1, 0>(grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt, 0);
    } else if (plan.mode == kModeBSplit) {
        // the workspace starts with the bf16 planes of d_out (none for bf16 d_out), then the partials
        const int64_t pb = bsplit_plane_bytes(g_dtype, M, w.N);
        const void* A = d_out;
        int fast = g_fast;
        const int64_t ap = bsplit_plane_elems(M, w.N);
        if (pb > 0) {
            uint32_t* hi = reinterpret_cast<uint32_t*>(ws);
            uint32_t* lo = hi + ap / 2;
            const int64_t total = M * w.N;
            const int64_t nb = (total + 2047) / 2048;
            if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
            const int vec = (reinterpret_cast<uintptr_t>(d_out) & 15u) == 0;
            if (g_dtype == kF32)
                hipLaunchKernelGGL((split_planes_kernel<kF32>), dim3((unsigned)nb), dim3(256), 0, s, d_out, total, vec,
                                   hi, lo);
            else
                hipLaunchKernelGGL((split_planes_kernel<kF16>), dim3((unsigned)nb), dim3(256), 0, s, d_out, total, vec,
                                   hi, lo);
            A = hi;
            fast = (w.N * 2) % 16 == 0;
            if (plan.splits > 1) out = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + pb);
        }
        if (pb > 0) {
            if (w.gs == 32) launch_fold<2, 2>(grid, s, w, A, M, out, ld, stride, limit, fast, per, sp, mt, ap);
            else launch_fold<1, 2>(grid, s, w, A, M, out, ld, stride, limit, fast, per, sp, mt, ap);
        } else {
            if (w.gs == 32) launch_fold<2, 1>(grid, s, w, A, M, out, ld, stride, limit, fast, per, sp, mt, ap);
            else launch_fold<1, 1>(grid, s, w, A, M, out, ld, stride, limit, fast, per, sp, mt, ap);
        }
        ws = (plan.splits > 1) ? out : ws;
    } else {
        const bool one = w.gs % 256 == 0;
        const int sf = w.scale_f16;
        switch (g_dtype) {
            case kF32:
                if (one) launch_split<kF32, 1>(sf, grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt);
                else launch_split<kF32, 2>(sf, grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt);
                break;
            case kF16:
                if (one) launch_split<kF16, 1>(sf, grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt);
                else launch_split<kF16, 2>(sf, grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt);
                break;
            default:
                if (one) launch_split<kBF16, 1>(sf, grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt);
                else launch_split<kBF16, 2>(sf, grid, s, w, d_out, M, out, ld, stride, limit, g_fast, per, sp, mt);
                break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const float* ys[1] = {d_x};
    const int64_t yld[1] = {w.K}, off[1] = {0}, cols[1] = {w.K};
    return launch_reduce_frags(ws, plan.splits, M, w.k_pad, ys, yld, off, cols, 1, plan.mode == kModeSplit ? 1 : 0, s,
                               lr);
}

}  // namespace q4gsw
